// Streaming decode kernel for few activation rows (1-2 for W4A16, up to 8 for
// FP8 and BF16), x broadcast by DPP.
//
// Same work split as the LDS-staged streaming kernel (one workgroup per
// 16-row block over all of K, W wavefronts on contiguous shares of K, fixed
// order reductions), but x never goes through LDS: each x register (the
// per-tile arithmetic is in wqd_bcast_tile.h) is loaded straight from L2 as
// one coalesced read per wavefront and handed to the lanes of a row by a DPP
// row broadcast.
//
// Why: the weights are read once per step, so the bandwidth is set by bytes
// in flight per compute unit.  Without the staged x (registers for the
// staging, LDS reads per tile) a wavefront needs far fewer registers, more
// wavefronts fit per SIMD and every one keeps a whole group of tiles in
// flight; small matrices can also use up to 16 wavefronts per workgroup.
#include "wqd_bcast_tile.h"
#include "wqd_device.h"
#include "wqd_internal.h"
#include "wqd_plan.h"

namespace wqd {

struct BcastArgs {
  const uint16_t* x;
  uint16_t* y;
  const uint4* w;
  const void* scales;
  const uint16_t* zeros;
  int64_t N, K, KT, G4;
  int per_wave;  // tiles per wavefront share of K (a multiple of 4)
  int swiglu;    // packed gate/up pairs: store silu(gate) * up (store_out)
};

// Loads for tiles t0 .. t0 + 3 of the share.  Weights go through a buffer
// resource that spans exactly the share: a tile past its end is out of range
// and reads as zero without touching memory, so every load is issued
// unconditionally (the in-order load counter then lets the arithmetic wait
// for exactly the group it needs).  x, scale and zero reads are clamped to
// the last tile; x dwords past K (a ragged last FP8 / BF16 tile) read an
// in-bounds dword and are zeroed.  Tiles past the end are never multiplied.
template <int FMT, int MR>
__device__ __forceinline__ void bload(BGroup<FMT, MR>& g, const BcastArgs& a, __amdgpu_buffer_rsrc_t wres,
                                      const uint2* sbase, const uint16_t* zbase, int64_t kt_begin, int t0,
                                      int last, int lane, int kb, int j) {
  using C = BcC<FMT>;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // cache policy 2: non-temporal (weights are read once per step)
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(wres, (t0 + i) * kTileBytes + lane * 16, 0, 2);
    g.w[i] = make_uint4(v.x, v.y, v.z, v.w);
  }
#pragma unroll
  for (int r = 0; r < C::XR; ++r) {
    // lane (kb, j): x dwords XW (j % LPS) .. + XW - 1 of slice kb of tile r TPX + j / LPS
    const int tt = min(t0 + r * C::TPX + j / C::LPS, last);
    const int64_t k = (kt_begin + tt) * C::TK + kb * C::SLK + 2 * C::XW * (j % C::LPS);
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      if (FMT == kFmtW4) {
        g.x[m][r] = *reinterpret_cast<const XReg<FMT>*>(a.x + int64_t(m) * a.K + k);
      } else {
        // K is a multiple of 8, so a register's 2 XW elements are all below K or all past it
        const int64_t kc = k < a.K ? k : a.K - 2 * C::XW;
        const XReg<FMT> v = *reinterpret_cast<const XReg<FMT>*>(a.x + int64_t(m) * a.K + kc);
        g.x[m][r] = k < a.K ? v : XReg<FMT>(0);
      }
    }
  }
  if (FMT == kFmtW4) {
    const int q = min(t0, last) / kScaleQuad;
    g.s = sbase[q * kTileRows];
    g.z = zbase[q * kTileRows];
  }
}

// Multiply group `g` (tiles t .. t + 3; fewer at the end of the share), then
// (unless LAST) refill it with the group two ahead, so two groups stay in
// flight.  Refills past the share read nothing from memory (the weight
// buffer resource ends with the share; x, scale and zero reads are clamped),
// which keeps every load unconditional and the compiler's waits exact.
// Returns whether tiles remain.
template <int FMT, int MR, int XC, int CB, bool LAST>
__device__ __forceinline__ bool bstep(BGroup<FMT, MR>& g, int& t, int total, const BcastArgs& a,
                                      __amdgpu_buffer_rsrc_t wres, const uint2* sbase, const uint16_t* zbase,
                                      int64_t kt_begin, int lane, int kb, int n, const float (&X)[MR][XC],
                                      float (&acc)[MR]) {
  const int left = total - t;
  if (left >= 4) {
    btile<FMT, MR, XC, 0, CB + 0>(g, X, acc);
    btile<FMT, MR, XC, 1, CB + 1>(g, X, acc);
    btile<FMT, MR, XC, 2, CB + 2>(g, X, acc);
    btile<FMT, MR, XC, 3, CB + 3>(g, X, acc);
    if (!LAST) bload<FMT, MR>(g, a, wres, sbase, zbase, kt_begin, t + 8, total - 1, lane, kb, n);
    // issue the refill here: left to itself the scheduler sinks loads to just
    // before their use, which would leave one group in flight instead of two
    __builtin_amdgcn_sched_barrier(0);
    t += 4;
    return t < total;
  }
  btile<FMT, MR, XC, 0, CB + 0>(g, X, acc);
  if (left > 1) btile<FMT, MR, XC, 1, CB + 1>(g, X, acc);
  if (left > 2) btile<FMT, MR, XC, 2, CB + 2>(g, X, acc);
  return false;
}

// Steps S .. NG - 1 as straight-line code with early exits (no loop, so no
// loop-carried registers with loads in flight): groups alternate between the
// two buffers, and the last two steps have nothing left to refill.  The
// second register of W4A16 x sums is formed just before its first tile, from
// loads issued after the first one's chain.
template <int FMT, int MR, int XC, int NG, int S>
__device__ __forceinline__ void bsteps(BGroup<FMT, MR>& g0, BGroup<FMT, MR>& g1, int& t, int total,
                                       const BcastArgs& a, __amdgpu_buffer_rsrc_t wres, const uint2* sbase,
                                       const uint16_t* zbase, int64_t kt_begin, int lane, int kb, int n,
                                       float (&X)[MR][XC], const uint4 (&xs)[MR][4], float (&acc)[MR]) {
  if constexpr (S < NG) {
    if constexpr (FMT == kFmtW4 && XC == 2 && S == 4) xsums<FMT, MR, XC>(X, xs, 1);
    BGroup<FMT, MR>& g = S % 2 == 0 ? g0 : g1;
    if (bstep<FMT, MR, XC, 4 * S, (S >= NG - 2)>(g, t, total, a, wres, sbase, zbase, kt_begin, lane, kb, n, X, acc))
      bsteps<FMT, MR, XC, NG, S + 1>(g0, g1, t, total, a, wres, sbase, zbase, kt_begin, lane, kb, n, X, xs, acc);
  }
}

// NG: groups of 4 tiles per wavefront share (4 or 8).  XC: registers of
// W4A16 x sums, 16 tiles each.
template <int FMT, int MR, int W, int NG>
__global__ __launch_bounds__(64 * W) void gemv_bcast_kernel(BcastArgs a) {
  using C = BcC<FMT>;
  constexpr int XC = FMT == kFmtW4 ? NG / 4 : 1;
  __shared__ float s_red[W][MR][kTileRows];

  const int lane = threadIdx.x & 63, kb = lane >> 4, n = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: scalar control flow
  const int64_t nb = blockIdx.x;
  const int64_t kt_begin = int64_t(wave) * a.per_wave;
  const int64_t rem = a.KT - kt_begin;
  const int total = rem <= 0 ? 0 : (rem < a.per_wave ? int(rem) : a.per_wave);

  float acc[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) acc[m] = 0.f;

  if (total > 0) {
    const int last = total - 1;
    const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint4*>(a.w + (nb * a.KT + kt_begin) * (kTileBytes / 16)), 0, total * kTileBytes, 0x00020000);
    const int64_t q0 = FMT == kFmtW4 ? (nb * a.G4 + kt_begin / kScaleQuad) * kTileRows + n : 0;
    const uint2* sbase = reinterpret_cast<const uint2*>(a.scales) + q0;
    const uint16_t* zbase = a.zeros + q0;

    // W4A16 x sums: lane (kb, n) of register c sums slice kb of tile 16 c + n
    // of the share.  Its 32 x values are loaded as 4 x 16 bytes per row.
    uint4 xs[MR][4];
    auto load_xs = [&](int c) {
      const int64_t k0 = (kt_begin + min(16 * c + n, last)) * C::TK + kb * C::SLK;
#pragma unroll
      for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int u = 0; u < 4; ++u) xs[m][u] = *reinterpret_cast<const uint4*>(a.x + int64_t(m) * a.K + k0 + 8 * u);
    };
    if constexpr (FMT == kFmtW4) load_xs(0);
    BGroup<FMT, MR> g0, g1;
    bload<FMT, MR>(g0, a, wres, sbase, zbase, kt_begin, 0, last, lane, kb, n);
    bload<FMT, MR>(g1, a, wres, sbase, zbase, kt_begin, 4, last, lane, kb, n);
    // keep every prologue load ahead of the first wait (the x sums wait for
    // their own loads; the scheduler would otherwise start them earlier)
    __builtin_amdgcn_sched_barrier(0);
    float X[MR][XC];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
      for (int c = 0; c < XC; ++c) X[m][c] = 0.f;
    if constexpr (FMT == kFmtW4) {
      xsums<FMT, MR, XC>(X, xs, 0);
      if constexpr (XC == 2) load_xs(1);
    }
    // Groups 0 and 1 are in flight; each step multiplies one and refills it
    // with the group two ahead.
    int t = 0;
    bsteps<FMT, MR, XC, NG, 0>(g0, g1, t, total, a, wres, sbase, zbase, kt_begin, lane, kb, n, X, xs, acc);
  }

  // the 4 slices of a row (lanes n, n+16, n+32, n+48), then the W wavefronts
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    float v = acc[m];
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    if (kb == 0) s_red[wave][m][n] = v;
  }
  __syncthreads();
  if (threadIdx.x < MR * kTileRows) {
    const int m = threadIdx.x / kTileRows, r = threadIdx.x % kTileRows;
    float v = s_red[0][m][r];
#pragma unroll
    for (int w = 1; w < W; ++w) v += s_red[w][m][r];
    const int64_t row = nb * kTileRows + r;
    const bool live = row < a.N;
    if (FMT == kFmtFP8 && live) v *= reinterpret_cast<const float*>(a.scales)[row];
    store_out<8>(a.y, a.N, a.swiglu, m, row, v, live);  // thread ^ 8 holds row ^ 8
  }
}

template <int FMT, int MR, int NG>
static hipError_t launch_bc_w(const BcastArgs& a, int waves, unsigned grid, hipStream_t st) {
  switch (waves) {
    case 4: hipLaunchKernelGGL((gemv_bcast_kernel<FMT, MR, 4, NG>), dim3(grid), dim3(256), 0, st, a); break;
    case 8: hipLaunchKernelGGL((gemv_bcast_kernel<FMT, MR, 8, NG>), dim3(grid), dim3(512), 0, st, a); break;
    case 16: hipLaunchKernelGGL((gemv_bcast_kernel<FMT, MR, 16, NG>), dim3(grid), dim3(1024), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Rows per launch: 1..2 for every format (four or eight groups per share);
// FP8 and BF16 also 3..8 (four groups: the x registers grow with the rows).
template <int FMT>
static hipError_t launch_bc_fmt(const BcastArgs& a, int mr, int waves, int ng, unsigned grid, hipStream_t st) {
  if (ng == 8) {
    if (mr == 1) return launch_bc_w<FMT, 1, 8>(a, waves, grid, st);
    if (mr == 2) return launch_bc_w<FMT, 2, 8>(a, waves, grid, st);
    return hipErrorInvalidValue;
  }
  if (ng != 4) return hipErrorInvalidValue;
  switch (mr) {
    case 1: return launch_bc_w<FMT, 1, 4>(a, waves, grid, st);
    case 2: return launch_bc_w<FMT, 2, 4>(a, waves, grid, st);
    default: break;
  }
  if constexpr (FMT != kFmtW4) {
    switch (mr) {
      case 3: return launch_bc_w<FMT, 3, 4>(a, waves, grid, st);
      case 4: return launch_bc_w<FMT, 4, 4>(a, waves, grid, st);
      case 5: return launch_bc_w<FMT, 5, 4>(a, waves, grid, st);
      case 6: return launch_bc_w<FMT, 6, 4>(a, waves, grid, st);
      case 7: return launch_bc_w<FMT, 7, 4>(a, waves, grid, st);
      case 8: return launch_bc_w<FMT, 8, 4>(a, waves, grid, st);
      default: break;
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemv_bcast(int fmt, const BcastPlan& p, const void* x, int64_t M, int64_t N, int64_t K,
                             const void* wp, const void* scales, const void* zeros, void* y, bool swiglu,
                             hipStream_t st) {
  if (M < 1 || M > (fmt == kFmtW4 ? kBcastMaxMW4 : kBcastMaxM)) return hipErrorInvalidValue;
  BcastArgs a;
  a.x = reinterpret_cast<const uint16_t*>(x);
  a.y = reinterpret_cast<uint16_t*>(y);
  a.w = reinterpret_cast<const uint4*>(wp);
  a.scales = scales;
  a.zeros = reinterpret_cast<const uint16_t*>(zeros);
  a.N = N;
  a.K = K;
  a.KT = p.KT;
  a.G4 = fmt == kFmtW4 ? ceil_div(K / kGroup, kScaleQuad) : 0;
  a.per_wave = p.per_wave;
  a.swiglu = swiglu;
  const unsigned grid = unsigned(p.NB);
  const int mr = int(M);
  if (fmt == kFmtBF16) return launch_bc_fmt<kFmtBF16>(a, mr, p.waves, p.groups, grid, st);
  if (fmt == kFmtFP8) return launch_bc_fmt<kFmtFP8>(a, mr, p.waves, p.groups, grid, st);
  return launch_bc_fmt<kFmtW4>(a, mr, p.waves, p.groups, grid, st);
}

}  // namespace wqd
