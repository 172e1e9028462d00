// Streaming decode kernel for M <= 8 activation rows: y = x . dequant(W)^T.
//
// Decode moves every weight byte once per step at about one FLOP per byte, so
// this kernel is bound by HBM ("Making each token cheaper", section "Why
// decode is usually bandwidth bound").  Design for gfx950:
//   * one workgroup owns one 16-row block over ALL of K, so no partial sums
//     ever leave the workgroup: no split-K workspace and no device-scope
//     fences (on a multi-XCD part those write back and invalidate L2);
//   * its W wavefronts take contiguous shares of K.  Lane l = 16 kb + n of a
//     wavefront owns slice kb of row n of every tile in its share: one
//     16-byte load per lane, 1 KiB contiguous per wavefront;
//   * each wavefront stages its own x range in a private LDS region (chunked
//     when it does not fit) and reads it back as 16-byte broadcast reads; no
//     workgroup barrier is needed until the final reduction.  The x loads are
//     issued ahead of the first two weight groups, so the start-up costs one
//     memory round trip, not two;
//   * weight tiles stream in groups of GT (4 or 8) with the next group in
//     flight during the arithmetic: the bytes in flight per compute unit are
//     what sets the bandwidth (Little's law).  Loads are branch-free (clamped
//     at the end of a share) so the in-order load counter lets the arithmetic
//     wait for exactly the group it needs; they are non-temporal (every byte
//     is read once per step);
//   * dequantisation in registers: W4A16 nibble pairs become bf16 (128 + q)
//     with one AND-OR, FP8 codes become bf16 with the hardware conversion;
//     v_dot2_f32_bf16 forms exact bf16 x bf16 products summed in float32.
//     A W4A16 slice contributes s * (sum x (128 + q) - (128 + z) * sum x),
//     where sum x comes from the same dot2 chain against (1, 1), so q == z
//     == 0 cancels exactly;
//   * the 4 lanes of a row and the W wavefronts are reduced in a fixed order
//     (deterministic, no atomics).
#include "wqd_device.h"
#include "wqd_internal.h"
#include "wqd_plan.h"

namespace wqd {

struct GemvArgs {
  const uint16_t* x;
  uint16_t* y;
  const uint4* w;
  const void* scales;
  const uint16_t* zeros;
  int64_t N, K, NB, KT, G4;
  int swiglu;  // packed gate/up pairs: store silu(gate) * up (store_out)
};

template <int FMT>
struct FmtC {
  static constexpr int TK = FMT == kFmtBF16 ? 32 : FMT == kFmtFP8 ? 64 : 128;  // K per tile
  static constexpr int SLK = TK / 4;                                             // K per slice
  static constexpr int SLU = SLK / 8;                                            // x uint4 per slice
  static constexpr int SLS = SLU + (FMT == kFmtW4 ? 1 : 0);  // padded LDS stride: spreads the 4 slices over banks
};

// x staged per wavefront and chunk: about 4 KiB (2048 k per activation row
// at M = 1).  Tiles per group: 8 for BF16 when the chunk holds 8 tiles (its
// arithmetic per byte is light, so more bytes in flight pay), else 4 (a
// W4A16 scale quad; W4A16 and FP8 measured faster with the smaller register
// footprint).  Tiles per chunk: a whole number of groups.  SPL: x slices each
// lane stages per chunk.
template <int FMT, int MR>
struct Plan {
  static constexpr int raw = 2048 / (MR * FmtC<FMT>::TK);
  static constexpr int GT = (FMT == kFmtBF16 && raw >= 8) ? 8 : 4;
  static constexpr int CT = raw / GT * GT < GT ? GT : raw / GT * GT;
  static constexpr int SPL = (MR * CT * 4 + 63) / 64;
};

template <int FMT, int GT>
struct Group {
  uint4 w[GT];
  uint2 s[GT / 4];     // W4A16: fp16 scales, 4 tiles per quad
  uint32_t z[GT / 4];  // W4A16: 4 zero nibbles per quad
};

// Load one group of GT tiles of this wavefront's rows: lane l reads its 16
// bytes of tile t at wbase + t * 64 (uint4 units), t = t0 .. t0 + GT - 1
// clamped to the last tile of the share, so every load is issued
// unconditionally (no branch: the in-order load counter stays exact) and
// stays in bounds; clamped tiles are never multiplied.  Non-temporal: weights
// are read once per decode step.
template <int FMT, int GT>
__device__ __forceinline__ void load_group(Group<FMT, GT>& g, const uint4* wbase, const uint2* sbase,
                                           const uint16_t* zbase, int t0, int last) {
#pragma unroll
  for (int i = 0; i < GT; ++i) g.w[i] = load_nt(wbase + min(t0 + i, last) * (kTileBytes / 16));
  if (FMT == kFmtW4) {
#pragma unroll
    for (int j = 0; j < GT / 4; ++j) {
      const int q = min(t0 + 4 * j, last) / kScaleQuad;
      g.s[j] = sbase[q * kTileRows];
      g.z[j] = zbase[q * kTileRows];
    }
  }
}

// acc[m] += the products of tile i of a group for every activation row.  One
// dot2 chain per tile and row: dependent VALU instructions issue back to back
// on CDNA and other wavefronts fill the LDS wait.  sl = slice index of this
// lane's part of the tile inside the staged x chunk.
template <int FMT, int MR, int CT, int GT>
__device__ __forceinline__ void tile_dot(const Group<FMT, GT>& g, int i, int sl, const uint4* __restrict__ xs,
                                         const float* __restrict__ xsum, float (&acc)[MR]) {
  using C = FmtC<FMT>;
  const uint32_t wd[4] = {g.w[i].x, g.w[i].y, g.w[i].z, g.w[i].w};
  if (FMT == kFmtW4) {
    const uint32_t mask = vgpr_const(0x000F000Fu), magic = vgpr_const(0x43004300u);
    float P[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) P[m] = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bf16x2_t b0 = as_bf16x2(and_or_v(wd[q], mask, magic));  // (128 + q) pairs
      const bf16x2_t b1 = as_bf16x2(and_or_v(wd[q] >> 4, mask, magic));
      const bf16x2_t b2 = as_bf16x2(and_or_v(wd[q] >> 8, mask, magic));
      const bf16x2_t b3 = as_bf16x2(and_or_v(wd[q] >> 12, mask, magic));
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        const uint4 xv = xs[(m * CT * 4 + sl) * C::SLS + q];
        P[m] = dot2_bf16(b0, as_bf16x2(xv.x), P[m]);
        P[m] = dot2_bf16(b1, as_bf16x2(xv.y), P[m]);
        P[m] = dot2_bf16(b2, as_bf16x2(xv.z), P[m]);
        P[m] = dot2_bf16(b3, as_bf16x2(xv.w), P[m]);
      }
    }
    const uint2 sq = g.s[i / 4];
    const uint32_t sbits = ((i & 3) < 2 ? sq.x : sq.y) >> (16 * (i & 1));
    const float s = __half2float(__ushort_as_half(uint16_t(sbits & 0xFFFFu)));
    const float zc = 128.0f + float((g.z[i / 4] >> (4 * (i & 3))) & 0xFu);
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      const float D = fmaf(-zc, xsum[m * CT * 4 + sl], P[m]);
      acc[m] = fmaf(s, D, acc[m]);
    }
  } else if (FMT == kFmtFP8) {
    bf16x2_t b[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      b[2 * q] = e4m3x2_to_bf16x2<false>(wd[q]);
      b[2 * q + 1] = e4m3x2_to_bf16x2<true>(wd[q]);
    }
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      const uint4 x0 = xs[(m * CT * 4 + sl) * C::SLS], x1 = xs[(m * CT * 4 + sl) * C::SLS + 1];
      float a0 = acc[m];
      a0 = dot2_bf16(b[0], as_bf16x2(x0.x), a0);
      a0 = dot2_bf16(b[1], as_bf16x2(x0.y), a0);
      a0 = dot2_bf16(b[2], as_bf16x2(x0.z), a0);
      a0 = dot2_bf16(b[3], as_bf16x2(x0.w), a0);
      a0 = dot2_bf16(b[4], as_bf16x2(x1.x), a0);
      a0 = dot2_bf16(b[5], as_bf16x2(x1.y), a0);
      a0 = dot2_bf16(b[6], as_bf16x2(x1.z), a0);
      a0 = dot2_bf16(b[7], as_bf16x2(x1.w), a0);
      acc[m] = a0;
    }
  } else {
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      const uint4 xv = xs[(m * CT * 4 + sl) * C::SLS];
      float a0 = acc[m];
      a0 = dot2_bf16(as_bf16x2(wd[0]), as_bf16x2(xv.x), a0);
      a0 = dot2_bf16(as_bf16x2(wd[1]), as_bf16x2(xv.y), a0);
      a0 = dot2_bf16(as_bf16x2(wd[2]), as_bf16x2(xv.z), a0);
      a0 = dot2_bf16(as_bf16x2(wd[3]), as_bf16x2(xv.w), a0);
      acc[m] = a0;
    }
  }
}

// Staging of x for tiles [kt0, kt0 + nt) of this wavefront's share, in two
// halves: load_x issues the global loads into registers, commit_x writes
// them to the wavefront's LDS region (and, for W4A16, the per-slice x sums).
// Weight loads issued between the two halves stay in flight: loads complete
// in issue order, so commit_x waits for x alone.  The region is private to
// the wavefront and LDS operations of one wavefront complete in order, so
// only compiler ordering is needed around it.
template <int FMT, int MR, int CT>
struct XStage {
  uint4 v[Plan<FMT, MR>::SPL][FmtC<FMT>::SLU];
};

template <int FMT, int MR, int CT>
__device__ __forceinline__ void load_x(XStage<FMT, MR, CT>& xr, const GemvArgs& a, int64_t kt0, int nt, int lane) {
  using C = FmtC<FMT>;
  const int per_m = nt * 4;  // slices per activation row in this chunk
#pragma unroll
  for (int j = 0; j < Plan<FMT, MR>::SPL; ++j) {
    const int i = lane + 64 * j;
    const int m = i / per_m, sl = i - m * per_m;
    const int64_t k = (kt0 + sl / 4) * C::TK + (sl & 3) * C::SLK;
#pragma unroll
    for (int u = 0; u < C::SLU; ++u) {
      xr.v[j][u] = make_uint4(0, 0, 0, 0);
      if (i < MR * per_m && k + 8 * u < a.K)
        xr.v[j][u] = *reinterpret_cast<const uint4*>(a.x + int64_t(m) * a.K + k + 8 * u);
    }
  }
}

template <int FMT, int MR, int CT>
__device__ __forceinline__ void commit_x(const XStage<FMT, MR, CT>& xr, int nt, int lane, uint4* __restrict__ xs,
                                         float* __restrict__ xsum) {
  using C = FmtC<FMT>;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  const int per_m = nt * 4;
#pragma unroll
  for (int j = 0; j < Plan<FMT, MR>::SPL; ++j) {
    const int i = lane + 64 * j;
    if (i < MR * per_m) {
      const int m = i / per_m, sl = i - m * per_m;
      uint4* dst = xs + (m * CT * 4 + sl) * C::SLS;
#pragma unroll
      for (int u = 0; u < C::SLU; ++u) dst[u] = xr.v[j][u];
      if (FMT == kFmtW4) {
        const bf16x2_t ones = as_bf16x2(0x3F803F80u);
        float X = 0.f;
#pragma unroll
        for (int u = 0; u < C::SLU; ++u) {
          X = dot2_bf16(ones, as_bf16x2(xr.v[j][u].x), X);
          X = dot2_bf16(ones, as_bf16x2(xr.v[j][u].y), X);
          X = dot2_bf16(ones, as_bf16x2(xr.v[j][u].z), X);
          X = dot2_bf16(ones, as_bf16x2(xr.v[j][u].w), X);
        }
        xsum[m * CT * 4 + sl] = X;
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

template <int FMT, int MR, int W>
__global__ __launch_bounds__(64 * W) void gemv_kernel(GemvArgs a) {
  using C = FmtC<FMT>;
  constexpr int GT = Plan<FMT, MR>::GT;
  constexpr int CT = Plan<FMT, MR>::CT;
  __shared__ uint4 s_x[W][MR * CT * 4 * C::SLS];
  __shared__ float s_xsum[W][FMT == kFmtW4 ? MR * CT * 4 : 1];
  __shared__ float s_red[W][MR][kTileRows];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, kb = lane >> 4, n = lane & 15;
  const int64_t nb = blockIdx.x;
  // contiguous share of K tiles for this wavefront, in whole groups
  const int64_t per_wave = (a.KT + int64_t(W) * GT - 1) / (int64_t(W) * GT) * GT;
  const int64_t kt_begin = wave * per_wave;
  const int64_t kt_end = min(a.KT, kt_begin + per_wave);
  uint4* xs = s_x[wave];
  float* xsum = s_xsum[wave];

  float acc[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) acc[m] = 0.f;

  const int total = int(max<int64_t>(0, kt_end - kt_begin));
  if (total > 0) {
    // weight, scale and zero streams of this lane
    const uint4* wbase = a.w + (nb * a.KT + kt_begin) * (kTileBytes / 16) + lane;
    const int64_t q0 = FMT == kFmtW4 ? (nb * a.G4 + kt_begin / kScaleQuad) * kTileRows + n : 0;
    const uint2* sbase = reinterpret_cast<const uint2*>(a.scales) + q0;
    const uint16_t* zbase = a.zeros + q0;
    int issued = 0;  // first tile of the next group to load
    auto issue = [&](Group<FMT, GT>& g) {
      load_group<FMT, GT>(g, wbase, sbase, zbase, issued, total - 1);
      issued += GT;
    };
    // One group in flight ahead of the one being multiplied.  The two
    // buffers alternate by unrolling the loop two ways (no register copies):
    // step(cur, dst) refills dst, the buffer consumed one step earlier.  At a
    // chunk boundary the x loads go out before dst's weight loads, so the
    // first step has x, group 0 and group 1 in flight together.
    Group<FMT, GT> g0, g1;
    XStage<FMT, MR, CT> xr;
    int t = 0;  // tiles multiplied so far
    auto step = [&](Group<FMT, GT>& cur, Group<FMT, GT>& dst) -> bool {
      if (t >= total) return false;
      const bool stage = t % CT == 0;
      const int nt = min(CT, total - t);
      if (stage && t > 0) load_x<FMT, MR, CT>(xr, a, kt_begin + t, nt, lane);
      issue(dst);
      if (stage) commit_x<FMT, MR, CT>(xr, nt, lane, xs, xsum);
      const int left = total - t;
      const int tl0 = t % CT;
      if (left >= GT) {
#pragma unroll
        for (int i = 0; i < GT; ++i) tile_dot<FMT, MR, CT, GT>(cur, i, (tl0 + i) * 4 + kb, xs, xsum, acc);
      } else {
#pragma unroll
        for (int i = 0; i < GT; ++i)
          if (i < left) tile_dot<FMT, MR, CT, GT>(cur, i, (tl0 + i) * 4 + kb, xs, xsum, acc);
      }
      t += GT;
      return true;
    };
    load_x<FMT, MR, CT>(xr, a, kt_begin, min(CT, total), lane);
    issue(g0);
    while (step(g0, g1) && step(g1, g0)) {
    }
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

template <int FMT, int W, int MR>
static hipError_t launch_fmt(const GemvArgs& a, unsigned grid, hipStream_t st) {
  hipLaunchKernelGGL((gemv_kernel<FMT, MR, W>), dim3(grid), dim3(64 * W), 0, st, a);
  return hipGetLastError();
}

template <int FMT>
static hipError_t launch_waves(const GemvArgs& a, int mr, int waves, unsigned grid, hipStream_t st) {
  // 8 wavefronts only for up to 2 activation rows (their LDS share fits)
  if (waves == 8 && mr == 1) return launch_fmt<FMT, 8, 1>(a, grid, st);
  if (waves == 8 && mr == 2) return launch_fmt<FMT, 8, 2>(a, grid, st);
  switch (mr) {
    case 1: return launch_fmt<FMT, 4, 1>(a, grid, st);
    case 2: return launch_fmt<FMT, 4, 2>(a, grid, st);
    case 3: return launch_fmt<FMT, 4, 3>(a, grid, st);
    case 4: return launch_fmt<FMT, 4, 4>(a, grid, st);
    case 5: return launch_fmt<FMT, 4, 5>(a, grid, st);
    case 6: return launch_fmt<FMT, 4, 6>(a, grid, st);
    case 7: return launch_fmt<FMT, 4, 7>(a, grid, st);
    case 8: return launch_fmt<FMT, 4, 8>(a, grid, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemv(int fmt, const GemvPlan& p, const void* x, int64_t M, int64_t N, int64_t K, const void* wp,
                       const void* scales, const void* zeros, void* y, bool swiglu, hipStream_t st) {
  GemvArgs a;
  a.swiglu = swiglu;
  a.w = reinterpret_cast<const uint4*>(wp);
  a.scales = scales;
  a.zeros = reinterpret_cast<const uint16_t*>(zeros);
  a.N = N;
  a.K = K;
  a.NB = p.NB;
  a.KT = p.KT;
  a.G4 = fmt == kFmtW4 ? ceil_div(K / kGroup, kScaleQuad) : 0;
  const unsigned grid = unsigned(p.NB);
  for (int c = 0; c < p.nchunks; ++c) {
    const int64_t m0 = int64_t(c) * kGemvMaxM;
    const int mr = int(M - m0 < kGemvMaxM ? M - m0 : int64_t(kGemvMaxM));
    a.x = reinterpret_cast<const uint16_t*>(x) + m0 * K;
    a.y = reinterpret_cast<uint16_t*>(y) + m0 * (swiglu ? N / 2 : N);  // SwiGLU output rows hold N / 2
    hipError_t e;
    if (fmt == kFmtBF16) e = launch_waves<kFmtBF16>(a, mr, p.waves, grid, st);
    else if (fmt == kFmtFP8) e = launch_waves<kFmtFP8>(a, mr, p.waves, grid, st);
    else e = launch_waves<kFmtW4>(a, mr, p.waves, grid, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace wqd
