// Streaming matrix-core decode kernel for a few activation rows (M <= 16).
//
// The work split of the streaming kernels (one workgroup per 16-row block of
// W over all of K, W wavefronts on contiguous shares of K, fixed-order
// reductions at the end), with the products on the matrix cores: per 32 k,
// one v_mfma_f32_16x16x32_bf16 takes the x fragment as A (lane 16 kb + j:
// 8 k of activation row j) and the dequantised tile slice as B (lane
// 16 kb + n: the same 8 k of weight row n, straight from the packed layout).
// The VALU only dequantises and applies scales, so its cost per weight byte
// no longer grows with the number of rows.
//
// x fragments are read from L2 per tile through a buffer resource: lanes of
// rows j >= M get an out-of-range offset and read zeros without touching
// memory.  Weights run seven tiles ahead of the arithmetic (three with two
// row blocks per wavefront) and x two tiles ahead; every load is unconditional (weights past the share are out of
// range of their buffer resource, x reads are clamped to the share) and the
// tile steps are straight-line code, so the compiler's waits are exact.
//
// W4A16: a tile contributes s * (P - (128 + z) * X) per weight row, with
// P = x . (128 + q) and X = x . 1 from matrix-core chains of the same shape
// (the all-ones B operand), so q == z == 0 cancels exactly.
#include "wqd_device.h"
#include "wqd_internal.h"
#include "wqd_plan.h"

namespace wqd {

typedef __bf16 mc_bf16x8_t __attribute__((ext_vector_type(8)));
typedef float mc_f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ mc_f32x4_t mc_mfma(uint4 a, uint4 b, mc_f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mc_bf16x8_t, a),
                                                 __builtin_bit_cast(mc_bf16x8_t, b), c, 0, 0, 0);
}

struct McArgs {
  const uint16_t* x;
  uint16_t* y;
  const uint4* w;
  const void* scales;
  const uint16_t* zeros;
  int64_t M, N, K, KT, G4, NB;
  int per_wave;
  int swiglu;  // packed gate/up pairs: store silu(gate) * up (store_out)
};

// RB: 16-row blocks per wavefront (each x fragment feeds RB weight tiles).
template <int FMT, int RB>
struct McC {
  static constexpr int TK = FMT == kFmtBF16 ? 32 : FMT == kFmtFP8 ? 64 : 128;  // K per tile
  static constexpr int SLK = TK / 4;                                             // K per slice
  static constexpr int XU = SLK / 8;  // x uint4 per lane and tile = matrix-core steps per tile
  static constexpr int LW = RB == 1 ? 7 : 3;  // tile steps whose weights are loaded ahead (RB = 2, 3: 3)
  static constexpr int LX = 2;                // x tiles loaded ahead
  static constexpr int RW = LW + 1;           // ring sizes
  static constexpr int RX = LX + 1;
};

template <int FMT, int RB>
struct McState {
  using C = McC<FMT, RB>;
  uint4 w[C::RW][RB];
  uint4 x[C::RX][C::XU];
  uint2 s[3][RB];     // W4A16 scale quads (4 fp16 of this lane's weight row)
  uint32_t z[3][RB];  // W4A16 zero quads (4 nibbles)
  mc_f32x4_t acc[RB];
  __amdgpu_buffer_rsrc_t wres[RB], xres;
  const uint2* sbase[RB];
  const uint16_t* zbase[RB];
  uint32_t xoff;  // this lane's x byte offset (out of range for rows >= M)
  int kslice;     // k of this lane's slice inside a tile
  int64_t klim;   // K - the share's first k: x pieces at or past it are zero
  int lane, total, last;
};

template <int FMT, int RB, int T>
__device__ __forceinline__ void mc_load_w(McState<FMT, RB>& st) {
  using C = McC<FMT, RB>;
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    // cache policy 2: non-temporal (weights are read once per step)
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(st.wres[b], T * kTileBytes + st.lane * 16, 0, 2);
    st.w[T % C::RW][b] = make_uint4(v.x, v.y, v.z, v.w);
  }
}

// x fragments of tile T (clamped to the share).  FP8 / BF16 tiles may end
// past K (K % 8 == 0, so a 16-byte piece lies wholly before or after it):
// pieces past K get an out-of-range offset and read as zero.
template <int FMT, int RB, int T>
__device__ __forceinline__ void mc_load_x(McState<FMT, RB>& st) {
  using C = McC<FMT, RB>;
  const int tt = T < st.last ? T : st.last;
  const uint32_t off = st.xoff + uint32_t(tt) * (C::TK * 2);
#pragma unroll
  for (int u = 0; u < C::XU; ++u) {
    uint32_t o = off + 16 * u;
    if constexpr (FMT != kFmtW4) o = tt * C::TK + st.kslice + 8 * u < st.klim ? o : 0x80000000u;
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(st.xres, o, 0, 0);
    st.x[T % C::RX][u] = make_uint4(v.x, v.y, v.z, v.w);
  }
}

template <int FMT, int RB, int Q>
__device__ __forceinline__ void mc_load_sz(McState<FMT, RB>& st) {
  const int q = (4 * Q < st.last ? 4 * Q : st.last) / kScaleQuad;
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    st.s[Q % 3][b] = st.sbase[b][q * kTileRows];
    st.z[Q % 3][b] = st.zbase[b][q * kTileRows];
  }
}

template <int FMT, int RB, int T>
__device__ __forceinline__ void mc_compute(McState<FMT, RB>& st) {
  using C = McC<FMT, RB>;
  const uint4* xf = st.x[T % C::RX];
  if constexpr (FMT == kFmtW4) {
    const uint32_t mask = vgpr_const(0x000F000Fu), magic = vgpr_const(0x43004300u);
    const uint4 ones = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);
    mc_f32x4_t X = {0.f, 0.f, 0.f, 0.f}, P[RB];
#pragma unroll
    for (int b = 0; b < RB; ++b) P[b] = mc_f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      X = mc_mfma(xf[s], ones, X);
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        const uint4 wv = st.w[T % C::RW][b];
        const uint32_t wd = s == 0 ? wv.x : s == 1 ? wv.y : s == 2 ? wv.z : wv.w;
        const uint4 bm = make_uint4(and_or_v(wd, mask, magic), and_or_v(wd >> 4, mask, magic),
                                    and_or_v(wd >> 8, mask, magic), and_or_v(wd >> 12, mask, magic));
        P[b] = mc_mfma(xf[s], bm, P[b]);
      }
    }
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      const uint2 sq = st.s[(T / 4) % 3][b];
      const uint32_t sw = ((T & 3) < 2 ? sq.x : sq.y) >> (16 * (T & 1));
      const float sc = __half2float(__ushort_as_half(uint16_t(sw & 0xFFFFu)));
      const float zc = 128.0f + float((st.z[(T / 4) % 3][b] >> (4 * (T & 3))) & 0xFu);
#pragma unroll
      for (int r = 0; r < 4; ++r) st.acc[b][r] = fmaf(sc, fmaf(-zc, X[r], P[b][r]), st.acc[b][r]);
    }
  } else if constexpr (FMT == kFmtFP8) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        const uint4 wv = st.w[T % C::RW][b];
        const uint32_t w0 = s == 0 ? wv.x : wv.z, w1 = s == 0 ? wv.y : wv.w;
        const uint4 bm = make_uint4(__builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<false>(w0)),
                                    __builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<true>(w0)),
                                    __builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<false>(w1)),
                                    __builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<true>(w1)));
        st.acc[b] = mc_mfma(xf[s], bm, st.acc[b]);
      }
  } else {
#pragma unroll
    for (int b = 0; b < RB; ++b) st.acc[b] = mc_mfma(xf[0], st.w[T % C::RW][b], st.acc[b]);
  }
}

// Prologue: weight tiles 0 .. LW - 1 and x tiles 0 .. LX - 1, the weights and
// x of one tile issued together (loads complete in issue order).
template <int FMT, int RB, int NT, int T>
__device__ __forceinline__ void mc_prologue(McState<FMT, RB>& st) {
  using C = McC<FMT, RB>;
  if constexpr (T < NT && (T < C::LW || T < C::LX)) {
    if constexpr (T < C::LW) mc_load_w<FMT, RB, T>(st);
    if constexpr (T < C::LX) mc_load_x<FMT, RB, T>(st);
    mc_prologue<FMT, RB, NT, T + 1>(st);
  }
}

// Tiles T .. NT - 1 as straight-line code with early exits: each step loads
// the weights LW tiles ahead, x LX tiles ahead and (W4A16, every fourth tile)
// the scale / zero quad two ahead, then multiplies tile T.
template <int FMT, int RB, int NT, int T>
__device__ __forceinline__ void mc_tiles(McState<FMT, RB>& st) {
  using C = McC<FMT, RB>;
  if constexpr (T < NT) {
    if (T >= st.total) return;
    if constexpr (T + C::LW < NT) mc_load_w<FMT, RB, T + C::LW>(st);
    if constexpr (T + C::LX < NT) mc_load_x<FMT, RB, T + C::LX>(st);
    if constexpr (FMT == kFmtW4 && T % 4 == 0 && T + 8 < NT) mc_load_sz<FMT, RB, T / 4 + 2>(st);
    // keep the loads here: left to itself the scheduler sinks them to just
    // before their use, which would leave nothing in flight during the math
    __builtin_amdgcn_sched_barrier(0);
    mc_compute<FMT, RB, T>(st);
    mc_tiles<FMT, RB, NT, T + 1>(st);
  }
}

template <int FMT, int W, int NT, int RB>
__global__ __launch_bounds__(64 * W) void gemv_mc_kernel(McArgs a) {
  using C = McC<FMT, RB>;
  __shared__ float s_red[W][RB][16][kTileRows];

  const int lane = threadIdx.x & 63, kb = lane >> 4, n = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nb0 = int64_t(blockIdx.x) * RB;
  const int64_t kt_begin = int64_t(wave) * a.per_wave;
  const int64_t rem = a.KT - kt_begin;

  McState<FMT, RB> st;
  st.lane = lane;
  st.total = rem <= 0 ? 0 : (rem < a.per_wave ? int(rem) : a.per_wave);
  st.last = st.total - 1;
#pragma unroll
  for (int b = 0; b < RB; ++b) st.acc[b] = mc_f32x4_t{0.f, 0.f, 0.f, 0.f};

  if (st.total > 0) {
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      // a block past N (odd block count) gets an empty resource: its loads
      // read zeros and its outputs are never stored
      const bool live = nb0 + b < a.NB;
      const int64_t nb = live ? nb0 + b : nb0;
      st.wres[b] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint4*>(a.w + (nb * a.KT + kt_begin) * (kTileBytes / 16)),
                                                     0, live ? st.total * kTileBytes : 0, 0x00020000);
      const int64_t q0 = FMT == kFmtW4 ? (nb * a.G4 + kt_begin / kScaleQuad) * kTileRows + n : 0;
      st.sbase[b] = reinterpret_cast<const uint2*>(a.scales) + q0;
      st.zbase[b] = a.zeros + q0;
    }
    // x rows of this share; row j of lane (kb, j), slice kb.  Rows past M
    // (and nothing else) fall outside the resource's 2 GiB range.
    st.xres = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.x + kt_begin * C::TK), 0, 0x7FFFFFF0,
                                                0x00020000);
    st.xoff = n < a.M ? uint32_t((int64_t(n) * a.K + kb * C::SLK) * 2) : 0x80000000u;
    st.kslice = kb * C::SLK;
    st.klim = a.K - kt_begin * C::TK;

    // prologue: the first LW weight tiles, LX x tiles and two scale quads
    if constexpr (FMT == kFmtW4) {
      mc_load_sz<FMT, RB, 0>(st);
      if constexpr (NT > 4) mc_load_sz<FMT, RB, 1>(st);
    }
    mc_prologue<FMT, RB, NT, 0>(st);
    __builtin_amdgcn_sched_barrier(0);
    mc_tiles<FMT, RB, NT, 0>(st);
  }

  // lane (kb, n) holds activation rows 4 kb + r of weight row n; then the W
  // wavefronts in a fixed order
#pragma unroll
  for (int b = 0; b < RB; ++b)
#pragma unroll
    for (int r = 0; r < 4; ++r) s_red[wave][b][4 * kb + r][n] = st.acc[b][r];
  __syncthreads();
  for (int i = threadIdx.x; i < RB * a.M * kTileRows; i += 64 * W) {
    const int b = i / (int(a.M) * kTileRows), mi = i % (int(a.M) * kTileRows);
    const int m = mi / kTileRows, r = mi % kTileRows;
    float v = s_red[0][b][m][r];
#pragma unroll
    for (int w = 1; w < W; ++w) v += s_red[w][b][m][r];
    const int64_t row = (nb0 + b) * kTileRows + r;
    const bool live = row < a.N;
    if (FMT == kFmtFP8 && live) v *= reinterpret_cast<const float*>(a.scales)[row];
    store_out<8>(a.y, a.N, a.swiglu, m, row, v, live);  // element i ^ 8 (thread ^ 8) is row ^ 8
  }
}

template <int FMT, int NT, int RB>
static hipError_t launch_mc_w(const McArgs& a, int waves, unsigned grid, hipStream_t st) {
  switch (waves) {
    case 4: hipLaunchKernelGGL((gemv_mc_kernel<FMT, 4, NT, RB>), dim3(grid), dim3(256), 0, st, a); break;
    case 8: hipLaunchKernelGGL((gemv_mc_kernel<FMT, 8, NT, RB>), dim3(grid), dim3(512), 0, st, a); break;
    case 16:
      // three row blocks do not fit the 128 registers of a 16-wavefront workgroup
      if constexpr (RB == 3) return hipErrorInvalidValue;
      else hipLaunchKernelGGL((gemv_mc_kernel<FMT, 16, NT, RB>), dim3(grid), dim3(1024), 0, st, a);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int FMT>
static hipError_t launch_mc_fmt(const McArgs& a, const McPlan& p, hipStream_t st) {
  const unsigned grid = unsigned(ceil_div(p.NB, p.rb));
  if (p.rb == 1) {
    if (p.per_wave <= 16) return launch_mc_w<FMT, 16, 1>(a, p.waves, grid, st);
    if (p.per_wave <= 32) return launch_mc_w<FMT, 32, 1>(a, p.waves, grid, st);
  } else if (p.rb == 2) {
    if (p.per_wave <= 16) return launch_mc_w<FMT, 16, 2>(a, p.waves, grid, st);
    if (p.per_wave <= 32) return launch_mc_w<FMT, 32, 2>(a, p.waves, grid, st);
  } else if (p.rb == 3) {
    if (p.per_wave <= 16) return launch_mc_w<FMT, 16, 3>(a, p.waves, grid, st);
    if (p.per_wave <= 32) return launch_mc_w<FMT, 32, 3>(a, p.waves, grid, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemv_mc(int fmt, const McPlan& p, const void* x, int64_t M, int64_t N, int64_t K, const void* wp,
                          const void* scales, const void* zeros, void* y, bool swiglu, hipStream_t st) {
  if (M < 1 || M > kMcMaxM) return hipErrorInvalidValue;
  McArgs a;
  a.swiglu = swiglu;
  a.x = reinterpret_cast<const uint16_t*>(x);
  a.y = reinterpret_cast<uint16_t*>(y);
  a.w = reinterpret_cast<const uint4*>(wp);
  a.scales = scales;
  a.zeros = reinterpret_cast<const uint16_t*>(zeros);
  a.M = M;
  a.N = N;
  a.K = K;
  a.KT = p.KT;
  a.G4 = fmt == kFmtW4 ? ceil_div(K / kGroup, kScaleQuad) : 0;
  a.NB = p.NB;
  a.per_wave = p.per_wave;
  if (fmt == kFmtBF16) return launch_mc_fmt<kFmtBF16>(a, p, st);
  if (fmt == kFmtFP8) return launch_mc_fmt<kFmtFP8>(a, p, st);
  return launch_mc_fmt<kFmtW4>(a, p, st);
}

}  // namespace wqd
