// Tiled matrix-core kernel for wide verify batches (more than 64 activation
// rows): y = x . dequant(W)^T as a dense contraction.
//
// With speculative verification the layer multiplies batch x (k + 1) rows
// ("Making each token cheaper", sections "Speculative decoding" and the lab
// on verify width; CS336 lecture 10 notes, 3.2-3.3: the MLP's arithmetic
// intensity grows with the batch), and from roughly a hundred W4A16 rows the
// matrix cores, not HBM, set the time.  Design for gfx950:
//   * a workgroup computes a BM x 256 tile of y (BM = 64 WM rows) with 4 WM
//     wavefronts, WM x 4, each owning 64 rows x 4 weight row blocks: 16
//     accumulators of v_mfma_f32_16x16x32_bf16 per wavefront;
//   * the packed 1 KiB weight tile is already the B-operand order (lane
//     16 kb + n: slice kb of weight row n), so weights go from memory straight
//     into registers, dequantised there (W4A16 nibble pairs become
//     bf16 128 + q with one AND-OR; FP8 codes convert exactly; BF16 as is),
//     each B fragment feeding 4 x row blocks;
//   * x is staged per chunk of 128 k in LDS (two buffers, one barrier per
//     chunk) in fragment order: fragment (tile, x row block i, K-step s) is
//     1 KiB, lane 16 kb + j holding the 8 k of row 16 i + j that pair with
//     slice kb of the weights; every wavefront loads 4 fragments of the next
//     chunk into registers while the current one is multiplied, then writes
//     them.  Reads back are conflict-free 16-byte LDS reads;
//   * weights and (W4A16) scale / zero of the next chunk are loaded during
//     the current one (two register sets, static indices: the loop body is
//     two chunks);
//   * W4A16 groups are 128 k, one chunk: P = x . (128 + q) and X = x . 1 come
//     from matrix-core chains of the same shape (so q == z == 0 cancels
//     exactly) and acc += s * (P - (128 + z) * X) in float32; FP8 applies the
//     row scale at the end.  Dequantised weights are never rounded;
//   * XCD-aware order: consecutive workgroups of one XCD (dispatch is
//     round-robin over the 8 XCDs) take the row blocks of x of one column
//     block, so its weights come from HBM once and then from that XCD's L2;
//   * when the tiles give too few workgroups, K is split S ways over grid y;
//     the float32 partials go to the workspace and the fixed-order split-K
//     sum finishes them.
#include "wqd_device.h"
#include "wqd_internal.h"
#include "wqd_plan.h"

namespace wqd {

typedef __bf16 gm_bf16x8_t __attribute__((ext_vector_type(8)));
typedef float gm_f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ gm_f32x4_t gm_mfma(uint4 a, uint4 b, gm_f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(gm_bf16x8_t, a),
                                                 __builtin_bit_cast(gm_bf16x8_t, b), c, 0, 0, 0);
}

struct GmArgs {
  const uint16_t* x;
  uint16_t* y;
  float* part;  // split partials [S][M][N] (S > 1)
  const uint4* w;
  const void* scales;
  const uint16_t* zeros;
  int64_t M, N, K, KT, G4, NB;
  int NBN, MB;  // 256-column blocks, BM-row blocks
  int nchunks;  // chunks of 128 k
  int cps;      // chunks per split
  int S;
};

constexpr int kGmMF = 4;   // x row blocks per wavefront
constexpr int kGmRB = 4;   // weight row blocks per wavefront
constexpr int kGmWN = 4;   // wavefronts along N
constexpr int kGmKC = 128;  // k per chunk

template <int FMT>
struct GmF {
  static constexpr int TK = FMT == kFmtBF16 ? 32 : FMT == kFmtFP8 ? 64 : 128;  // K per tile
  static constexpr int SLK = TK / 4;                                             // K per slice
  static constexpr int STEPS = SLK / 8;                                          // 32-k steps per tile
  static constexpr int TPC = kGmKC / TK;                                         // tiles per chunk
};

template <int FMT, int WM>
struct GmL {
  static constexpr int XB = 4 * WM;                          // x row blocks per workgroup
  static constexpr int FRAGS = GmF<FMT>::TPC * XB * GmF<FMT>::STEPS;  // 1 KiB fragments per chunk (4 XB)
  static constexpr int BUF = FRAGS * 64;                      // uint4 per LDS buffer
  static constexpr int XPW = FRAGS / (WM * kGmWN);           // fragments each wavefront stages
  static_assert(XPW * WM * kGmWN == FRAGS, "whole fragments per wavefront");
};

template <int FMT>
struct GmState {
  using F = GmF<FMT>;
  uint4 w[2][kGmRB][F::TPC];
  uint32_t sw[2][kGmRB], zw[2][kGmRB];  // W4A16: fp16 scale bits and zero quad of the chunk's group
  uint4 xr[kGmMF];                      // x fragments of the next chunk (XPW == kGmMF)
  gm_f32x4_t acc[kGmMF][kGmRB];
  __amdgpu_buffer_rsrc_t wres[kGmRB], sres[kGmRB], zres[kGmRB], xres;
  int64_t kt0, m0;
  int lane, wave, wm, nch;
};

// Weights (and W4A16 scale / zero) of chunk c of the split into set H.
template <int FMT, int H>
__device__ __forceinline__ void gm_load_w(GmState<FMT>& st, int c) {
  using F = GmF<FMT>;
#pragma unroll
  for (int b = 0; b < kGmRB; ++b) {
#pragma unroll
    for (int t = 0; t < F::TPC; ++t) {
      // cache policy 2: non-temporal (each weight byte is read by the few
      // workgroups of its column block, then not again)
      const u32x4_t v =
          __builtin_amdgcn_raw_buffer_load_b128(st.wres[b], st.lane * 16, (c * F::TPC + t) * kTileBytes, 2);
      st.w[H][b][t] = make_uint4(v.x, v.y, v.z, v.w);
    }
    if constexpr (FMT == kFmtW4) {
      const int64_t kt = st.kt0 + c;
      const int q = int(kt / kScaleQuad), j = int(kt % kScaleQuad);
      const int n = st.lane & 15;
      st.sw[H][b] = __builtin_amdgcn_raw_buffer_load_b16(st.sres[b], n * (kScaleQuad * 2),
                                                         q * (kTileRows * kScaleQuad * 2) + j * 2, 0);
      st.zw[H][b] = __builtin_amdgcn_raw_buffer_load_b16(st.zres[b], n * 2, q * (kTileRows * 2), 0);
    }
  }
}

// x fragments this wavefront stages for chunk c: fragment f = wave * XPW + u
// of (tile t, x row block i, step s) order.
template <int FMT, int WM>
__device__ __forceinline__ void gm_load_x(GmState<FMT>& st, const GmArgs& a, int c) {
  using F = GmF<FMT>;
  using L = GmL<FMT, WM>;
  const int kb = st.lane >> 4, j = st.lane & 15;
#pragma unroll
  for (int u = 0; u < L::XPW; ++u) {
    const int f = st.wave * L::XPW + u;
    const int t = f / (L::XB * F::STEPS), i = (f / F::STEPS) % L::XB, s = f % F::STEPS;
    const int64_t row = st.m0 + 16 * i + j;
    const int64_t k = (st.kt0 + int64_t(c) * F::TPC + t) * F::TK + kb * F::SLK + 8 * s;
    const uint32_t off = row < a.M && k < a.K ? uint32_t((row * a.K + k) * 2) : 0x80000000u;
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(st.xres, off, 0, 0);
    st.xr[u] = make_uint4(v.x, v.y, v.z, v.w);
  }
}

template <int FMT, int WM>
__device__ __forceinline__ void gm_store_x(const GmState<FMT>& st, uint4* buf) {
  using L = GmL<FMT, WM>;
#pragma unroll
  for (int u = 0; u < L::XPW; ++u) buf[(st.wave * L::XPW + u) * 64 + st.lane] = st.xr[u];
}

// Multiply chunk c (x in buf, weights in set H).
template <int FMT, int WM, int H>
__device__ __forceinline__ void gm_compute(GmState<FMT>& st, const uint4* buf, int c) {
  using F = GmF<FMT>;
  using L = GmL<FMT, WM>;
  const uint4* xf = buf + st.lane;
  if constexpr (FMT == kFmtW4) {
    const uint32_t mask = vgpr_const(0x000F000Fu), magic = vgpr_const(0x43004300u);
    const uint4 ones = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);
    gm_f32x4_t X[kGmMF], P[kGmMF][kGmRB];
#pragma unroll
    for (int i = 0; i < kGmMF; ++i) {
      X[i] = gm_f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int b = 0; b < kGmRB; ++b) P[i][b] = gm_f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint4 bm[kGmRB];
#pragma unroll
      for (int b = 0; b < kGmRB; ++b) {
        const uint4 wv = st.w[H][b][0];
        const uint32_t wd = s == 0 ? wv.x : s == 1 ? wv.y : s == 2 ? wv.z : wv.w;
        bm[b] = make_uint4(and_or_v(wd, mask, magic), and_or_v(wd >> 4, mask, magic), and_or_v(wd >> 8, mask, magic),
                           and_or_v(wd >> 12, mask, magic));
      }
#pragma unroll
      for (int i = 0; i < kGmMF; ++i) {
        const uint4 af = xf[((st.wm * kGmMF + i) * 4 + s) * 64];
        X[i] = gm_mfma(af, ones, X[i]);
#pragma unroll
        for (int b = 0; b < kGmRB; ++b) P[i][b] = gm_mfma(af, bm[b], P[i][b]);
      }
    }
    // the chunk is one group; chunks past the split get scale 0
    const int jq = int((st.kt0 + c) % kScaleQuad);
    const bool live = c < st.nch;
#pragma unroll
    for (int b = 0; b < kGmRB; ++b) {
      const float s0 = __half2float(__ushort_as_half(uint16_t(st.sw[H][b])));
      const float sc = live ? s0 : 0.f;
      const float zc = 128.0f + float((st.zw[H][b] >> (4 * jq)) & 0xFu);
#pragma unroll
      for (int i = 0; i < kGmMF; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) st.acc[i][b][r] = fmaf(sc, fmaf(-zc, X[i][r], P[i][b][r]), st.acc[i][b][r]);
    }
  } else if constexpr (FMT == kFmtFP8) {
#pragma unroll
    for (int t = 0; t < F::TPC; ++t)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        uint4 bm[kGmRB];
#pragma unroll
        for (int b = 0; b < kGmRB; ++b) {
          const uint4 wv = st.w[H][b][t];
          const uint32_t w0 = s == 0 ? wv.x : wv.z, w1 = s == 0 ? wv.y : wv.w;
          bm[b] = make_uint4(__builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<false>(w0)),
                             __builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<true>(w0)),
                             __builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<false>(w1)),
                             __builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<true>(w1)));
        }
#pragma unroll
        for (int i = 0; i < kGmMF; ++i) {
          const uint4 af = xf[((t * L::XB + st.wm * kGmMF + i) * 2 + s) * 64];
#pragma unroll
          for (int b = 0; b < kGmRB; ++b) st.acc[i][b] = gm_mfma(af, bm[b], st.acc[i][b]);
        }
      }
  } else {
#pragma unroll
    for (int t = 0; t < F::TPC; ++t)
#pragma unroll
      for (int i = 0; i < kGmMF; ++i) {
        const uint4 af = xf[(t * L::XB + st.wm * kGmMF + i) * 64];
#pragma unroll
        for (int b = 0; b < kGmRB; ++b) st.acc[i][b] = gm_mfma(af, st.w[H][b][t], st.acc[i][b]);
      }
  }
}

template <int FMT, int WM>
__global__ __launch_bounds__(64 * WM * kGmWN) void gemm_kernel(GmArgs a) {
  using F = GmF<FMT>;
  using L = GmL<FMT, WM>;
  static_assert(L::XPW == kGmMF, "x staging registers");
  __shared__ uint4 s_x[2][L::BUF];

  // XCD-aware order: the workgroups of one XCD sweep the row blocks of x of
  // one column block back to back
  const int Lb = blockIdx.x, xcd = Lb & 7, wi = Lb >> 3;
  const int nbn = (wi / a.MB) * 8 + xcd, mb = wi % a.MB;
  if (nbn >= a.NBN) return;  // whole workgroup, before any barrier

  GmState<FMT> st;
  st.lane = threadIdx.x & 63;
  st.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  st.wm = st.wave / kGmWN;
  const int wn = st.wave % kGmWN;
  const int split = blockIdx.y;
  const int c0 = split * a.cps;
  st.nch = a.nchunks - c0 < a.cps ? a.nchunks - c0 : a.cps;  // >= 1: the planner sizes S so
  st.kt0 = int64_t(c0) * F::TPC;
  st.m0 = int64_t(mb) * 64 * WM;
  const int64_t tiles = a.KT - st.kt0 < int64_t(st.nch) * F::TPC ? a.KT - st.kt0 : int64_t(st.nch) * F::TPC;
  const int64_t nb0 = int64_t(nbn) * 16 + wn * kGmRB;
#pragma unroll
  for (int b = 0; b < kGmRB; ++b) {
    // row blocks past the matrix get empty resources: zeros, never stored
    const bool live = nb0 + b < a.NB;
    const int64_t nb = live ? nb0 + b : 0;
    st.wres[b] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint4*>(a.w + (nb * a.KT + st.kt0) * (kTileBytes / 16)),
                                                   0, live ? uint32_t(tiles) * kTileBytes : 0u, 0x00020000);
    if constexpr (FMT == kFmtW4) {
      const uint16_t* sb = reinterpret_cast<const uint16_t*>(a.scales) + nb * a.G4 * kTileRows * kScaleQuad;
      const uint16_t* zb = a.zeros + nb * a.G4 * kTileRows;
      st.sres[b] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(sb), 0,
                                                     live ? uint32_t(a.G4 * kTileRows * kScaleQuad * 2) : 0u,
                                                     0x00020000);
      st.zres[b] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(zb), 0,
                                                     live ? uint32_t(a.G4 * kTileRows * 2) : 0u, 0x00020000);
    }
#pragma unroll
    for (int i = 0; i < kGmMF; ++i) st.acc[i][b] = gm_f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  st.xres = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.x), 0, 0x7FFFFFF0, 0x00020000);

  // chunk 0 staged, its weights requested
  gm_load_x<FMT, WM>(st, a, 0);
  gm_load_w<FMT, 0>(st, 0);
  gm_store_x<FMT, WM>(st, s_x[0]);
  __syncthreads();
  const int nch2 = (st.nch + 1) & ~1;
  for (int c = 0; c < nch2; c += 2) {
    // chunk c + 1 requested (x first: its wait comes first), chunk c multiplied
    gm_load_x<FMT, WM>(st, a, c + 1);
    gm_load_w<FMT, 1>(st, c + 1);
    gm_compute<FMT, WM, 0>(st, s_x[0], c);
    gm_store_x<FMT, WM>(st, s_x[1]);  // buffer 1 held chunk c - 1: released by the last barrier
    __syncthreads();
    if (c + 2 < nch2) {
      gm_load_x<FMT, WM>(st, a, c + 2);
      gm_load_w<FMT, 0>(st, c + 2);
    }
    gm_compute<FMT, WM, 1>(st, s_x[1], c + 1);
    if (c + 2 < nch2) gm_store_x<FMT, WM>(st, s_x[0]);
    __syncthreads();
  }

  // lane (kb, n) holds rows 4 kb + r of each x row block, column n of each row block
  const int kb = st.lane >> 4, n = st.lane & 15;
#pragma unroll
  for (int b = 0; b < kGmRB; ++b) {
    const int64_t col = (nb0 + b) * kTileRows + n;
    if (nb0 + b >= a.NB || col >= a.N) continue;
    const float cs = FMT == kFmtFP8 && a.S == 1 ? reinterpret_cast<const float*>(a.scales)[col] : 1.f;
#pragma unroll
    for (int i = 0; i < kGmMF; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = st.m0 + (st.wm * kGmMF + i) * 16 + 4 * kb + r;
        if (row >= a.M) continue;
        if (a.S > 1)
          a.part[(int64_t(split) * a.M + row) * a.N + col] = st.acc[i][b][r];
        else
          a.y[row * a.N + col] = uint16_t(f32_to_bf16_rne(st.acc[i][b][r] * cs));
      }
  }
}

template <int FMT>
static hipError_t launch_gm_fmt(const GmArgs& a, const GmPlan& p, hipStream_t st) {
  const unsigned grid = unsigned(ceil_div(p.NBN, 8) * 8 * p.MB);
  if (p.wm == 2 && FMT != kFmtW4)
    hipLaunchKernelGGL((gemm_kernel<FMT, FMT != kFmtW4 ? 2 : 1>), dim3(grid, unsigned(p.S)), dim3(64 * 2 * kGmWN), 0,
                       st, a);
  else if (p.wm == 1)
    hipLaunchKernelGGL((gemm_kernel<FMT, 1>), dim3(grid, unsigned(p.S)), dim3(64 * 1 * kGmWN), 0, st, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_gemm(int fmt, const GmPlan& p, const void* x, int64_t M, int64_t N, int64_t K, const void* wp,
                       const void* scales, const void* zeros, void* y, void* ws, hipStream_t st) {
  GmArgs a;
  a.x = reinterpret_cast<const uint16_t*>(x);
  a.y = reinterpret_cast<uint16_t*>(y);
  a.part = reinterpret_cast<float*>(ws);
  a.w = reinterpret_cast<const uint4*>(wp);
  a.scales = scales;
  a.zeros = reinterpret_cast<const uint16_t*>(zeros);
  a.M = M;
  a.N = N;
  a.K = K;
  a.KT = p.KT;
  a.G4 = fmt == kFmtW4 ? ceil_div(K / kGroup, kScaleQuad) : 0;
  a.NB = p.NB;
  a.NBN = int(p.NBN);
  a.MB = int(p.MB);
  a.nchunks = int(p.nchunks);
  a.cps = int(p.cps);
  a.S = p.S;
  hipError_t e;
  if (fmt == kFmtBF16)
    e = launch_gm_fmt<kFmtBF16>(a, p, st);
  else if (fmt == kFmtFP8)
    e = launch_gm_fmt<kFmtFP8>(a, p, st);
  else
    e = launch_gm_fmt<kFmtW4>(a, p, st);
  if (e != hipSuccess || p.S == 1) return e;
  return launch_splitk_reduce(fmt, a.part, p.S, M, N, scales, y, st);
}

}  // namespace wqd
