// Tiled matrix-core kernel for wide verify batches (FP8 / BF16 weights, many
// activation rows): y = x . dequant(W)^T as a dense contraction.
//
// With speculative verification the layer multiplies batch x (k + 1) rows
// ("Making each token cheaper", sections "Speculative decoding" and the lab
// on verify width; CS336 lecture 10 notes, 3.2-3.3: the MLP's arithmetic
// intensity grows with the batch), and from a few hundred rows the matrix
// cores, not HBM, set the time.  Design for gfx950:
//   * a workgroup computes a BM x 256 tile of y (BM = 64 WM rows) with 4 WM
//     wavefronts, WM x 4, each owning 64 rows x 4 weight row blocks: 16
//     accumulators of v_mfma_f32_16x16x32_bf16 per wavefront;
//   * the packed 1 KiB weight tile is already the B-operand order (lane
//     16 kb + n: slice kb of weight row n), so weights go from memory straight
//     into registers (FP8 codes convert exactly to bf16, BF16 feeds as is),
//     each B fragment feeding 4 x row blocks; the FP8 row scale is applied
//     once at the end;
//   * K advances in chunks of 64 through an NS-stage pipeline (3 for BF16, 4
//     for FP8, whose weights take half the registers): while chunk c is
//     multiplied, the weights and x of chunks up to c + NS - 1 are in flight
//     (NS register sets for the weights, NS for this wavefront's x
//     fragments) and the x of chunk c + 1 is written into its LDS buffer (one
//     barrier per chunk).  The loop body is NS chunks, so every index is a
//     compile-time constant.  x sits in LDS in fragment order: fragment
//     (tile, x row block i, K-step s) is 1 KiB, lane 16 kb + j holding the 8 k
//     of row 16 i + j that pair with slice kb of the weights; reads are
//     conflict-free 16-byte LDS reads, all of a chunk's issued before its
//     first multiply;
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
  int nchunks;  // chunks of 64 k
  int cps;      // chunks per split
  int S;
};

constexpr int kGmMF = 4;   // x row blocks per wavefront
constexpr int kGmRB = 4;   // weight row blocks per wavefront
constexpr int kGmWN = 4;   // wavefronts along N
constexpr int kGmKC = 64;  // k per chunk

template <int FMT>
struct GmF {
  static_assert(FMT != kFmtW4, "W4A16 takes the LDS matrix-core kernel");
  static constexpr int TK = FMT == kFmtBF16 ? 32 : 64;  // K per tile
  static constexpr int SLK = TK / 4;                    // K per slice
  static constexpr int STEPS = SLK / 8;                 // 32-k steps per tile
  static constexpr int TPC = kGmKC / TK;                // tiles per chunk
  // pipeline stages: chunk c is multiplied while chunks up to c + NS - 1 are
  // in flight (FP8 weights take half the registers, so one more stage fits)
  static constexpr int NS = FMT == kFmtFP8 ? 4 : 3;
};

template <int FMT, int WM>
struct GmL {
  static constexpr int XB = 4 * WM;                                   // x row blocks per workgroup
  static constexpr int FRAGS = GmF<FMT>::TPC * XB * GmF<FMT>::STEPS;  // 1 KiB fragments per chunk (2 XB)
  static constexpr int BUF = FRAGS * 64;                               // uint4 per LDS buffer
  static constexpr int XPW = FRAGS / (WM * kGmWN);                    // fragments each wavefront stages
  static_assert(XPW * WM * kGmWN == FRAGS, "whole fragments per wavefront");
};

template <int FMT, int WM>
struct GmState {
  using F = GmF<FMT>;
  uint4 w[F::NS][kGmRB][F::TPC];       // weights of chunks c .. c + NS - 1
  uint4 xr[F::NS][GmL<FMT, WM>::XPW];  // x fragments loaded NS - 1 chunks ahead
  gm_f32x4_t acc[kGmMF][kGmRB];
  __amdgpu_buffer_rsrc_t wres[kGmRB], xres;
  int64_t kt0, m0;
  int lane, wave, wm;
};

// Weights of chunk c of the split into set H.
template <int FMT, int WM, int H>
__device__ __forceinline__ void gm_load_w(GmState<FMT, WM>& st, int c) {
  using F = GmF<FMT>;
#pragma unroll
  for (int b = 0; b < kGmRB; ++b)
#pragma unroll
    for (int t = 0; t < F::TPC; ++t) {
      // default cache policy: every x row block of the column block (and both
      // of its wavefront rows) reads these bytes, so they must stay in L2
      // (streaming them non-temporally cost 5-20% on the 70B verify shapes)
      const u32x4_t v =
          __builtin_amdgcn_raw_buffer_load_b128(st.wres[b], st.lane * 16, (c * F::TPC + t) * kTileBytes, 0);
      st.w[H][b][t] = make_uint4(v.x, v.y, v.z, v.w);
    }
}

// x fragments this wavefront stages for chunk c into set H: fragment
// f = wave * XPW + u of (tile t, x row block i, step s) order.
template <int FMT, int WM, int H>
__device__ __forceinline__ void gm_load_x(GmState<FMT, WM>& st, const GmArgs& a, int c) {
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
    st.xr[H][u] = make_uint4(v.x, v.y, v.z, v.w);
  }
}

template <int FMT, int WM, int H>
__device__ __forceinline__ void gm_store_x(const GmState<FMT, WM>& st, uint4* buf) {
  using L = GmL<FMT, WM>;
#pragma unroll
  for (int u = 0; u < L::XPW; ++u) buf[(st.wave * L::XPW + u) * 64 + st.lane] = st.xr[H][u];
}

// x fragments of the chunk in buf that this wavefront multiplies: 32-k step
// q, x row block i.
template <int FMT>
struct GmFrag {
  static constexpr int NQ = GmF<FMT>::TPC * GmF<FMT>::STEPS;  // 32-k steps per chunk (2)
  uint4 a[NQ][kGmMF];
};

template <int FMT, int WM>
__device__ __forceinline__ void gm_read_x(const GmState<FMT, WM>& st, const uint4* buf, GmFrag<FMT>& f) {
  using F = GmF<FMT>;
  using L = GmL<FMT, WM>;
  const uint4* xf = buf + st.lane;
#pragma unroll
  for (int q = 0; q < GmFrag<FMT>::NQ; ++q)
#pragma unroll
    for (int i = 0; i < kGmMF; ++i) {
      const int t = q / F::STEPS, s = q % F::STEPS;
      f.a[q][i] = xf[((t * L::XB + st.wm * kGmMF + i) * F::STEPS + s) * 64];
    }
}

// Multiply the x fragments with the weights of set H.
template <int FMT, int WM, int H>
__device__ __forceinline__ void gm_compute(GmState<FMT, WM>& st, const GmFrag<FMT>& f) {
  using F = GmF<FMT>;
  if constexpr (FMT == kFmtFP8) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      uint4 bm[kGmRB];
#pragma unroll
      for (int b = 0; b < kGmRB; ++b) {
        const uint4 wv = st.w[H][b][0];
        const uint32_t w0 = s == 0 ? wv.x : wv.z, w1 = s == 0 ? wv.y : wv.w;
        bm[b] = make_uint4(__builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<false>(w0)),
                           __builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<true>(w0)),
                           __builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<false>(w1)),
                           __builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<true>(w1)));
      }
#pragma unroll
      for (int i = 0; i < kGmMF; ++i)
#pragma unroll
        for (int b = 0; b < kGmRB; ++b) st.acc[i][b] = gm_mfma(f.a[s][i], bm[b], st.acc[i][b]);
    }
  } else {
#pragma unroll
    for (int t = 0; t < F::TPC; ++t)
#pragma unroll
      for (int i = 0; i < kGmMF; ++i)
#pragma unroll
        for (int b = 0; b < kGmRB; ++b) st.acc[i][b] = gm_mfma(f.a[t][i], st.w[H][b][t], st.acc[i][b]);
  }
}

// Step for chunk c = 3 it + H: read this wavefront's x fragments of chunk c
// from LDS, request chunk c + 2 (x first: its wait comes first; the LDS reads
// land meanwhile), multiply chunk c, write the x of chunk c + 1 (loaded a
// chunk ago) into its LDS buffer (that of chunk c - 2, released by the last
// barrier).  Loads and stores are unconditional: chunks past the split read
// zero weights (out of range of the weight resources), so no register of the
// ring is ever a merge of an old and a new value, which would make the
// compiler copy it (and wait for its load) at the loop's back edge.
template <int FMT, int WM, int H>
__device__ __forceinline__ void gm_step(GmState<FMT, WM>& st, const GmArgs& a, uint4 (*s_x)[GmL<FMT, WM>::BUF],
                                        int c) {
  constexpr int NS = GmF<FMT>::NS;
  constexpr int H1 = (H + 1) % NS, HL = (H + NS - 1) % NS;
  GmFrag<FMT> f;
  gm_read_x<FMT, WM>(st, s_x[H], f);
  __builtin_amdgcn_sched_barrier(0);
  gm_load_x<FMT, WM, HL>(st, a, c + NS - 1);
  gm_load_w<FMT, WM, HL>(st, c + NS - 1);
  __builtin_amdgcn_sched_barrier(0);
  gm_compute<FMT, WM, H>(st, f);
  gm_store_x<FMT, WM, H1>(st, s_x[H1]);
  __syncthreads();
}

template <int FMT, int WM>
__global__ __launch_bounds__(64 * WM * kGmWN) void gemm_kernel(GmArgs a) {
  using F = GmF<FMT>;
  using L = GmL<FMT, WM>;
  constexpr int NS = F::NS;
  __shared__ uint4 s_x[NS][L::BUF];

  // XCD-aware order: the workgroups of one XCD sweep the row blocks of x of
  // one column block back to back
  const int Lb = blockIdx.x, xcd = Lb & 7, wi = Lb >> 3;
  const int nbn = (wi / a.MB) * 8 + xcd, mb = wi % a.MB;
  if (nbn >= a.NBN) return;  // whole workgroup, before any barrier

  GmState<FMT, WM> st;
  st.lane = threadIdx.x & 63;
  st.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  st.wm = st.wave / kGmWN;
  const int wn = st.wave % kGmWN;
  const int split = blockIdx.y;
  const int c0 = split * a.cps;
  const int nch = a.nchunks - c0 < a.cps ? a.nchunks - c0 : a.cps;  // >= 1: the planner sizes S so
  const int nchp = (nch + NS - 1) / NS * NS;  // padded: chunks past the split read zero weights
  st.kt0 = int64_t(c0) * F::TPC;
  st.m0 = int64_t(mb) * 64 * WM;
  const int64_t tiles = a.KT - st.kt0 < int64_t(nch) * F::TPC ? a.KT - st.kt0 : int64_t(nch) * F::TPC;
  const int64_t nb0 = int64_t(nbn) * 16 + wn * kGmRB;
#pragma unroll
  for (int b = 0; b < kGmRB; ++b) {
    // row blocks past the matrix and tiles past the split read zeros
    const bool live = nb0 + b < a.NB;
    const int64_t nb = live ? nb0 + b : 0;
    st.wres[b] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint4*>(a.w + (nb * a.KT + st.kt0) * (kTileBytes / 16)),
                                                   0, live ? uint32_t(tiles) * kTileBytes : 0u, 0x00020000);
#pragma unroll
    for (int i = 0; i < kGmMF; ++i) st.acc[i][b] = gm_f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  st.xres = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.x), 0, 0x7FFFFFF0, 0x00020000);

  // prologue: chunks 0 .. NS - 2 requested, chunk 0 staged
  gm_load_x<FMT, WM, 0>(st, a, 0);
  gm_load_w<FMT, WM, 0>(st, 0);
  gm_load_x<FMT, WM, 1>(st, a, 1);
  gm_load_w<FMT, WM, 1>(st, 1);
  if constexpr (NS > 3) {
    gm_load_x<FMT, WM, 2>(st, a, 2);
    gm_load_w<FMT, WM, 2>(st, 2);
  }
  gm_store_x<FMT, WM, 0>(st, s_x[0]);
  __syncthreads();
  for (int c = 0; c < nchp; c += NS) {
    gm_step<FMT, WM, 0>(st, a, s_x, c);
    gm_step<FMT, WM, 1>(st, a, s_x, c + 1);
    gm_step<FMT, WM, 2>(st, a, s_x, c + 2);
    if constexpr (NS > 3) gm_step<FMT, WM, 3 % NS>(st, a, s_x, c + 3);
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
  if (p.wm == 2)
    hipLaunchKernelGGL((gemm_kernel<FMT, 2>), dim3(grid, unsigned(p.S)), dim3(64 * 2 * kGmWN), 0, st, a);
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
  a.G4 = 0;
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
    return hipErrorInvalidValue;  // W4A16 takes the LDS matrix-core kernel
  if (e != hipSuccess || p.S == 1) return e;
  return launch_splitk_reduce(fmt, a.part, p.S, M, N, scales, y, st);
}

}  // namespace wqd
