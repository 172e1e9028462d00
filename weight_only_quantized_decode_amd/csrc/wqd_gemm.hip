// Tiled matrix-core kernel for wide verify batches (many activation rows):
// y = x . dequant(W)^T as a dense contraction.
//
// With speculative verification the layer multiplies batch x (k + 1) rows
// ("Making each token cheaper", sections "Speculative decoding" and the lab
// on verify width; CS336 lecture 10 notes, 3.2-3.3: the MLP's arithmetic
// intensity grows with the batch), and from about a hundred rows the matrix
// cores, not HBM, set the time.  Design for gfx950:
//   * a workgroup computes a BM x 256 tile of y (BM = 64 WM rows) with WM x WN
//     wavefronts, each owning 64 rows x RB weight row blocks (BF16 / FP8: 4
//     row blocks, 4 x 2 wavefronts; W4A16: 2 row blocks, 8 x 1 wavefronts,
//     whose group partials need a second set of accumulators):
//     v_mfma_f32_16x16x32_bf16 throughout;
//   * the packed 1 KiB weight tile is already the B-operand order (lane
//     16 kb + n: slice kb of weight row n), so weights go from memory straight
//     into registers and become exact bf16 B fragments there (FP8 codes by the
//     hardware conversion, W4A16 codes as 128 + q by OR-ing them into the
//     mantissa of 128.0, BF16 as is), each feeding 4 x row blocks.  The FP8
//     row scale is applied once at the end.  W4A16 follows the group's
//     definition of the dequantised weight, s (q - z): a chunk is one 128-k
//     group, its product P = sum x (128 + q) is formed in fresh accumulators,
//     and acc += s (P - (128 + z) X) with X the group's x sum, which a small
//     first kernel writes to the workspace ([group][row], float32) and the
//     kernel stages with the x tile;
//   * K advances in chunks (64 k; W4A16 128) through an NS-stage pipeline (3
//     for BF16, 4 for FP8, whose weights take half the registers, 2 for
//     W4A16, whose chunks are twice as long):
//     while chunk c is multiplied, the weights (and W4A16 scales, zero points
//     and x sums) and x of chunks up to c + NS - 1 are in flight and the x of
//     chunk c + 1 is written into its LDS buffer (one barrier per chunk).  The
//     loop body is NS chunks, so every index is a compile-time constant.  x
//     sits in LDS in fragment order: fragment (tile, x row block i, K-step s)
//     is 1 KiB, lane 16 kb + j holding the 8 k of row 16 i + j that pair with
//     slice kb of the weights; reads are conflict-free 16-byte LDS reads, all
//     of a chunk's issued before its first multiply;
//   * weights are read with the default cache policy: every x row block of a
//     column block re-reads them, and XCD-aware order keeps them in one L2:
//     consecutive workgroups of one XCD (dispatch is round-robin over the 8
//     XCDs) take the row blocks of x of one column block;
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
  float* part;        // split partials [S][M][N] (S > 1)
  const float* xsum;  // W4A16: x sums [KT][Mp]
  const uint4* w;
  const void* scales;
  const uint16_t* zeros;
  int64_t M, N, K, KT, G4, NB, Mp;
  int NBN, MB;  // 256-column blocks, BM-row blocks
  int nchunks;  // chunks of K
  int cps;      // chunks per split
  int S;
};

template <int FMT>
struct GmF {
  static constexpr bool W4 = FMT == kFmtW4;
  static constexpr int TK = FMT == kFmtBF16 ? 32 : FMT == kFmtFP8 ? 64 : 128;  // K per tile
  static constexpr int SLK = TK / 4;                                           // K per slice
  static constexpr int STEPS = SLK / 8;                                        // 32-k steps per tile
  static constexpr int KC = W4 ? 128 : 64;                                     // K per chunk
  static constexpr int TPC = KC / TK;                                          // tiles per chunk
  static constexpr int NQ = TPC * STEPS;                                       // 32-k steps per chunk
  static constexpr int MF = 4;                                                 // x row blocks per wavefront
  static constexpr int RB = W4 ? 2 : 4;                                        // weight row blocks per wavefront
  static constexpr int WN = 16 / RB;                                           // wavefronts along N
  // pipeline stages: FP8 weights take half the registers of BF16, so one
  // more fits; W4A16 chunks are twice as long and its group partials need
  // the registers, so one fewer
  static constexpr int NS = FMT == kFmtFP8 ? 4 : FMT == kFmtW4 ? 2 : 3;
};

// Per (format, wavefront rows): BF16 and FP8 with two wavefront rows take
// 128-row wavefront tiles (8 x row blocks, 256 rows per workgroup; the
// accumulators then need the registers of further pipeline stages and of the
// second step's x fragments, which are read after the first step's
// multiplies).
template <int FMT, int WM>
struct GmT : GmF<FMT> {
  static constexpr bool WIDE = (FMT == kFmtBF16 || FMT == kFmtFP8) && WM == 2;
  static constexpr int MF = WIDE ? 8 : GmF<FMT>::MF;
  static constexpr int NS = WIDE ? 2 : GmF<FMT>::NS;
  static constexpr int NA = GmF<FMT>::W4 || WIDE ? 1 : GmF<FMT>::NQ;  // 32-k steps read before the multiplies
};

template <int FMT, int WM>
struct GmL {
  using F = GmT<FMT, WM>;
  static constexpr int XB = F::MF * WM;                 // x row blocks per workgroup
  static constexpr int FRAGS = F::TPC * XB * F::STEPS;  // 1 KiB fragments per chunk
  static constexpr int XS = F::W4 ? 4 * XB : 0;         // uint4 of group x sums per chunk (16 rows per block)
  static constexpr int BUF = FRAGS * 64 + XS;           // uint4 per LDS buffer
  static constexpr int NW = WM * F::WN;                 // wavefronts per workgroup
  static constexpr int XPW = FRAGS / NW;                // fragments each wavefront stages
  static_assert(XPW * NW == FRAGS, "whole fragments per wavefront");
  static_assert(XS <= 64, "one wavefront stages the x sums");
};

template <int FMT, int WM>
struct GmState {
  using F = GmT<FMT, WM>;
  uint4 w[F::NS][F::RB][F::TPC];         // weights of chunks c .. c + NS - 1
  uint4 xr[F::NS][GmL<FMT, WM>::XPW];    // x fragments loaded NS - 1 chunks ahead
  uint4 xsr[F::NS];                      // W4A16: x sums (lanes below XS)
  uint32_t sc16[F::NS][F::RB];           // W4A16: fp16 scale bits of this lane's column
  uint32_t zq16[F::NS][F::RB];           // W4A16: the 4 zero nibbles of its scale quad
  gm_f32x4_t acc[F::MF][F::RB];
  __amdgpu_buffer_rsrc_t wres[F::RB], xres, sres[F::W4 ? F::RB : 1], zres[F::W4 ? F::RB : 1], xsres;
  uint32_t xvo[GmL<FMT, WM>::XPW];  // W4A16: this lane's x byte offsets (chunk 0 of the matrix)
  uint32_t xsvo;                    // W4A16: this lane's x-sum byte offset (group 0)
  int64_t kt0, m0, nb0;
  int lane, wave, wm, nch;
};

// Weights of chunk c of the split into set H (chunks past the split read
// zeros).
template <int FMT, int WM, int H>
__device__ __forceinline__ void gm_load_w(GmState<FMT, WM>& st, const GmArgs& a, int c) {
  using F = GmT<FMT, WM>;
#pragma unroll
  for (int b = 0; b < F::RB; ++b)
#pragma unroll
    for (int t = 0; t < F::TPC; ++t) {
      // default cache policy: every x row block of the column block (and each
      // of its wavefront rows) reads these bytes, so they must stay in L2
      // (streaming them non-temporally cost 5-20% on the 70B verify shapes)
      const u32x4_t v =
          __builtin_amdgcn_raw_buffer_load_b128(st.wres[b], st.lane * 16, (c * F::TPC + t) * kTileBytes, 0);
      st.w[H][b][t] = make_uint4(v.x, v.y, v.z, v.w);
    }
}

// W4A16: scales and zero words of chunk c (one group) into set H, requested
// one chunk ahead (before that chunk's x and weights, so waiting for them
// does not wait for those): the row block's scales [quad][row][4] and zero
// words [quad][row], the lane's row in the vector offset, the group in the
// scalar one (past the split: beyond the resource, so 0).
template <int FMT, int WM, int H>
__device__ __forceinline__ void gm_load_sz(GmState<FMT, WM>& st, int c) {
  if constexpr (GmF<FMT>::W4) {
    const int g = int(st.kt0) + c;
    const bool ok = c < st.nch;
    const uint32_t so = ok ? uint32_t(((g / kScaleQuad) * kTileRows * kScaleQuad + g % kScaleQuad) * 2) : 0x40000000u;
    const uint32_t zo = ok ? uint32_t((g / kScaleQuad) * kTileRows * 2) : 0x40000000u;
    const int n = st.lane & 15;
#pragma unroll
    for (int b = 0; b < GmF<FMT>::RB; ++b) {
      // kept apart until the group is multiplied: combining them here would
      // wait for the loads
      st.sc16[H][b] = __builtin_amdgcn_raw_buffer_load_b16(st.sres[b], n * kScaleQuad * 2, so, 0);
      st.zq16[H][b] = __builtin_amdgcn_raw_buffer_load_b16(st.zres[b], n * 2, zo, 0);
    }
  }
}

// x fragments this wavefront stages for chunk c into set H: fragment
// f = wave * XPW + u of (tile t, x row block i, step s) order; W4A16: the
// group's x sums of the workgroup's rows too (each wavefront loads them, the
// first one stores them).
template <int FMT, int WM, int H>
__device__ __forceinline__ void gm_load_x(GmState<FMT, WM>& st, const GmArgs& a, int c) {
  using F = GmT<FMT, WM>;
  using L = GmL<FMT, WM>;
  if constexpr (F::W4) {
    // K is a whole number of groups, so a chunk is either inside x or past it
    const int64_t g = st.kt0 + c;
    const uint32_t so = g < a.KT ? uint32_t(g * kGroup * 2) : 0x7FFFFFF0u;
#pragma unroll
    for (int u = 0; u < L::XPW; ++u) {
      const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(st.xres, st.xvo[u], so, 0);
      st.xr[H][u] = make_uint4(v.x, v.y, v.z, v.w);
    }
    const uint32_t sso = g < a.KT ? uint32_t(g * a.Mp * 4) : 0x7FFFFFF0u;
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(st.xsres, st.xsvo, sso, 0);
    st.xsr[H] = make_uint4(v.x, v.y, v.z, v.w);
    return;
  }
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
  if constexpr (GmF<FMT>::W4) {
    if (st.wave == 0 && st.lane < L::XS) buf[L::FRAGS * 64 + st.lane] = st.xsr[H];
  }
}

// x fragments of the chunk in buf that this wavefront multiplies: 32-k step
// q, x row block i (W4A16: step 0; the rest, and the x sums of rows
// 4 kb .. 4 kb + 3 of each block, are read as they are needed).
template <int FMT, int WM>
struct GmFrag {
  static constexpr int NA = GmT<FMT, WM>::NA;
  uint4 a[NA][GmT<FMT, WM>::MF];
  uint4 xs[GmF<FMT>::W4 ? GmT<FMT, WM>::MF : 1];
};

template <int FMT, int WM>
__device__ __forceinline__ void gm_read_x(const GmState<FMT, WM>& st, const uint4* buf, GmFrag<FMT, WM>& f) {
  using F = GmT<FMT, WM>;
  using L = GmL<FMT, WM>;
  const uint4* xf = buf + st.lane;
#pragma unroll
  for (int q = 0; q < GmFrag<FMT, WM>::NA; ++q)
#pragma unroll
    for (int i = 0; i < F::MF; ++i) {
      const int t = q / F::STEPS, s = q % F::STEPS;
      f.a[q][i] = xf[((t * L::XB + st.wm * F::MF + i) * F::STEPS + s) * 64];
    }
}

// Multiply the x fragments with the weights of set H (chunk c).
template <int FMT, int WM, int H>
__device__ __forceinline__ void gm_compute(GmState<FMT, WM>& st, GmFrag<FMT, WM>& f, const uint4* buf, int c) {
  using F = GmT<FMT, WM>;
  if constexpr (FMT == kFmtW4) {
    using L = GmL<FMT, WM>;
    const uint32_t mask = vgpr_const(0x000F000Fu), magic = vgpr_const(0x43004300u);
    gm_f32x4_t P[F::MF][F::RB];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      // steps 1 to 3: their fragments replace those of the step before once
      // it has been multiplied (16 fragments would not fit in registers)
      if (s > 0) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < F::MF; ++i) f.a[0][i] = buf[((st.wm * F::MF + i) * F::STEPS + s) * 64 + st.lane];
      }
      uint4 bm[F::RB];
#pragma unroll
      for (int b = 0; b < F::RB; ++b) {
        const uint4 wv = st.w[H][b][0];
        const uint32_t wd = s == 0 ? wv.x : s == 1 ? wv.y : s == 2 ? wv.z : wv.w;
        bm[b] = make_uint4(and_or_v(wd, mask, magic), and_or_v(wd >> 4, mask, magic), and_or_v(wd >> 8, mask, magic),
                           and_or_v(wd >> 12, mask, magic));
      }
#pragma unroll
      for (int i = 0; i < F::MF; ++i)
#pragma unroll
        for (int b = 0; b < F::RB; ++b)
          P[i][b] = gm_mfma(f.a[0][i], bm[b], s == 0 ? gm_f32x4_t{0.f, 0.f, 0.f, 0.f} : P[i][b]);
    }
    // acc += s (P - (128 + z) X): the group's zero point is nibble g % 4 of
    // the quad's zero word; the x sums are read only now (held through the
    // multiplies they would not leave room for the accumulators)
    __builtin_amdgcn_sched_barrier(0);
    const int kb = st.lane >> 4;
#pragma unroll
    for (int i = 0; i < F::MF; ++i) f.xs[i] = buf[L::FRAGS * 64 + (st.wm * F::MF + i) * 4 + kb];
    const int zsh = 4 * int((st.kt0 + c) % kScaleQuad);
#pragma unroll
    for (int b = 0; b < F::RB; ++b) {
      const float sc = __half2float(__ushort_as_half(uint16_t(st.sc16[H][b])));
      const float zc = 128.0f + float((st.zq16[H][b] >> zsh) & 0xFu);
#pragma unroll
      for (int i = 0; i < F::MF; ++i) {
        const gm_f32x4_t X = __builtin_bit_cast(gm_f32x4_t, f.xs[i]);
#pragma unroll
        for (int r = 0; r < 4; ++r) st.acc[i][b][r] = fmaf(sc, fmaf(-zc, X[r], P[i][b][r]), st.acc[i][b][r]);
      }
    }
  } else if constexpr (FMT == kFmtFP8) {
    using L = GmL<FMT, WM>;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (s >= F::NA) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < F::MF; ++i) f.a[s % F::NA][i] = buf[((st.wm * F::MF + i) * F::STEPS + s) * 64 + st.lane];
      }
      uint4 bm[F::RB];
#pragma unroll
      for (int b = 0; b < F::RB; ++b) {
        const uint4 wv = st.w[H][b][0];
        const uint32_t w0 = s == 0 ? wv.x : wv.z, w1 = s == 0 ? wv.y : wv.w;
        bm[b] = make_uint4(__builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<false>(w0)),
                           __builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<true>(w0)),
                           __builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<false>(w1)),
                           __builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<true>(w1)));
      }
#pragma unroll
      for (int i = 0; i < F::MF; ++i)
#pragma unroll
        for (int b = 0; b < F::RB; ++b) st.acc[i][b] = gm_mfma(f.a[s % F::NA][i], bm[b], st.acc[i][b]);
    }
  } else {
    using L = GmL<FMT, WM>;
#pragma unroll
    for (int t = 0; t < F::TPC; ++t) {
      if (t >= F::NA) {
        // a later step's fragments replace the first step's once those are
        // multiplied
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < F::MF; ++i) f.a[t % F::NA][i] = buf[(t * L::XB + st.wm * F::MF + i) * 64 + st.lane];
      }
#pragma unroll
      for (int i = 0; i < F::MF; ++i)
#pragma unroll
        for (int b = 0; b < F::RB; ++b) st.acc[i][b] = gm_mfma(f.a[t % F::NA][i], st.w[H][b][t], st.acc[i][b]);
    }
  }
}

// Step for chunk c = NS it + H: read this wavefront's x fragments of chunk c
// from LDS, request chunk c + NS - 1 (x first: its wait comes first; the LDS
// reads land meanwhile), multiply chunk c, write the x of chunk c + 1 (loaded
// NS - 2 chunks ago) into its LDS buffer (that of chunk c + 1 - NS, released
// by the last barrier).  Loads and stores are unconditional: chunks past the
// split read zero weights (out of range of the weight resources), so no
// register of the ring is ever a merge of an old and a new value, which
// would make the compiler copy it (and wait for its load) at the loop's back
// edge.
template <int FMT, int WM, int H>
__device__ __forceinline__ void gm_step(GmState<FMT, WM>& st, const GmArgs& a, uint4 (*s_x)[GmL<FMT, WM>::BUF],
                                        int c) {
  constexpr int NS = GmT<FMT, WM>::NS;
  constexpr int H1 = (H + 1) % NS, HL = (H + NS - 1) % NS;
  GmFrag<FMT, WM> f;
  gm_read_x<FMT, WM>(st, s_x[H], f);
  __builtin_amdgcn_sched_barrier(0);
  gm_load_sz<FMT, WM, H1>(st, c + 1);
  gm_load_x<FMT, WM, HL>(st, a, c + NS - 1);
  gm_load_w<FMT, WM, HL>(st, a, c + NS - 1);
  __builtin_amdgcn_sched_barrier(0);
  gm_compute<FMT, WM, H>(st, f, s_x[H], c);
  gm_store_x<FMT, WM, H1>(st, s_x[H1]);
  __syncthreads();
}

template <int FMT, int WM>
__global__ __launch_bounds__(64 * WM * GmF<FMT>::WN) void gemm_kernel(GmArgs a) {
  using F = GmT<FMT, WM>;
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
  st.wm = st.wave / F::WN;
  const int wn = st.wave % F::WN;
  const int split = blockIdx.y;
  const int c0 = split * a.cps;
  const int nch = a.nchunks - c0 < a.cps ? a.nchunks - c0 : a.cps;  // >= 1: the planner sizes S so
  const int nchp = (nch + NS - 1) / NS * NS;  // padded: chunks past the split read zero weights
  st.nch = nch;
  st.kt0 = int64_t(c0) * F::TPC;
  st.m0 = int64_t(mb) * 16 * F::MF * WM;
  const int64_t tiles = a.KT - st.kt0 < int64_t(nch) * F::TPC ? a.KT - st.kt0 : int64_t(nch) * F::TPC;
  st.nb0 = int64_t(nbn) * 16 + wn * F::RB;
#pragma unroll
  for (int b = 0; b < F::RB; ++b) {
    // row blocks past the matrix and tiles past the split read zeros
    const bool live = st.nb0 + b < a.NB;
    const int64_t nb = live ? st.nb0 + b : 0;
    st.wres[b] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint4*>(a.w + (nb * a.KT + st.kt0) * (kTileBytes / 16)),
                                                   0, live ? uint32_t(tiles) * kTileBytes : 0u, 0x00020000);
#pragma unroll
    for (int i = 0; i < F::MF; ++i) st.acc[i][b] = gm_f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  st.xres = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.x), 0, 0x7FFFFFF0, 0x00020000);
  if constexpr (F::W4) {
    const int64_t qb = a.G4 * kTileRows;  // (scale quad, row) entries per row block
#pragma unroll
    for (int b = 0; b < F::RB; ++b) {
      const bool live = st.nb0 + b < a.NB;
      const int64_t nb = live ? st.nb0 + b : 0;
      st.sres[b] = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(reinterpret_cast<const uint16_t*>(a.scales) + nb * qb * kScaleQuad), 0,
          live ? uint32_t(qb * kScaleQuad * 2) : 0u, 0x00020000);
      st.zres[b] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.zeros + nb * qb), 0,
                                                     live ? uint32_t(qb * 2) : 0u, 0x00020000);
    }
    st.xsres = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(a.xsum), 0, uint32_t(a.KT * a.Mp * 4), 0x00020000);
    const int kb = st.lane >> 4, j = st.lane & 15;
#pragma unroll
    for (int u = 0; u < L::XPW; ++u) {
      // fragment f = wave * XPW + u of (x row block i, step s) order; rows
      // past M read zeros
      const int f = st.wave * L::XPW + u, i = f / F::STEPS, sx = f % F::STEPS;
      const int64_t row = st.m0 + 16 * i + j;
      st.xvo[u] = row < a.M ? uint32_t((row * a.K + int64_t(kb) * F::SLK + 8 * sx) * 2) : 0x7FFFFFF0u;
    }
    st.xsvo = st.lane < L::XS ? uint32_t((st.m0 + 4 * st.lane) * 4) : 0x7FFFFFF0u;
  }

  // prologue: chunks 0 .. NS - 2 requested, chunk 0 staged
  gm_load_sz<FMT, WM, 0>(st, 0);
  gm_load_x<FMT, WM, 0>(st, a, 0);
  gm_load_w<FMT, WM, 0>(st, a, 0);
  if constexpr (NS > 2) {
    gm_load_x<FMT, WM, 1>(st, a, 1);
    gm_load_w<FMT, WM, 1>(st, a, 1);
  }
  if constexpr (NS > 3) {
    gm_load_x<FMT, WM, 2>(st, a, 2);
    gm_load_w<FMT, WM, 2>(st, a, 2);
  }
  gm_store_x<FMT, WM, 0>(st, s_x[0]);
  __syncthreads();
  for (int c = 0; c < nchp; c += NS) {
    gm_step<FMT, WM, 0>(st, a, s_x, c);
    gm_step<FMT, WM, 1>(st, a, s_x, c + 1);
    if constexpr (NS > 2) gm_step<FMT, WM, 2 % NS>(st, a, s_x, c + 2);
    if constexpr (NS > 3) gm_step<FMT, WM, 3 % NS>(st, a, s_x, c + 3);
  }

  // lane (kb, n) holds rows 4 kb + r of each x row block, column n of each row block
  const int kb = st.lane >> 4, n = st.lane & 15;
#pragma unroll
  for (int b = 0; b < F::RB; ++b) {
    const int64_t col = (st.nb0 + b) * kTileRows + n;
    if (st.nb0 + b >= a.NB || col >= a.N) continue;
    const float cs = FMT == kFmtFP8 && a.S == 1 ? reinterpret_cast<const float*>(a.scales)[col] : 1.f;
#pragma unroll
    for (int i = 0; i < F::MF; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = st.m0 + (st.wm * F::MF + i) * 16 + 4 * kb + r;
        if (row >= a.M) continue;
        if (a.S > 1)
          a.part[(int64_t(split) * a.M + row) * a.N + col] = st.acc[i][b][r];
        else
          a.y[row * a.N + col] = uint16_t(f32_to_bf16_rne(st.acc[i][b][r] * cs));
      }
  }
}

// W4A16 x sums: xs[g][m] = the float32 sum of the 128 x of group g in row m
// (rows M .. Mp - 1: 0), in k order.
__global__ __launch_bounds__(256) void gm_xsum_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                      int64_t Mp, int64_t G, float* __restrict__ xs) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= G * Mp) return;
  const int64_t g = i / Mp, m = i % Mp;
  float s = 0.f;
  if (m < M) {
    const uint4* p = reinterpret_cast<const uint4*>(x + m * K + g * kGroup);
#pragma unroll 4
    for (int j = 0; j < kGroup / 8; ++j) {
      const uint4 v = p[j];
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s += bf16_bits_to_f32(u[e] & 0xFFFFu);
        s += bf16_bits_to_f32(u[e] >> 16);
      }
    }
  }
  xs[i] = s;
}

template <int FMT>
static hipError_t launch_gm_fmt(const GmArgs& a, const GmPlan& p, hipStream_t st) {
  constexpr int WN = GmF<FMT>::WN;
  const unsigned grid = unsigned(ceil_div(p.NBN, 8) * 8 * p.MB);
  if (p.wm == 2 && FMT != kFmtW4)
    hipLaunchKernelGGL((gemm_kernel<FMT, (FMT == kFmtW4 ? 1 : 2)>), dim3(grid, unsigned(p.S)), dim3(64 * 2 * WN), 0,
                       st, a);
  else if (p.wm == 1)
    hipLaunchKernelGGL((gemm_kernel<FMT, 1>), dim3(grid, unsigned(p.S)), dim3(64 * 1 * WN), 0, st, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_gemm(int fmt, const GmPlan& p, const void* x, int64_t M, int64_t N, int64_t K, const void* wp,
                       const void* scales, const void* zeros, void* y, void* ws, hipStream_t st) {
  GmArgs a;
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
  a.Mp = p.Mp;
  a.NBN = int(p.NBN);
  a.MB = int(p.MB);
  a.nchunks = int(p.nchunks);
  a.cps = int(p.cps);
  a.S = p.S;
  // workspace: [W4A16 x sums][split partials]
  a.xsum = reinterpret_cast<const float*>(ws);
  a.part = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + p.xs_bytes);
  hipError_t e;
  if (fmt == kFmtBF16) {
    e = launch_gm_fmt<kFmtBF16>(a, p, st);
  } else if (fmt == kFmtFP8) {
    e = launch_gm_fmt<kFmtFP8>(a, p, st);
  } else {
    if (p.wm != 1 || p.Mp < M || p.Mp % 64 != 0) return hipErrorInvalidValue;
    const int64_t n = p.KT * p.Mp;
    hipLaunchKernelGGL(gm_xsum_kernel, dim3(unsigned(ceil_div(n, int64_t(256)))), dim3(256), 0, st, a.x, M, K, p.Mp,
                       p.KT, reinterpret_cast<float*>(ws));
    e = hipGetLastError();
    if (e == hipSuccess) e = launch_gm_fmt<kFmtW4>(a, p, st);
  }
  if (e != hipSuccess || p.S == 1) return e;
  return launch_splitk_reduce(fmt, a.part, p.S, M, N, scales, y, st);
}

}  // namespace wqd
