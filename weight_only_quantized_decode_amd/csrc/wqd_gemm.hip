// Tiled matrix-core kernel for wide verify batches (many activation rows):
// y = x . dequant(W)^T as a dense contraction.
//
// With speculative verification the layer multiplies batch x (k + 1) rows
// ("Making each token cheaper", sections "Speculative decoding" and the lab
// on verify width; CS336 lecture 10 notes, 3.2-3.3: the MLP's arithmetic
// intensity grows with the batch), and from about a hundred rows the matrix
// cores, not HBM, set the time.  Design for gfx950:
//   * a workgroup computes a BM x 256 tile of y with WR x WN wavefronts, each
//     owning 16 MF rows x RB weight row blocks.  WM = 1: 64-row wavefront
//     tiles, BM = 64 (BF16 / FP8: 4 row blocks, 4 wavefronts; W4A16: 2 row
//     blocks, 8 wavefronts, whose group partials need a second set of
//     accumulators).  WM = 2: 128-row wavefront tiles, BM = 256 for BF16 /
//     FP8 (two wavefront rows, 8 wavefronts) and 128 for W4A16 (one row of 8);
//     v_mfma_f32_16x16x32_bf16 throughout;
//   * the packed 1 KiB weight tile is already the B-operand order (lane
//     16 kb + n: slice kb of weight row n), so weights go from memory straight
//     into registers and become exact bf16 B fragments there (FP8 codes by the
//     hardware conversion, W4A16 codes as 128 + q by OR-ing them into the
//     mantissa of 128.0, BF16 as is), each feeding MF x row blocks.  The FP8
//     row scale is applied once at the end.  W4A16 follows the group's
//     definition of the dequantised weight, s (q - z): a chunk is one 128-k
//     group, its product P = sum x (128 + q) is formed in fresh accumulators,
//     and acc += s (P - (128 + z) X) with X the group's x sum, which a small
//     first kernel writes to the workspace ([group][row], float32);
//   * x goes from memory straight into LDS (16-byte loads that write LDS
//     instead of registers), in fragment order: fragment (tile, x row block
//     i, K-step s) is 1 KiB, lane 16 kb + j holding the 8 k of row 16 i + j
//     that pair with slice kb of the weights, which is exactly the lane order
//     in which one such load writes LDS; reads are conflict-free 16-byte LDS
//     reads.  W4A16 scales, zero words and x sums take the same way into a
//     slot of each wavefront, so no register carries them across a chunk;
//   * K advances in chunks (64 k; W4A16 128) through an NS-stage pipeline: one
//     LDS buffer per stage, and while chunk c is multiplied the loads of
//     chunks up to c + NS - 1 are in flight.  Each step ends with an explicit
//     wait for this wavefront's x of chunk c + 1 (loads complete in issue
//     order, so the count of later loads is exact) and a bare barrier; a
//     barrier with a memory fence would make the compiler wait for every
//     pending load into LDS, including those of chunks c + 2 ...  Each stage
//     buffer is its own LDS array, which lets the compiler see that reading
//     one does not wait for loads into another.  The loop body is NS chunks,
//     so every index is a compile-time constant; the last nch % NS chunks
//     follow as steps that request nothing;
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
  int swiglu;   // packed gate/up pairs: store silu(gate) * up (store_out)
  // tail split (S2 > 0, S == 1): the column blocks from nbn1 run as S2 K
  // splits of cps2 chunks after the unsplit ones, their float32 partials to
  // tpart [S2][M][N - 256 nbn1]
  int nbn1, S2, cps2;
  float* tpart;
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
  // pipeline stages (measured: the kernel is bound by its multiply, dequant
  // and LDS issue, so one more stage changes the time by a few percent)
  static constexpr int NS = FMT == kFmtFP8 ? 4 : 3;
};

// Per (format, WM): WM = 2 takes 128-row wavefront tiles (8 x row blocks;
// BF16 and FP8 in two wavefront rows, 256 rows per workgroup, W4A16 in one,
// 128 rows).  Each weight fragment then feeds 8 x row blocks, which halves
// the weight traffic through the texture path (BF16 / FP8) and the
// dequantisation (W4A16) per multiply.  Two pipeline stages for BF16 and
// W4A16: the accumulators take the registers (and for W4A16 the 128-row x
// chunks the LDS) of the others.  FP8 weights take half the registers of
// BF16 ones, so FP8 keeps three stages (247 registers, 96 KiB of LDS;
// measured 0.7-1.8% faster than two on the 70B gate and down at 512 and
// 1024 rows).
template <int FMT, int WM>
struct GmT : GmF<FMT> {
  static constexpr bool WIDE = WM == 2;
  static constexpr int MF = WIDE ? 8 : GmF<FMT>::MF;
  static constexpr int WR = GmF<FMT>::W4 ? 1 : WM;  // wavefront rows
  static constexpr int NS = WIDE ? (FMT == kFmtFP8 ? 3 : 2) : GmF<FMT>::NS;
  static constexpr int NA = GmF<FMT>::W4 || WIDE ? 1 : GmF<FMT>::NQ;  // 32-k steps read before the multiplies
};

template <int FMT, int WM>
struct GmL {
  using F = GmT<FMT, WM>;
  static constexpr int XB = F::MF * F::WR;              // x row blocks per workgroup
  static constexpr int FRAGS = F::TPC * XB * F::STEPS;  // 1 KiB fragments per chunk
  static constexpr int NW = F::WR * F::WN;              // wavefronts per workgroup
  static constexpr int XPW = FRAGS / NW;                // fragments each wavefront stages
  // W4A16: each wavefront's slot after the fragments, 1 KiB per load (lanes
  // out of range may write zeros where their bytes would go): the group's x
  // sums of the workgroup's rows, the 128-byte scale quads of the wavefront's
  // row blocks, their 32-byte zero words
  static constexpr int SLOT = 192, SL_XS = 0, SL_S = 64, SL_Z = 128;  // uint4
  static constexpr int BUF = FRAGS * 64 + (F::W4 ? NW * SLOT : 0);  // uint4 per LDS buffer
  static_assert(XPW * NW == FRAGS, "whole fragments per wavefront");
  static_assert(!F::W4 || (4 * XB <= 64 && 8 * F::RB <= 64), "one load holds the x sums and the scale quads");
};

template <int FMT, int WM>
struct GmState {
  using F = GmT<FMT, WM>;
  uint4 w[F::NS][F::RB][F::TPC];  // weights of chunks c .. c + NS - 1
  gm_f32x4_t acc[F::MF][F::RB];
  __amdgpu_buffer_rsrc_t wres[F::RB], xres, sres, zres, xsres;
  uint32_t xvo[GmL<FMT, WM>::XPW];  // W4A16: this lane's x byte offsets (chunk 0 of the matrix)
  uint32_t xsvo;                    // W4A16: this lane's x-sum byte offset (group 0)
  uint32_t svo, zvo;                // W4A16: this lane's scale / zero-word byte offsets (quad 0)
  int64_t kt0, m0, nb0;
  int lane, wave, wm;
};

// 16 bytes per lane from r into LDS: lane i's bytes land at dst + 16 i.
__device__ __forceinline__ void gm_dma(__amdgpu_buffer_rsrc_t r, uint4* dst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, voff, soff, 0, 0);
}

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

// W4A16: the scale quads ([quad][row][4] fp16, 128 bytes per row block) and
// zero words ([quad][row], 32 bytes) holding chunk c's group, for this
// wavefront's row blocks, into its slot of buf; the quad goes in the scalar
// offset.  Chunks past the split are multiplied with scale 0 whatever lands.
template <int FMT, int WM>
__device__ __forceinline__ void gm_load_sz(GmState<FMT, WM>& st, int c, uint4* buf) {
  if constexpr (GmF<FMT>::W4) {
    using L = GmL<FMT, WM>;
    static_assert(kScaleQuad == 4, "four groups per scale quad");
    const uint32_t q = (uint32_t(st.kt0) + uint32_t(c)) >> 2;
    uint4* slot = buf + L::FRAGS * 64 + st.wave * L::SLOT;
    gm_dma(st.sres, slot + L::SL_S, st.svo, q * (kTileRows * kScaleQuad * 2));
    gm_dma(st.zres, slot + L::SL_Z, st.zvo, q * (kTileRows * 2));
  }
}

// x of chunk c into buf: this wavefront's fragments f = wave * XPW + u of
// (tile t, x row block i, step s) order (rows past M and k past K are out of
// range of the resource); W4A16: first the group's x sums into its slot.
template <int FMT, int WM>
__device__ __forceinline__ void gm_load_x(GmState<FMT, WM>& st, const GmArgs& a, int c, uint4* buf) {
  using F = GmT<FMT, WM>;
  using L = GmL<FMT, WM>;
  if constexpr (F::W4) {
    // K is a whole number of groups, so a chunk is either inside x or past it
    const int64_t g = st.kt0 + c;
    const uint32_t so = g < a.KT ? uint32_t(g * kGroup * 2) : 0x7FFFFFF0u;
    const uint32_t sso = g < a.KT ? uint32_t(g * a.Mp * 4) : 0x7FFFFFF0u;
    gm_dma(st.xsres, buf + L::FRAGS * 64 + st.wave * L::SLOT + L::SL_XS, st.xsvo, sso);
#pragma unroll
    for (int u = 0; u < L::XPW; ++u) gm_dma(st.xres, buf + (st.wave * L::XPW + u) * 64, st.xvo[u], so);
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
    gm_dma(st.xres, buf + f * 64, off, 0);
  }
}

// All loads of chunk c, in a fixed order that the wait below counts on: W4A16
// scale quads, zero words and x sums, then x, then weights.
template <int FMT, int WM, int H>
__device__ __forceinline__ void gm_load_group(GmState<FMT, WM>& st, const GmArgs& a, int c, uint4* buf) {
  gm_load_sz<FMT, WM>(st, c, buf);
  gm_load_x<FMT, WM>(st, a, c, buf);
  __builtin_amdgcn_sched_barrier(0);
  gm_load_w<FMT, WM, H>(st, a, c);
}

// End of a step that requested nothing: wait for everything in flight.
__device__ __forceinline__ void gm_wait_all() {
  __builtin_amdgcn_s_waitcnt(0x7 << 4);  // vmcnt(0) lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// End of a step: wait until this wavefront's loads into LDS for chunk c + 1
// (requested NS - 2 steps ago) have landed and its LDS reads of chunk c are
// done, then meet the other wavefronts.  Loads complete in issue order; after
// chunk c + 1's x this wavefront has issued that chunk's weights and, in each
// later step, a whole group (W4A16 scale quads, zero words and x sums, then
// x, then weights).  The barrier carries no memory fence: with one the
// compiler would also wait for the loads of chunks c + 2 ... into LDS.
template <int FMT, int WM>
__device__ __forceinline__ void gm_wait_step() {
  using F = GmT<FMT, WM>;
  using L = GmL<FMT, WM>;
  constexpr int RBT = F::RB * F::TPC, SZ = F::W4 ? 3 : 0;
  constexpr int N = RBT + (F::NS - 2) * (SZ + L::XPW + RBT);
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | ((N >> 4) << 14));  // vmcnt(N) lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
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
    // acc += s (P - (128 + z) X): the group is entry g % 4 of the scale quad
    // and nibble g % 4 of the zero word; the x sums are read only now (held
    // through the multiplies they would not leave room for the accumulators)
    __builtin_amdgcn_sched_barrier(0);
    const int kb = st.lane >> 4;
#pragma unroll
    for (int i = 0; i < F::MF; ++i) f.xs[i] = buf[L::FRAGS * 64 + st.wave * L::SLOT + L::SL_XS + (st.wm * F::MF + i) * 4 + kb];
    const int zsh = 4 * int((uint32_t(st.kt0) + uint32_t(c)) & 3u);
    // this lane's row n in each row block: its 4 scales (8 bytes) and its
    // zero word (half of a dword), read one at a time: the compiler merges
    // adjacent reads into one that no longer shows which LDS array it reads,
    // and then waits for every load into LDS in flight
    const int n = st.lane & 15;
    uint2 sqv[F::RB];
    uint32_t zwv[F::RB];
#pragma unroll
    for (int b = 0; b < F::RB; ++b) {
      sqv[b] = reinterpret_cast<const uint2*>(buf + L::FRAGS * 64 + st.wave * L::SLOT + L::SL_S)[b * 16 + n];
      __builtin_amdgcn_sched_barrier(0);
      zwv[b] = reinterpret_cast<const uint32_t*>(buf + L::FRAGS * 64 + st.wave * L::SLOT + L::SL_Z)[b * 8 + (n >> 1)];
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int b = 0; b < F::RB; ++b) {
      const uint2 sq = sqv[b];
      const uint32_t zw = zwv[b];
      const uint32_t sw = ((zsh & 8) ? sq.y : sq.x) >> (4 * (zsh & 4));
      const float sc = __half2float(__ushort_as_half(uint16_t(sw & 0xFFFFu)));
      const float zc = 128.0f + float(((zw >> (16 * (n & 1))) >> zsh) & 0xFu);
#pragma unroll
      for (int i = 0; i < F::MF; ++i) {
        const gm_f32x4_t X = __builtin_bit_cast(gm_f32x4_t, f.xs[i]);
#pragma unroll
        for (int r = 0; r < 4; ++r) st.acc[i][b][r] = fmaf(sc, fmaf(-zc, X[r], P[i][b][r]), st.acc[i][b][r]);
      }
    }
  } else if constexpr (FMT == kFmtFP8) {
    // 64-row tiles read both steps' fragments before the multiplies (NA = 2)
#pragma unroll
    for (int s = 0; s < 2; ++s) {
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
      for (int i = 0; i < F::MF; ++i) {
#pragma unroll
        for (int b = 0; b < F::RB; ++b) st.acc[i][b] = gm_mfma(f.a[s % F::NA][i], bm[b], st.acc[i][b]);
        // 128-row tiles: the second step's fragment i replaces the first's as
        // soon as its multiplies are issued, so the LDS reads overlap the rest
        if constexpr (F::NA == 1) {
          if (s == 0) f.a[0][i] = buf[((st.wm * F::MF + i) * F::STEPS + 1) * 64 + st.lane];
        }
      }
    }
  } else {
    using L = GmL<FMT, WM>;
    // 64-row tiles read both tiles' fragments before the multiplies (NA = 2)
#pragma unroll
    for (int t = 0; t < F::TPC; ++t) {
#pragma unroll
      for (int i = 0; i < F::MF; ++i) {
#pragma unroll
        for (int b = 0; b < F::RB; ++b) st.acc[i][b] = gm_mfma(f.a[t % F::NA][i], st.w[H][b][t], st.acc[i][b]);
        // 128-row tiles: the next tile's fragment i replaces this one as soon
        // as its multiplies are issued, so the LDS reads overlap the rest
        if constexpr (F::NA == 1) {
          if (t + 1 < F::TPC) f.a[0][i] = buf[((t + 1) * L::XB + st.wm * F::MF + i) * 64 + st.lane];
        }
      }
    }
  }
}

// Step for chunk c = NS it + H: read this wavefront's x fragments of chunk c
// from LDS, request chunk c + NS - 1 into the buffer of chunk c - 1 (released
// by the last barrier; the LDS reads land meanwhile), multiply chunk c, wait
// for chunk c + 1.  Every step issues the same loads in the same order, as
// the prologue does for its chunks, so the compiler's count of loads in
// flight is exact at every wait.  Loads are unconditional: chunks past the
// split read zero weights (out of range of the weight resources), so no
// register of the ring is ever a merge of an old and a new value, which
// would make the compiler copy it (and wait for its load) at the loop's back
// edge.  The steps after the loop (TAIL) request nothing: the compiler would
// drop their weight loads, whose values are never used, and the count of
// loads that the wait relies on would be wrong.
template <int FMT, int WM, int H, bool TAIL = false>
__device__ __forceinline__ void gm_step(GmState<FMT, WM>& st, const GmArgs& a, uint4* const* s_x, int c) {
  constexpr int NS = GmT<FMT, WM>::NS;
  constexpr int HL = (H + NS - 1) % NS;
  GmFrag<FMT, WM> f;
  gm_read_x<FMT, WM>(st, s_x[H], f);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (!TAIL) gm_load_group<FMT, WM, HL>(st, a, c + NS - 1, s_x[HL]);
  __builtin_amdgcn_sched_barrier(0);
  gm_compute<FMT, WM, H>(st, f, s_x[H], c);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (TAIL)
    gm_wait_all();
  else
    gm_wait_step<FMT, WM>();
}

template <int FMT, int WM>
__global__ __launch_bounds__((64 * GmT<FMT, WM>::WR * GmF<FMT>::WN)) void gemm_kernel(GmArgs a) {
  using F = GmT<FMT, WM>;
  using L = GmL<FMT, WM>;
  constexpr int NS = F::NS;
  // one LDS array per pipeline stage (see gm_wait_step)
  __shared__ uint4 s_x0[L::BUF], s_x1[L::BUF], s_x2[NS > 2 ? L::BUF : 1], s_x3[NS > 3 ? L::BUF : 1];
  uint4* const s_x[4] = {s_x0, s_x1, s_x2, s_x3};

  // XCD-aware order: the workgroups of one XCD sweep the row blocks of x of
  // one column block back to back.  With a tail split the workgroups past
  // the unsplit column blocks' take the tail's (column block, row block,
  // split) in the same order.
  const int Lb = blockIdx.x, g1 = a.nbn1 * a.MB;
  const bool tail = a.S2 > 0 && Lb >= g1;
  const int Lt = tail ? Lb - g1 : Lb, xcd = Lt & 7, wi = Lt >> 3;
  const int per = tail ? a.MB * a.S2 : a.MB;  // workgroups per column block
  const int nbn = (tail ? a.nbn1 : 0) + (wi / per) * 8 + xcd, mb = (wi % per) % a.MB;
  if (nbn >= a.NBN) return;  // whole workgroup, before any barrier

  GmState<FMT, WM> st;
  st.lane = threadIdx.x & 63;
  st.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  st.wm = st.wave / F::WN;
  const int wn = st.wave % F::WN;
  const int split = tail ? (wi % per) / a.MB : int(blockIdx.y);
  const int cps = tail ? a.cps2 : a.cps;
  const int c0 = split * cps;
  const int nch = a.nchunks - c0 < cps ? a.nchunks - c0 : cps;  // >= 1: the planner sizes the splits so
  st.kt0 = int64_t(c0) * F::TPC;
  st.m0 = int64_t(mb) * 16 * F::MF * F::WR;
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
    // lanes 0-15: the 128-byte scale quads of this wavefront's two row
    // blocks (8 lanes each); lanes 0-3: their 32-byte zero words (2 each);
    // row blocks past the matrix are out of range
    st.sres = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.scales), 0, uint32_t(a.NB * qb * kScaleQuad * 2),
                                                0x00020000);
    st.zres = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.zeros), 0, uint32_t(a.NB * qb * 2), 0x00020000);
    {
      const int64_t nbs = st.nb0 + (st.lane >> 3), nbz = st.nb0 + (st.lane >> 1);
      st.svo = st.lane < 8 * F::RB && nbs < a.NB ? uint32_t(nbs * qb * kScaleQuad * 2 + (st.lane & 7) * 16) : 0x7FFFFFF0u;
      st.zvo = st.lane < 2 * F::RB && nbz < a.NB ? uint32_t(nbz * qb * 2 + (st.lane & 1) * 16) : 0x7FFFFFF0u;
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
    st.xsvo = st.lane < 4 * L::XB ? uint32_t((st.m0 + 4 * st.lane) * 4) : 0x7FFFFFF0u;
  }

  // prologue: chunks 0 .. NS - 2 requested, chunk 0 in LDS
  {
    // the buffers start as zeros: lanes out of range of their resource may
    // leave their LDS bytes unwritten (those bytes then only ever hold zeros
    // or earlier values of the same rows, never NaN)
#pragma unroll
    for (int h = 0; h < NS; ++h)
      for (int i = threadIdx.x; i < L::BUF; i += 64 * L::NW) s_x[h][i] = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();
  }
  gm_load_group<FMT, WM, 0>(st, a, 0, s_x[0]);
  if constexpr (NS > 2) gm_load_group<FMT, WM, 1>(st, a, 1, s_x[1]);
  if constexpr (NS > 3) gm_load_group<FMT, WM, 2>(st, a, 2, s_x[2]);
  __syncthreads();
  int c = 0;
  for (; c + NS <= nch; c += NS) {
    gm_step<FMT, WM, 0>(st, a, s_x, c);
    gm_step<FMT, WM, 1>(st, a, s_x, c + 1);
    if constexpr (NS > 2) gm_step<FMT, WM, 2 % NS>(st, a, s_x, c + 2);
    if constexpr (NS > 3) gm_step<FMT, WM, 3 % NS>(st, a, s_x, c + 3);
  }
  // the last nch % NS chunks, already requested
  const int rest = nch - c;
  if (rest > 0) gm_step<FMT, WM, 0, true>(st, a, s_x, c);
  if constexpr (NS > 2) {
    if (rest > 1) gm_step<FMT, WM, 1, true>(st, a, s_x, c + 1);
  }
  if constexpr (NS > 3) {
    if (rest > 2) gm_step<FMT, WM, 2, true>(st, a, s_x, c + 2);
  }

  // lane (kb, n) holds rows 4 kb + r of each x row block, column n of each row block
  const int kb = st.lane >> 4, n = st.lane & 15;
#pragma unroll
  for (int b = 0; b < F::RB; ++b) {
    const int64_t col = (st.nb0 + b) * kTileRows + n;
    if (st.nb0 + b >= a.NB || col >= a.N) continue;
    const float cs = FMT == kFmtFP8 && a.S == 1 && !tail ? reinterpret_cast<const float*>(a.scales)[col] : 1.f;
    const int64_t nt = a.N - int64_t(a.nbn1) * 256, ct = col - int64_t(a.nbn1) * 256;  // tail: width, column
#pragma unroll
    for (int i = 0; i < F::MF; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = st.m0 + (st.wm * F::MF + i) * 16 + 4 * kb + r;
        if (row >= a.M) continue;  // the same for lanes n and n ^ 8
        if (tail)
          a.tpart[(int64_t(split) * a.M + row) * nt + ct] = st.acc[i][b][r];
        else if (a.S > 1)
          a.part[(int64_t(split) * a.M + row) * a.N + col] = st.acc[i][b][r];
        else
          store_out<8>(a.y, a.N, a.swiglu, row, col, st.acc[i][b][r] * cs, true);  // lane ^ 8: column ^ 8
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

// The tail split's sum: y[m][256 nbn1 + c] for the tail's nt columns, in
// split order (FP8: times the row scale).  Four consecutive outputs of a row
// per thread where nt % 4 == 0 (SwiGLU: columns c and c ^ 8 are then two
// threads apart, nt % 16 == 0), else one.
template <int FMT>
__global__ __launch_bounds__(256) void gm_tail_reduce_kernel(const float* __restrict__ tpart, int S2, int64_t M,
                                                             int64_t N, int64_t col0, const float* __restrict__ colscale,
                                                             uint16_t* __restrict__ y, int swiglu) {
  const int64_t nt = N - col0, MN = M * nt;
  const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if ((nt & 3) == 0) {
    const int64_t i0 = t * 4;
    if (i0 >= MN) return;  // SwiGLU: 4-thread groups (16 outputs) are all live or all not
    float4 a = *reinterpret_cast<const float4*>(tpart + i0);
    for (int s = 1; s < S2; ++s) {
      const float4 v = *reinterpret_cast<const float4*>(tpart + int64_t(s) * MN + i0);
      a.x += v.x;
      a.y += v.y;
      a.z += v.z;
      a.w += v.w;
    }
    const int64_t row = i0 / nt, c = i0 % nt;
    float f[4] = {a.x, a.y, a.z, a.w};
    if (FMT == kFmtFP8)
#pragma unroll
      for (int e = 0; e < 4; ++e) f[e] *= colscale[col0 + c + e];
    if (swiglu) {
#pragma unroll
      for (int e = 0; e < 4; ++e) store_out<2>(y, N, true, row, col0 + c + e, f[e], true);  // thread ^ 2: column ^ 8
      return;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) y[row * N + col0 + c + e] = uint16_t(f32_to_bf16_rne(f[e]));
    return;
  }
  if (t >= MN) return;  // (no SwiGLU here: it needs nt % 16 == 0)
  const int64_t row = t / nt, c = t % nt;
  float v = 0.f;
  for (int s = 0; s < S2; ++s) v += tpart[int64_t(s) * MN + t];
  if (FMT == kFmtFP8) v *= colscale[col0 + c];
  y[row * N + col0 + c] = uint16_t(f32_to_bf16_rne(v));
}

template <int FMT>
static hipError_t launch_gm_fmt(const GmArgs& a, const GmPlan& p, hipStream_t st) {
  constexpr int WN = GmF<FMT>::WN;
  const unsigned grid = unsigned(p.S2 > 0 ? p.nbn1 * p.MB + ceil_div(p.NBN - p.nbn1, int64_t(8)) * 8 * p.MB * p.S2
                                          : ceil_div(p.NBN, 8) * 8 * p.MB);
  if (p.wm == 2)
    hipLaunchKernelGGL((gemm_kernel<FMT, 2>), dim3(grid, unsigned(p.S)), dim3(64 * GmT<FMT, 2>::WR * WN), 0, st, a);
  else if (p.wm == 1)
    hipLaunchKernelGGL((gemm_kernel<FMT, 1>), dim3(grid, unsigned(p.S)), dim3(64 * GmT<FMT, 1>::WR * WN), 0, st, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_gemm(int fmt, const GmPlan& p, const void* x, int64_t M, int64_t N, int64_t K, const void* wp,
                       const void* scales, const void* zeros, void* y, void* ws, bool swiglu, hipStream_t st) {
  GmArgs a;
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
  a.Mp = p.Mp;
  a.NBN = int(p.NBN);
  a.MB = int(p.MB);
  a.nchunks = int(p.nchunks);
  a.cps = int(p.cps);
  a.S = p.S;
  a.nbn1 = int(p.nbn1);
  a.S2 = p.S2;
  a.cps2 = int(p.cps2);
  // workspace: [W4A16 x sums][split partials, or the tail split's]
  a.xsum = reinterpret_cast<const float*>(ws);
  a.part = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + p.xs_bytes);
  a.tpart = a.part;
  if (p.S2 > 0 && (p.S != 1 || p.nbn1 % 8 != 0 || p.nbn1 <= 0 || p.nbn1 >= p.NBN || p.S2 > 8))
    return hipErrorInvalidValue;
  hipError_t e;
  if (p.wm == 3) {
    e = launch_gemm_lds(fmt, p, x, M, N, K, wp, scales, y, a.part, swiglu, st);
  } else if (fmt == kFmtBF16) {
    e = launch_gm_fmt<kFmtBF16>(a, p, st);
  } else if (fmt == kFmtFP8) {
    e = launch_gm_fmt<kFmtFP8>(a, p, st);
  } else {
    if (p.Mp < M || p.Mp % (p.wm == 2 ? 128 : 64) != 0) return hipErrorInvalidValue;
    const int64_t n = p.KT * p.Mp;
    hipLaunchKernelGGL(gm_xsum_kernel, dim3(unsigned(ceil_div(n, int64_t(256)))), dim3(256), 0, st, a.x, M, K, p.Mp,
                       p.KT, reinterpret_cast<float*>(ws));
    e = hipGetLastError();
    if (e == hipSuccess) e = launch_gm_fmt<kFmtW4>(a, p, st);
  }
  if (e != hipSuccess) return e;
  if (p.S2 > 0) {
    const int64_t col0 = p.nbn1 * 256, n = M * (N - col0);
    const dim3 g(unsigned(ceil_div((N - col0) % 4 == 0 ? n / 4 : n, int64_t(256))));
    const float* cs = reinterpret_cast<const float*>(scales);
    uint16_t* yo = reinterpret_cast<uint16_t*>(y);
    if (fmt == kFmtFP8)
      hipLaunchKernelGGL(gm_tail_reduce_kernel<kFmtFP8>, g, dim3(256), 0, st, a.tpart, p.S2, M, N, col0, cs, yo,
                         int(swiglu));
    else
      hipLaunchKernelGGL(gm_tail_reduce_kernel<kFmtBF16>, g, dim3(256), 0, st, a.tpart, p.S2, M, N, col0, cs, yo,
                         int(swiglu));
    return hipGetLastError();
  }
  if (p.S == 1) return e;
  return launch_splitk_reduce(fmt, a.part, p.S, M, N, scales, y, swiglu, st);
}

}  // namespace wqd
