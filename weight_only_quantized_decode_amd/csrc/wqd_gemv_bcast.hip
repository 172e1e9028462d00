// Streaming decode kernel for few activation rows (1-2 for W4A16, up to 8 for
// FP8 and BF16), x broadcast by DPP.
//
// Same work split as the LDS-staged streaming kernel (one workgroup per
// 16-row block over all of K, W wavefronts on contiguous shares of K, fixed
// order reductions), but x never goes through LDS.  In a packed tile, the 16
// lanes of one DPP row (kb fixed, n = 0..15) all multiply the same k-slice,
// and a slice holds at most 16 dwords of x (32 bf16).  So one 32-bit x
// register per tile covers the whole tile: lane (kb, j) holds dword j of
// slice kb, loaded straight from L2 as one coalesced 256-byte read per
// wavefront, and `row_newbcast:j` hands dword j to every lane of the row as
// the first operand of v_dot2c_f32_bf16.  The DPP row broadcast exists on
// gfx90a and later.
//
// Why: the weights are read once per step, so the bandwidth is set by bytes
// in flight per compute unit.  Without the staged x (registers for the
// staging, LDS reads per tile) a wavefront needs far fewer registers, more
// wavefronts fit per SIMD and every one keeps a whole group of tiles in
// flight; small matrices can also use up to 16 wavefronts per workgroup.
//
// W4A16 zero points: a tile contributes s * (P - (128 + z) * X) with
// P = sum x (128 + q) over a lane's slice and X = sum x over the same slice
// from an identical dot2 chain (so q == z == 0 cancels exactly).  X depends
// on (tile, slice) only: at the start each lane (kb, n) computes X for tiles
// n, 16 + n of its wavefront's share (at most 32 tiles), and the correction
// reads it back with the same row broadcast (v_fmac_f32 with DPP on X).
//
// DPP wait states.  The DPP instructions live in inline assembly, where the
// compiler's hazard tracking cannot see them, so each block keeps its own
// distances.  Measured on gfx950 (shorter distances gave wrong results,
// intermittently and with no error):
//  * a VALU write to a register read through DPP needs two wait states: every
//    block's first instructions do not write the broadcast register, or it
//    starts with s_nop 1;
//  * after a DPP v_dot2c / v_fmac, the next ordinary VALU instructions must
//    not touch its result or its operands at once (a read of the result one
//    wait state later missed the last products; a temporary rewritten two
//    instructions after its DPP read was read in its new state).  A DPP
//    successor accumulating into the same register may follow at once.  So
//    every block ends with s_nop: 1 after a word, 4 after a tile's last block.
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
};

template <int FMT>
struct BcC {
  static constexpr int TK = FMT == kFmtBF16 ? 32 : FMT == kFmtFP8 ? 64 : 128;  // K per tile
  static constexpr int SLK = TK / 4;                                             // K per slice
  static constexpr int DPS = SLK / 2;   // x dwords per slice: 16, 8, 4
  static constexpr int TPX = 16 / DPS;  // tiles per x register: 1, 2, 4
  static constexpr int GT = 4;          // tiles per group (a W4A16 scale quad)
  static constexpr int XR = GT / TPX;   // x registers per activation row and group
};

template <int FMT, int MR>
struct BGroup {
  uint4 w[4];
  uint32_t x[MR][BcC<FMT>::XR];
  uint2 s;     // W4A16: 4 fp16 scales of this lane's row, one per tile
  uint32_t z;  // W4A16: 4 zero nibbles
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
    const int tt = min(t0 + r * C::TPX + j / C::DPS, last);
    const int64_t k = (kt_begin + tt) * C::TK + kb * C::SLK + 2 * (j % C::DPS);
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      if (FMT == kFmtW4) {
        g.x[m][r] = *reinterpret_cast<const uint32_t*>(a.x + int64_t(m) * a.K + k);
      } else {
        const int64_t kc = k < a.K ? k : a.K - 2;
        const uint32_t v = *reinterpret_cast<const uint32_t*>(a.x + int64_t(m) * a.K + kc);
        g.x[m][r] = k < a.K ? v : 0u;
      }
    }
  }
  if (FMT == kFmtW4) {
    const int q = min(t0, last) / kScaleQuad;
    g.s = sbase[q * kTileRows];
    g.z = zbase[q * kTileRows];
  }
}

// ---- inline-assembly blocks (DPP operands) --------------------------------

// One packed W4A16 word (8 nibbles = 8 consecutive k of the slice) against x
// dwords B .. B + 3 of the row broadcast: P += sum x (128 + q).  The first
// broadcast read comes after seven VALU instructions that do not write x;
// the block ends with s_nop 1 before anything else may touch P or the
// temporaries.
template <int B>
__device__ __forceinline__ void w4_word(float& P, uint32_t w, uint32_t x, uint32_t mask, uint32_t magic) {
  uint32_t t0, t1, t2, t3;
  asm("v_lshrrev_b32 %[t1], 4, %[w]\n\t"
      "v_lshrrev_b32 %[t2], 8, %[w]\n\t"
      "v_lshrrev_b32 %[t3], 12, %[w]\n\t"
      "v_and_or_b32 %[t0], %[w], %[mk], %[mg]\n\t"
      "v_and_or_b32 %[t1], %[t1], %[mk], %[mg]\n\t"
      "v_and_or_b32 %[t2], %[t2], %[mk], %[mg]\n\t"
      "v_and_or_b32 %[t3], %[t3], %[mk], %[mg]\n\t"
      "v_dot2c_f32_bf16_dpp %[p], %[x], %[t0] row_newbcast:%[b0] row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %[p], %[x], %[t1] row_newbcast:%[b1] row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %[p], %[x], %[t2] row_newbcast:%[b2] row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %[p], %[x], %[t3] row_newbcast:%[b3] row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1"
      : [p] "+v"(P), [t0] "=&v"(t0), [t1] "=&v"(t1), [t2] "=&v"(t2), [t3] "=&v"(t3)
      : [w] "v"(w), [x] "v"(x), [mk] "v"(mask), [mg] "v"(magic), [b0] "n"(B), [b1] "n"(B + 1), [b2] "n"(B + 2),
        [b3] "n"(B + 3));
}

// The same for two activation rows sharing the dequantised word.
template <int B>
__device__ __forceinline__ void w4_word2(float& P0, float& P1, uint32_t w, uint32_t x0, uint32_t x1, uint32_t mask,
                                         uint32_t magic) {
  uint32_t t0, t1, t2, t3;
  asm("v_lshrrev_b32 %[t1], 4, %[w]\n\t"
      "v_lshrrev_b32 %[t2], 8, %[w]\n\t"
      "v_lshrrev_b32 %[t3], 12, %[w]\n\t"
      "v_and_or_b32 %[t0], %[w], %[mk], %[mg]\n\t"
      "v_and_or_b32 %[t1], %[t1], %[mk], %[mg]\n\t"
      "v_and_or_b32 %[t2], %[t2], %[mk], %[mg]\n\t"
      "v_and_or_b32 %[t3], %[t3], %[mk], %[mg]\n\t"
      "v_dot2c_f32_bf16_dpp %[p0], %[x0], %[t0] row_newbcast:%[b0] row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %[p1], %[x1], %[t0] row_newbcast:%[b0] row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %[p0], %[x0], %[t1] row_newbcast:%[b1] row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %[p1], %[x1], %[t1] row_newbcast:%[b1] row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %[p0], %[x0], %[t2] row_newbcast:%[b2] row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %[p1], %[x1], %[t2] row_newbcast:%[b2] row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %[p0], %[x0], %[t3] row_newbcast:%[b3] row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %[p1], %[x1], %[t3] row_newbcast:%[b3] row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1"
      : [p0] "+v"(P0), [p1] "+v"(P1), [t0] "=&v"(t0), [t1] "=&v"(t1), [t2] "=&v"(t2), [t3] "=&v"(t3)
      : [w] "v"(w), [x0] "v"(x0), [x1] "v"(x1), [mk] "v"(mask), [mg] "v"(magic), [b0] "n"(B), [b1] "n"(B + 1),
        [b2] "n"(B + 2), [b3] "n"(B + 3));
}

// P += X(broadcast from lane C of the row) * nz, where nz = -(128 + z).
template <int C>
__device__ __forceinline__ void fmac_bcast(float& P, float X, float nz) {
  asm("s_nop 1\n\t"
      "v_fmac_f32_dpp %[p], %[X], %[nz] row_newbcast:%[c] row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 4"
      : [p] "+v"(P)
      : [X] "v"(X), [nz] "v"(nz), [c] "n"(C));
}

// acc += sum over 8 dwords of x (broadcast from lanes B .. B + 7) * b[0..7].
template <int B>
__device__ __forceinline__ void dot8_bcast(float& acc, uint32_t x, const uint32_t (&b)[8]) {
  asm("s_nop 1\n\t"
      "v_dot2c_f32_bf16_dpp %[a], %[x], %[b0] row_newbcast:%[c0] row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %[a], %[x], %[b1] row_newbcast:%[c1] row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %[a], %[x], %[b2] row_newbcast:%[c2] row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %[a], %[x], %[b3] row_newbcast:%[c3] row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %[a], %[x], %[b4] row_newbcast:%[c4] row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %[a], %[x], %[b5] row_newbcast:%[c5] row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %[a], %[x], %[b6] row_newbcast:%[c6] row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %[a], %[x], %[b7] row_newbcast:%[c7] row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 4"
      : [a] "+v"(acc)
      : [x] "v"(x), [b0] "v"(b[0]), [b1] "v"(b[1]), [b2] "v"(b[2]), [b3] "v"(b[3]), [b4] "v"(b[4]),
        [b5] "v"(b[5]), [b6] "v"(b[6]), [b7] "v"(b[7]), [c0] "n"(B), [c1] "n"(B + 1), [c2] "n"(B + 2),
        [c3] "n"(B + 3), [c4] "n"(B + 4), [c5] "n"(B + 5), [c6] "n"(B + 6), [c7] "n"(B + 7));
}

// acc += sum over 4 dwords of x (broadcast from lanes B .. B + 3) * w[0..3].
template <int B>
__device__ __forceinline__ void dot4_bcast(float& acc, uint32_t x, uint4 w) {
  asm("s_nop 1\n\t"
      "v_dot2c_f32_bf16_dpp %[a], %[x], %[w0] row_newbcast:%[c0] row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %[a], %[x], %[w1] row_newbcast:%[c1] row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %[a], %[x], %[w2] row_newbcast:%[c2] row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_bf16_dpp %[a], %[x], %[w3] row_newbcast:%[c3] row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 4"
      : [a] "+v"(acc)
      : [x] "v"(x), [w0] "v"(w.x), [w1] "v"(w.y), [w2] "v"(w.z), [w3] "v"(w.w), [c0] "n"(B), [c1] "n"(B + 1),
        [c2] "n"(B + 2), [c3] "n"(B + 3));
}

// ---- per-tile arithmetic ---------------------------------------------------

// Tile I of a group; CI = its position in the wavefront's share (register
// CI / 16 of the W4A16 x sums holds it, in lane CI % 16 of each row).
template <int FMT, int MR, int XC, int I, int CI>
__device__ __forceinline__ void btile(const BGroup<FMT, MR>& g, const float (&X)[MR][XC], float (&acc)[MR]) {
  using C = BcC<FMT>;
  const uint4 wv = g.w[I];
  constexpr int R = I / C::TPX;               // x register of this tile
  constexpr int B = (I % C::TPX) * C::DPS;    // first broadcast lane of its dwords
  if constexpr (FMT == kFmtW4) {
    const uint32_t mask = 0x000F000Fu, magic = 0x43004300u;
    const uint32_t sw = (I < 2 ? g.s.x : g.s.y) >> (16 * (I & 1));
    const float s = __half2float(__ushort_as_half(uint16_t(sw & 0xFFFFu)));
    const float nz = -(128.0f + float((g.z >> (4 * I)) & 0xFu));
    float P[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) P[m] = 0.f;
    if constexpr (MR == 1) {
      w4_word<0>(P[0], wv.x, g.x[0][R], mask, magic);
      w4_word<4>(P[0], wv.y, g.x[0][R], mask, magic);
      w4_word<8>(P[0], wv.z, g.x[0][R], mask, magic);
      w4_word<12>(P[0], wv.w, g.x[0][R], mask, magic);
    } else {
      w4_word2<0>(P[0], P[1], wv.x, g.x[0][R], g.x[1][R], mask, magic);
      w4_word2<4>(P[0], P[1], wv.y, g.x[0][R], g.x[1][R], mask, magic);
      w4_word2<8>(P[0], P[1], wv.z, g.x[0][R], g.x[1][R], mask, magic);
      w4_word2<12>(P[0], P[1], wv.w, g.x[0][R], g.x[1][R], mask, magic);
    }
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      fmac_bcast<CI % 16>(P[m], X[m][CI / 16], nz);
      acc[m] = fmaf(s, P[m], acc[m]);
    }
  } else if constexpr (FMT == kFmtFP8) {
    uint32_t b[8];
    const uint32_t wd[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      b[2 * q] = __builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<false>(wd[q]));
      b[2 * q + 1] = __builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<true>(wd[q]));
    }
#pragma unroll
    for (int m = 0; m < MR; ++m) dot8_bcast<B>(acc[m], g.x[m][R], b);
  } else {
#pragma unroll
    for (int m = 0; m < MR; ++m) dot4_bcast<B>(acc[m], g.x[m][R], wv);
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

// The x sums of one register (16 tiles): the dot2 chain of x against ones,
// in the order of the products' chain.
template <int FMT, int MR, int XC>
__device__ __forceinline__ void xsums(float (&X)[MR][XC], const uint4 (&xs)[MR][4], int c) {
  const bf16x2_t ones = as_bf16x2(0x3F803F80u);
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    float v = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      v = dot2_bf16(as_bf16x2(xs[m][u].x), ones, v);
      v = dot2_bf16(as_bf16x2(xs[m][u].y), ones, v);
      v = dot2_bf16(as_bf16x2(xs[m][u].z), ones, v);
      v = dot2_bf16(as_bf16x2(xs[m][u].w), ones, v);
    }
    X[m][c] = v;
  }
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
    if (row < a.N) {
      if (FMT == kFmtFP8) v *= reinterpret_cast<const float*>(a.scales)[row];
      a.y[int64_t(m) * a.N + row] = uint16_t(f32_to_bf16_rne(v));
    }
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
                             const void* wp, const void* scales, const void* zeros, void* y, hipStream_t st) {
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
  const unsigned grid = unsigned(p.NB);
  const int mr = int(M);
  if (fmt == kFmtBF16) return launch_bc_fmt<kFmtBF16>(a, mr, p.waves, p.groups, grid, st);
  if (fmt == kFmtFP8) return launch_bc_fmt<kFmtFP8>(a, mr, p.waves, p.groups, grid, st);
  return launch_bc_fmt<kFmtW4>(a, mr, p.waves, p.groups, grid, st);
}

}  // namespace wqd
