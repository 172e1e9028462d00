// Streaming decode kernel for few activation rows (1-2 for W4A16, up to 8 for
// FP8 and BF16), x broadcast by DPP.
//
// Same work split as the LDS-staged streaming kernel (one workgroup per
// 16-row block over all of K, W wavefronts on contiguous shares of K, fixed
// order reductions), but x never goes through LDS.  In a packed tile, the 16
// lanes of one DPP row (kb fixed, n = 0..15) all multiply the same k-slice,
// and a slice holds at most 16 dwords of x (32 bf16).  So one x register per
// one to four tiles covers them: for W4A16 and FP8 a 64-bit register, lane
// (kb, j) holding dwords 2j, 2j + 1 of a slice (8 lanes per W4A16 slice, 4
// per FP8 slice), for BF16 a 32-bit one (dword j, 4 lanes per slice), loaded
// straight from L2 as one coalesced read per wavefront.  A DPP row broadcast
// (row_newbcast:j, gfx90a and later) hands lane j's value to every lane of
// the row, where it feeds v_dot2c_f32_bf16.
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
// DPP.  The row broadcast is a compiler builtin (a v_mov_b32 with the
// row_newbcast control) feeding ordinary dot2 / fma builtins, so the
// compiler's hazard recognizer inserts the wait states around it: gfx950 has
// no folded DPP form of v_dot2c_f32_bf16 that the compiler would form, so
// each broadcast dword costs one move.
#include <type_traits>

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

template <int FMT>
struct BcC {
  static constexpr int TK = FMT == kFmtBF16 ? 32 : FMT == kFmtFP8 ? 64 : 128;  // K per tile
  static constexpr int SLK = TK / 4;                                             // K per slice
  static constexpr int DPS = SLK / 2;   // x dwords per slice: 16, 8, 4
  // x register width in dwords: W4A16 and FP8 broadcast two dwords per move
  // (v_mov_b64 with row_newbcast), BF16 one
  static constexpr int XW = FMT == kFmtBF16 ? 1 : 2;
  static constexpr int LPS = DPS / XW;  // lanes of a row holding one slice: 8, 4, 4
  static constexpr int TPX = 16 / LPS;  // tiles per x register: 2, 4, 4
  static constexpr int GT = 4;          // tiles per group (a W4A16 scale quad)
  static constexpr int XR = GT / TPX;   // x registers per activation row and group: 2, 1, 1
};

template <int FMT>
using XReg = typename std::conditional<BcC<FMT>::XW == 2, uint64_t, uint32_t>::type;

template <int FMT, int MR>
struct BGroup {
  uint4 w[4];
  XReg<FMT> x[MR][BcC<FMT>::XR];
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

// ---- row broadcast (DPP) --------------------------------------------------

// Dword J of `x` as held by lane J of each 16-lane row, handed to every lane of
// that row (row_newbcast:J, DPP control 0x150 + J on gfx90a and later).  Plain
// builtins, so the compiler sees the data movement and places the wait states
// the hardware needs around it (a VALU write before the DPP read of its
// result; a VALU read after a dot product's write).
template <int J>
__device__ __forceinline__ uint32_t row_bcast(uint32_t x) {
  static_assert(J >= 0 && J < 16, "a row has 16 lanes");
  return uint32_t(__builtin_amdgcn_mov_dpp(int(x), 0x150 + J, 0xF, 0xF, false));
}

// Dwords 2J and 2J + 1 of a row's x (held by lane J) to every lane of the row:
// one v_mov_b64 with row_newbcast:J.
template <int J>
__device__ __forceinline__ uint64_t row_bcast64(uint64_t x) {
  static_assert(J >= 0 && J < 16, "a row has 16 lanes");
  return __builtin_amdgcn_mov_dpp(x, 0x150 + J, 0xF, 0xF, false);
}

__device__ __forceinline__ uint32_t lo32(uint64_t v) { return uint32_t(v); }
__device__ __forceinline__ uint32_t hi32(uint64_t v) { return uint32_t(v >> 32); }

template <int J>
__device__ __forceinline__ float row_bcast_f(float x) {
  return __builtin_bit_cast(float, row_bcast<J>(__builtin_bit_cast(uint32_t, x)));
}

// One packed W4A16 word (8 nibbles = 8 consecutive k of the slice) against x
// dwords 2L .. 2L + 3 of the row (held by lanes L, L + 1): P += sum x (128 + q).
template <int L>
__device__ __forceinline__ void w4_word(float& P, uint32_t w, uint64_t x, uint32_t mask, uint32_t magic) {
  const uint32_t t0 = and_or_v(w, mask, magic);
  const uint32_t t1 = and_or_v(w >> 4, mask, magic);
  const uint32_t t2 = and_or_v(w >> 8, mask, magic);
  const uint32_t t3 = and_or_v(w >> 12, mask, magic);
  const uint64_t xa = row_bcast64<L>(x), xb = row_bcast64<L + 1>(x);
  P = dot2_bf16(as_bf16x2(lo32(xa)), as_bf16x2(t0), P);
  P = dot2_bf16(as_bf16x2(hi32(xa)), as_bf16x2(t1), P);
  P = dot2_bf16(as_bf16x2(lo32(xb)), as_bf16x2(t2), P);
  P = dot2_bf16(as_bf16x2(hi32(xb)), as_bf16x2(t3), P);
}

// The same for two activation rows sharing the dequantised word.
template <int L>
__device__ __forceinline__ void w4_word2(float& P0, float& P1, uint32_t w, uint64_t x0, uint64_t x1, uint32_t mask,
                                         uint32_t magic) {
  const uint32_t t[4] = {and_or_v(w, mask, magic), and_or_v(w >> 4, mask, magic), and_or_v(w >> 8, mask, magic),
                         and_or_v(w >> 12, mask, magic)};
  const uint64_t a0 = row_bcast64<L>(x0), b0 = row_bcast64<L + 1>(x0);
  const uint64_t a1 = row_bcast64<L>(x1), b1 = row_bcast64<L + 1>(x1);
  P0 = dot2_bf16(as_bf16x2(lo32(a0)), as_bf16x2(t[0]), P0);
  P1 = dot2_bf16(as_bf16x2(lo32(a1)), as_bf16x2(t[0]), P1);
  P0 = dot2_bf16(as_bf16x2(hi32(a0)), as_bf16x2(t[1]), P0);
  P1 = dot2_bf16(as_bf16x2(hi32(a1)), as_bf16x2(t[1]), P1);
  P0 = dot2_bf16(as_bf16x2(lo32(b0)), as_bf16x2(t[2]), P0);
  P1 = dot2_bf16(as_bf16x2(lo32(b1)), as_bf16x2(t[2]), P1);
  P0 = dot2_bf16(as_bf16x2(hi32(b0)), as_bf16x2(t[3]), P0);
  P1 = dot2_bf16(as_bf16x2(hi32(b1)), as_bf16x2(t[3]), P1);
}

// P += X(from lane C of the row) * nz, where nz = -(128 + z).
template <int C>
__device__ __forceinline__ void fmac_bcast(float& P, float X, float nz) {
  P = fmaf(row_bcast_f<C>(X), nz, P);
}

// acc += sum over 8 dwords of x (from lanes L .. L + 3, two each) * b[0..7].
template <int L>
__device__ __forceinline__ void dot8_bcast(float& acc, uint64_t x, const uint32_t (&b)[8]) {
  const uint64_t x0 = row_bcast64<L>(x), x1 = row_bcast64<L + 1>(x);
  const uint64_t x2 = row_bcast64<L + 2>(x), x3 = row_bcast64<L + 3>(x);
  acc = dot2_bf16(as_bf16x2(lo32(x0)), as_bf16x2(b[0]), acc);
  acc = dot2_bf16(as_bf16x2(hi32(x0)), as_bf16x2(b[1]), acc);
  acc = dot2_bf16(as_bf16x2(lo32(x1)), as_bf16x2(b[2]), acc);
  acc = dot2_bf16(as_bf16x2(hi32(x1)), as_bf16x2(b[3]), acc);
  acc = dot2_bf16(as_bf16x2(lo32(x2)), as_bf16x2(b[4]), acc);
  acc = dot2_bf16(as_bf16x2(hi32(x2)), as_bf16x2(b[5]), acc);
  acc = dot2_bf16(as_bf16x2(lo32(x3)), as_bf16x2(b[6]), acc);
  acc = dot2_bf16(as_bf16x2(hi32(x3)), as_bf16x2(b[7]), acc);
}

// acc += sum over 4 dwords of x (from lanes B .. B + 3) * w[0..3].
template <int B>
__device__ __forceinline__ void dot4_bcast(float& acc, uint32_t x, uint4 w) {
  acc = dot2_bf16(as_bf16x2(row_bcast<B>(x)), as_bf16x2(w.x), acc);
  acc = dot2_bf16(as_bf16x2(row_bcast<B + 1>(x)), as_bf16x2(w.y), acc);
  acc = dot2_bf16(as_bf16x2(row_bcast<B + 2>(x)), as_bf16x2(w.z), acc);
  acc = dot2_bf16(as_bf16x2(row_bcast<B + 3>(x)), as_bf16x2(w.w), acc);
}

// ---- per-tile arithmetic ---------------------------------------------------

// Tile I of a group; CI = its position in the wavefront's share (register
// CI / 16 of the W4A16 x sums holds it, in lane CI % 16 of each row).
template <int FMT, int MR, int XC, int I, int CI>
__device__ __forceinline__ void btile(const BGroup<FMT, MR>& g, const float (&X)[MR][XC], float (&acc)[MR]) {
  using C = BcC<FMT>;
  const uint4 wv = g.w[I];
  constexpr int R = I / C::TPX;               // x register of this tile
  constexpr int B = (I % C::TPX) * C::LPS;    // first lane of the row holding its x
  if constexpr (FMT == kFmtW4) {
    // constants in VGPRs, so each nibble pair is one v_and_or_b32
    const uint32_t mask = vgpr_const(0x000F000Fu), magic = vgpr_const(0x43004300u);
    const uint32_t sw = (I < 2 ? g.s.x : g.s.y) >> (16 * (I & 1));
    const float s = __half2float(__ushort_as_half(uint16_t(sw & 0xFFFFu)));
    const float nz = -(128.0f + float((g.z >> (4 * I)) & 0xFu));
    float P[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) P[m] = 0.f;
    if constexpr (MR == 1) {
      w4_word<B + 0>(P[0], wv.x, g.x[0][R], mask, magic);
      w4_word<B + 2>(P[0], wv.y, g.x[0][R], mask, magic);
      w4_word<B + 4>(P[0], wv.z, g.x[0][R], mask, magic);
      w4_word<B + 6>(P[0], wv.w, g.x[0][R], mask, magic);
    } else {
      w4_word2<B + 0>(P[0], P[1], wv.x, g.x[0][R], g.x[1][R], mask, magic);
      w4_word2<B + 2>(P[0], P[1], wv.y, g.x[0][R], g.x[1][R], mask, magic);
      w4_word2<B + 4>(P[0], P[1], wv.z, g.x[0][R], g.x[1][R], mask, magic);
      w4_word2<B + 6>(P[0], P[1], wv.w, g.x[0][R], g.x[1][R], mask, magic);
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
