// Per-tile arithmetic of the streaming decode kernels that broadcast x by
// DPP (the one-launch-per-matrix kernel in wqd_gemv_bcast.hip and the
// persistent chain kernel in wqd_chain.hip): the register groups, the row
// broadcasts, and the products of one packed 1 KiB tile against one or two
// activation rows.
//
// In a packed tile the 16 lanes of one DPP row (kb fixed, n = 0..15) all
// multiply the same k-slice, and a slice holds at most 16 dwords of x (32
// bf16), so one x register per one to four tiles covers them: for W4A16 and
// FP8 a 64-bit register, lane (kb, j) holding dwords 2j, 2j + 1 of a slice (8
// lanes per W4A16 slice, 4 per FP8 slice), for BF16 a 32-bit one (dword j, 4
// lanes per slice).  A DPP row broadcast (row_newbcast:j, gfx90a and later)
// hands lane j's value to every lane of the row, where it feeds
// v_dot2_f32_bf16.
//
// W4A16 zero points: a tile contributes s * (P - (128 + z) * X) with
// P = sum x (128 + q) over a lane's slice and X = sum x over the same slice
// from an identical dot2 chain (so q == z == 0 cancels exactly).  X depends
// on (tile, slice) only: lane (kb, n) of register c holds X for tile 16 c + n
// of the share, and the correction reads it back with the same row broadcast.
//
// DPP.  The row broadcast is a compiler builtin (a v_mov with the
// row_newbcast control) feeding ordinary dot2 / fma builtins, so the
// compiler's hazard recognizer inserts the wait states around it: gfx950 has
// no folded DPP form of v_dot2c_f32_bf16 that the compiler would form, so
// each broadcast dword costs one move.
#pragma once
#include <type_traits>

#include "wqd_device.h"
#include "wqd_internal.h"

namespace wqd {

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

}  // namespace wqd
