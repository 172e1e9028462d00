// Device helpers shared by the gfx950 kernels: number-format conversions and
// the in-register dequantisation primitives.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace wqd {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte load marked non-temporal (streamed data that is read once).
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// float32 -> bfloat16 bits, round to nearest even (finite inputs; subnormals kept).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Gate/up pairs packed for the SwiGLU epilogue (the MLP's gate and up
// projections share their input, and its output is silu(gate) * up: CS336
// lecture 10 notes, section 3.2 on the MLP's three matrices): the packed
// matrix has N = 2F rows, 16-row block b holding gate rows 8b .. 8b + 7 and
// then up rows 8b .. 8b + 7, from a source W = [gate rows 0 .. F - 1;
// up rows F .. 2F - 1].  src_row gives the source row of packed row n (F = 0:
// no interleave).
__device__ __forceinline__ int64_t src_row(int64_t n, int64_t F) {
  if (F == 0) return n;
  const int64_t b = n / 16, r = n % 16;
  return r < 8 ? 8 * b + r : F + 8 * b + (r - 8);
}

// The output of element (activation row m, packed row n) with final float32
// value v.  Plain: y[m][n] = bf16(v), y with N columns.  SwiGLU: y has N / 2
// columns; the gate element (n % 16 < 8) stores y[m][8 (n / 16) + n % 8] =
// bf16(silu(v) * u), u = silu's partner value of packed row n + 8, which the
// caller's lane `lane ^ PX` holds.  swiglu must be uniform over the
// wavefront, and under it both lanes of a pair call this together (it
// shuffles); `live` = this lane's element exists (the same for both of a pair).
template <int PX>
__device__ __forceinline__ void store_out(uint16_t* y, int64_t N, bool swiglu, int64_t m, int64_t n, float v,
                                          bool live) {
  if (!swiglu) {
    if (live) y[m * N + n] = uint16_t(f32_to_bf16_rne(v));
    return;
  }
  const float u = __shfl_xor(v, PX);
  if (live && (n & 8) == 0) {
    const float h = v / (1.0f + expf(-v)) * u;
    y[m * (N / 2) + (n >> 4) * 8 + (n & 7)] = uint16_t(f32_to_bf16_rne(h));
  }
}

// Two FP8-E4M3 codes (bytes 0,1 or bytes 2,3 of `w`) -> two bf16 in one register.
// gfx950's conversion decodes the OCP E4M3FN encoding; every E4M3 value is
// exactly representable in bf16, and a scale of 1 leaves it unchanged.
template <bool HI>
__device__ __forceinline__ bf16x2_t e4m3x2_to_bf16x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
}

// Nearest FP8-E4M3FN value of v, ties to even mantissa, magnitudes above 448
// saturate to 448; the sign bit is v's sign bit.  Written from the format's
// definition ("Making each token cheaper", "Weight quantization / Formats":
// 4 exponent bits, 3 mantissa bits, largest normal 448): the spacing of
// representable values in the binade [2^E, 2^(E+1)) is 2^(E-3), and below
// 2^-6 (the subnormals) it is 2^-9.
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fminf(fabsf(v), 448.0f);
  if (a == 0.0f) return sign;
  int e;
  (void)frexpf(a, &e);            // a = m * 2^e, m in [0.5, 1)
  int E = e - 1;                  // binade of a
  if (E < -6) E = -6;             // subnormals use the spacing of 2^-6's binade
  const float r = rintf(ldexpf(a, 3 - E));  // a / 2^(E-3), exact power-of-two scaling
  const uint32_t mr = uint32_t(r);          // in [0, 16]
  if (E == -6 && mr < 8) return sign | mr;  // subnormal: value = mr * 2^-9
  int Eb = E;
  uint32_t mant = mr;
  if (mant == 16) {  // rounded up into the next binade
    Eb += 1;
    mant = 8;
  }
  return sign | (uint32_t(Eb + 7) << 3) | (mant - 8);
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t code) {
  bf16x2_t v = e4m3x2_to_bf16x2<false>(code & 0xFFu);
  return bf16_bits_to_f32(__builtin_bit_cast(uint32_t, v) & 0xFFFFu);
}

// W4A16 nibble order inside a packed 32-bit word: nibble t (bits 4t..4t+3)
// holds element kNibElem[t] of the word's 8 consecutive k, so that
// (w >> 4t) & 0x000F000F yields elements (2t, 2t+1) in the low and high half.
__device__ __forceinline__ int nib_elem(int t) { return (t & 3) * 2 + (t >> 2); }

// Elements (2t, 2t+1) of a packed word as bf16 (128 + q0, 128 + q1): OR-ing a
// 4-bit code into the low mantissa bits of 128.0 (0x4300) gives 128 + q exactly.
template <int T>
__device__ __forceinline__ bf16x2_t u4x2_to_bf16x2_offset128(uint32_t w) {
  uint32_t v = ((w >> (4 * T)) & 0x000F000Fu) | 0x43004300u;
  return __builtin_bit_cast(bf16x2_t, v);
}

// (a & mask) | orv, which the compiler turns into one v_and_or_b32 when both
// constants sit in VGPRs: a gfx9 VOP3 instruction takes no literal and one
// scalar operand, so with literal constants it would split the operation
// into v_and + v_or.  vgpr_const() makes a constant opaque so that it stays in
// a VGPR.  Plain code (no inline assembly) keeps the result visible to the
// compiler's hazard tracking, e.g. before a matrix-core instruction reads it.
__device__ __forceinline__ uint32_t vgpr_const(uint32_t c) {
  asm volatile("" : "+v"(c));
  return c;
}

__device__ __forceinline__ uint32_t and_or_v(uint32_t a, uint32_t mask, uint32_t orv) { return (a & mask) | orv; }

__device__ __forceinline__ float dot2_bf16(bf16x2_t a, bf16x2_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
}

__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2_t, v); }

}  // namespace wqd
