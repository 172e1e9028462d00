// Decode attention over a KV cache, split along the context (Flash-Decoding).
//
// A decode step has one query per sequence, so attention is a matrix-vector
// product over the cache, and its time is the time to read the keys and
// values ("Making each token cheaper", section "Why kernels matter most for
// long prefill": decode attention is dominated by reading the KV cache; with
// one query per sequence, parallelising over batch and queries alone leaves
// most of the GPU idle, so Flash-Decoding splits the keys and values into
// chunks processed in parallel, then merges them).  Grouped-query heads
// ("LLM 推理是怎么变快的", section 2.3): the G = Hq / Hkv query heads of a
// group read one KV head, so one pass over that head's cache serves all G.
//
// Cache layout (library-defined; wqd_kv_pack / wqd_kv_append write it): per
// (sequence b, KV head g), 1 KiB tiles in the operand order of the matrix
// cores, so that every wavefront load is one contiguous 1 KiB:
//   K: tile (t / 16) * 4 + d / 32 holds positions 16 (t / 16) .. + 15 x head
//      dimensions 32 (d / 32) .. + 31: lane 16 kb + j (kb = (d % 32) / 8,
//      j = t % 16) holds the 8 dimensions 8 kb .. 8 kb + 7 of position j;
//   V: tile (t / 32) * 8 + d / 16 holds positions 32 (t / 32) .. + 31 x head
//      dimensions 16 (d / 16) .. + 15: lane 16 kb + n (n = d % 16) holds 8
//      positions u = t % 32 of dimension n, element e = 4 (u / 16) + u % 4
//      for kb = (u % 16) / 4, i.e. positions 4 kb .. 4 kb + 3 and
//      16 + 4 kb .. 16 + 4 kb + 3 (the order in which the score tiles leave
//      the softmax weights, below).
// Both take Lmax * 128 * 2 bytes per (b, g); Lmax is a multiple of 32.
//
// An FP8 cache ("LLM 推理是怎么变快的", section 4, C: keys and values stored
// as FP8 halve the cache's bytes) holds E4M3FN codes of K / k_scale and
// V / v_scale (one float32 scale per tensor), Lmax * 128 bytes per (b, g),
// in 1 KiB tiles that give each lane, in one 16-byte load, the codes of two
// of the bf16 operands above (bytes 0-7 the first, 8-15 the second):
//   K: tile (t / 16) * 2 + d / 64 holds positions 16 (t / 16) .. + 15 x
//      dimensions 64 (d / 64) .. + 63: lane 16 kb + j (kb = (d % 32) / 8,
//      j = t % 16), byte 8 ((d % 64) / 32) + d % 8, i.e. the operands of
//      head-dimension steps 2 (d / 64) and 2 (d / 64) + 1;
//   V: tile (t / 32) * 4 + d / 32 holds positions 32 (t / 32) .. + 31 x
//      dimensions 32 (d / 32) .. + 31: lane 16 kb + n (n = d % 16), byte
//      8 ((d % 32) / 16) + e (kb, e as for the bf16 V tile), i.e. the
//      operands of dimension blocks 2 (d / 32) and 2 (d / 32) + 1.
// Every E4M3 value is exact in bf16, so the kernel converts the codes to
// bf16 operands (scale 1) and runs the bf16 arithmetic below on them: the
// K scale joins the softmax scale, the V scale the final normalisation.  A
// step is 64 positions (16 loads of 1 KiB, as a bf16 step), computed as two
// halves of 32.
//
// attn_split_kernel: one workgroup of 4 wavefronts per (sequence b, KV head
// g, split s); the split's positions in steps of 32 (64 over an FP8 cache),
// wavefront w taking steps w, w + 4, ...  Per 32 positions, on bf16 matrix
// cores (v_mfma_f32_16x16x32_bf16):
//   * S^T = K Q^T as two 16-position tiles x 4 head-dimension steps: A = one
//     K tile (one 1 KiB load), B = Q^T, lane (kb, n) holding 8 head
//     dimensions of query head n of the group (heads G .. 15 zero).  Output
//     row 4 kb + r of tile tau is position 16 tau + 4 kb + r, so lane (kb, n)
//     ends up with 8 positions of query head n;
//   * online softmax in float32 with exp2 (scores times scale log2 e): the
//     running maximum and sum per head, reduced over the four lanes of a head
//     (shfl_xor 16, 32); positions at or past the sequence's length are set
//     to -inf by selection and their values to 0, so stale cache contents
//     never reach the sums;
//   * O += P V as 8 head-dimension blocks of 16: A = P, which the score tiles
//     left in operand order (lane (kb, n): head n, the 8 positions above),
//     split into bf16 high and low parts (two multiplies, error ~2^-17 of
//     each weight) so P is not rounded to 8 bits; B = one V tile, whose lane
//     (kb, n) holds dimension n at the same 8 positions;
//   * the next step's tiles are loaded before this step's arithmetic.
// The 4 wavefronts merge their running maxima, sums and unnormalised outputs
// through LDS, in wavefront order; with one split the workgroup normalises
// and stores the output, otherwise it writes its split's partials to the
// workspace and attn_combine_kernel merges the splits of each (b, head) in
// split order: o = sum_s 2^(m_s - m) o_s / sum_s 2^(m_s - m) l_s, rounded to
// bf16 (a sequence of length 0 gives zeros).
#include "wqd_device.h"
#include "wqd_internal.h"
#include "wqd_plan.h"

namespace wqd {

typedef __bf16 at_bf16x8_t __attribute__((ext_vector_type(8)));
typedef float at_f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kHeadDim = 128;
constexpr int kAttnWaves = 4;  // wavefronts per split, interleaving its 32-position steps
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ at_f32x4_t at_mfma(uint4 a, uint4 b, at_f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(at_bf16x8_t, a), __builtin_bit_cast(at_bf16x8_t, b),
                                                 c, 0, 0, 0);
}

struct AttnArgs {
  const uint16_t* q;    // [B][Hq][128]
  const uint16_t* k;    // K tiles, Lmax * 128 per (b, g)
  const uint16_t* v;    // V tiles, Lmax * 128 per (b, g)
  const int32_t* lens;  // [B]
  uint16_t* out;        // [B][Hq][128]
  float* part_ml;       // [B][Hq][S][2]: running maximum (log2 units), sum
  float* part_o;        // [B][Hq][S][128]: unnormalised output
  float scale_log2;     // softmax scale (times the K scale of an FP8 cache) times log2 e
  float out_scale;      // the V scale of an FP8 cache, 1 for bf16
  int64_t Lmax;
  int Hq, Hkv, G, S, chunk;  // chunk: positions per split, a multiple of the step (32 or 64)
};

struct AttnStepLoads {
  uint4 k[2][4];  // [tile][head-dimension step]
  uint4 v[8];     // [head-dimension block]
};

// The K and V tiles of the 32 positions from t0 (a multiple of 32): 16 loads
// of one contiguous 1 KiB each.  Past Lmax the tiles lie outside the
// resources and read zeros.
__device__ __forceinline__ void attn_load(AttnStepLoads& ld, __amdgpu_buffer_rsrc_t kres, __amdgpu_buffer_rsrc_t vres,
                                          int64_t t0, int lane) {
  const uint32_t kt = uint32_t(t0 / 16) * 4, vt = uint32_t(t0 / 32) * 8;
#pragma unroll
  for (int tau = 0; tau < 2; ++tau)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(kres, lane * 16, (kt + 4 * tau + s) * 1024, 0);
      ld.k[tau][s] = make_uint4(v.x, v.y, v.z, v.w);
    }
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(vres, lane * 16, (vt + c) * 1024, 0);
    ld.v[c] = make_uint4(v.x, v.y, v.z, v.w);
  }
}

// FP8 cache: the K and V tiles of the 64 positions from t0 (a multiple of
// 64): k[tau][h] = positions t0 + 16 tau .., dimensions 64 h ..;
// v[u][c] = positions t0 + 32 u .., dimensions 32 c ...
struct AttnStepLoads8 {
  uint4 k[4][2];
  uint4 v[2][4];
};

__device__ __forceinline__ void attn_load8(AttnStepLoads8& ld, __amdgpu_buffer_rsrc_t kres,
                                           __amdgpu_buffer_rsrc_t vres, int64_t t0, int lane) {
  const uint32_t kt = uint32_t(t0 / 16) * 2, vt = uint32_t(t0 / 32) * 4;
#pragma unroll
  for (int tau = 0; tau < 4; ++tau)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(kres, lane * 16, (kt + 2 * tau + h) * 1024, 0);
      ld.k[tau][h] = make_uint4(v.x, v.y, v.z, v.w);
    }
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(vres, lane * 16, (vt + 4 * u + c) * 1024, 0);
      ld.v[u][c] = make_uint4(v.x, v.y, v.z, v.w);
    }
}

// Eight E4M3 codes (two words) -> eight bf16, exact.
__device__ __forceinline__ uint4 e4m3x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  return make_uint4(__builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<false>(w0)),
                    __builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<true>(w0)),
                    __builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<false>(w1)),
                    __builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<true>(w1)));
}

__device__ __forceinline__ uint4 e4m3_half_to_bf16(const uint4& w, int half) {
  return half == 0 ? e4m3x8_to_bf16x8(w.x, w.y) : e4m3x8_to_bf16x8(w.z, w.w);
}

struct AttnState {
  at_f32x4_t o[8];  // [head-dimension block]: lane (kb, n) rows 4 kb + r, column n
  float m, l;       // running maximum (log2 units) and sum of head n (lane (kb, n))
};

__device__ __forceinline__ uint32_t bf16_pair(float a, float b) {
  return f32_to_bf16_rne(a) | (f32_to_bf16_rne(b) << 16);
}

// One step over positions t0 .. t0 + 31, of which those below `len` count.
__device__ __forceinline__ void attn_step(AttnState& st, AttnStepLoads& ld, const uint4 (&qf)[4], float sl2,
                                         int64_t t0, int64_t len, int kb, int n) {
  at_f32x4_t sc[2];
#pragma unroll
  for (int tau = 0; tau < 2; ++tau) {
    sc[tau] = at_f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) sc[tau] = at_mfma(ld.k[tau][s], qf[s], sc[tau]);
  }
  // lane (kb, n): head n, position t0 + 16 tau + 4 kb + r in element i = 4 tau + r
  float x[8];
  const int64_t rel = len - t0 - 4 * kb;  // element i counts when 16 (i / 4) + i % 4 < rel
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float v = sc[i >> 2][i & 3] * sl2;
    x[i] = 16 * (i >> 2) + (i & 3) < rel ? v : -INFINITY;
  }
  float mt = x[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) mt = fmaxf(mt, x[i]);
  mt = fmaxf(mt, __shfl_xor(mt, 16));
  mt = fmaxf(mt, __shfl_xor(mt, 32));
  const float mn = fmaxf(st.m, mt);  // finite: position t0 < len is in this step
  const float alpha = exp2f(st.m - mn);
  float p[8], ps = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    p[i] = exp2f(x[i] - mn);
    ps += p[i];
  }
  ps += __shfl_xor(ps, 16);
  ps += __shfl_xor(ps, 32);
  st.l = st.l * alpha + ps;
  st.m = mn;
  // P as operand A: high and low bf16 parts
  uint32_t hi[4], lo[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t h = bf16_pair(p[2 * e], p[2 * e + 1]);
    hi[e] = h;
    lo[e] = bf16_pair(p[2 * e] - bf16_bits_to_f32(h & 0xFFFFu), p[2 * e + 1] - bf16_bits_to_f32(h >> 16));
  }
  const uint4 ph = make_uint4(hi[0], hi[1], hi[2], hi[3]), pl = make_uint4(lo[0], lo[1], lo[2], lo[3]);
  // V elements of positions past the length are zeroed (stale cache slots);
  // only a step that reaches the length has any (a wave-uniform test)
  if (t0 + 32 > len) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      uint32_t w[4] = {ld.v[c].x, ld.v[c].y, ld.v[c].z, ld.v[c].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i0 = 2 * e, i1 = 2 * e + 1;
        const uint32_t keep = (16 * (i0 >> 2) + (i0 & 3) < rel ? 0x0000FFFFu : 0u) |
                              (16 * (i1 >> 2) + (i1 & 3) < rel ? 0xFFFF0000u : 0u);
        w[e] &= keep;
      }
      ld.v[c] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
  // rescale the running output: its row 4 kb + r is head 4 kb + r, whose
  // alpha lane 4 kb + r holds
  float ar[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * kb + r);
#pragma unroll
  for (int c = 0; c < 8; ++c) {
#pragma unroll
    for (int r = 0; r < 4; ++r) st.o[c][r] *= ar[r];
    st.o[c] = at_mfma(ph, ld.v[c], st.o[c]);
    st.o[c] = at_mfma(pl, ld.v[c], st.o[c]);
  }
}

// One FP8 step over positions t0 .. t0 + 63: each half of 32 positions is
// converted to the bf16 operands of attn_step (exactly) and run through it;
// the second half is skipped when it lies wholly at or past the length.
__device__ __forceinline__ void attn_step8(AttnState& st, const AttnStepLoads8& l8, const uint4 (&qf)[4], float sl2,
                                          int64_t t0, int64_t len, int kb, int n) {
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    if (u == 1 && t0 + 32 >= len) break;  // wave-uniform
    AttnStepLoads ld;
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int s = 0; s < 4; ++s) ld.k[tau][s] = e4m3_half_to_bf16(l8.k[2 * u + tau][s >> 1], s & 1);
#pragma unroll
    for (int c = 0; c < 8; ++c) ld.v[c] = e4m3_half_to_bf16(l8.v[u][c >> 1], c & 1);
    attn_step(st, ld, qf, sl2, t0 + 32 * u, len, kb, n);
  }
}

template <bool FP8>
__global__ __launch_bounds__(64 * kAttnWaves) void attn_split_kernel(AttnArgs a) {
  constexpr int W = kAttnWaves;
  __shared__ float s_ml[W][2][16];
  __shared__ float s_o[W][16][kHeadDim];
  const int lane = threadIdx.x & 63, kb = lane >> 4, n = lane & 15;
  const int wave = threadIdx.x >> 6;
  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int64_t Lmax = a.Lmax;
  int64_t len = a.lens[b];
  len = len < 0 ? 0 : (len > Lmax ? Lmax : len);
  const int64_t t_begin = int64_t(s) * a.chunk;
  const int64_t t_end = t_begin + a.chunk < len ? t_begin + a.chunk : len;

  // query heads of the group as operand B (heads G .. 15 zero)
  uint4 qf[4];
  const int64_t hq = int64_t(g) * a.G + n;
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    qf[st] = make_uint4(0u, 0u, 0u, 0u);
    if (n < a.G) qf[st] = *reinterpret_cast<const uint4*>(a.q + (int64_t(b) * a.Hq + hq) * kHeadDim + 32 * st + 8 * kb);
  }
  const int64_t head = int64_t(b) * a.Hkv + g;
  constexpr int EB = FP8 ? 1 : 2;  // bytes per cache element
  const int64_t region = Lmax * kHeadDim * EB;
  const __amdgpu_buffer_rsrc_t kres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(reinterpret_cast<const char*>(a.k) + head * region), 0, uint32_t(region), 0x00020000);
  const __amdgpu_buffer_rsrc_t vres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(reinterpret_cast<const char*>(a.v) + head * region), 0, uint32_t(region), 0x00020000);

  AttnState st;
#pragma unroll
  for (int c = 0; c < 8; ++c) st.o[c] = at_f32x4_t{0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;
  st.l = 0.f;
  // wavefront w takes the split's steps w, w + W, w + 2 W, ...
  constexpr int64_t STEP = FP8 ? 64 : 32;
  constexpr int64_t STRIDE = STEP * W;
  const int64_t t0 = t_begin + STEP * wave;
  if (FP8 && t0 < t_end) {
    // as below, on 64-position steps (the chunk is a multiple of 64, so a
    // step ends at or before its split's end)
    AttnStepLoads8 l0, l1;
    attn_load8(l0, kres, vres, t0, lane);
    int64_t t = t0;
    for (; t + STRIDE < t_end; t += 2 * STRIDE) {
      attn_load8(l1, kres, vres, t + STRIDE, lane);
      attn_step8(st, l0, qf, a.scale_log2, t, len, kb, n);
      attn_load8(l0, kres, vres, t + 2 * STRIDE, lane);
      attn_step8(st, l1, qf, a.scale_log2, t + STRIDE, len, kb, n);
    }
    if (t < t_end) attn_step8(st, l0, qf, a.scale_log2, t, len, kb, n);
  } else if (!FP8 && t0 < t_end) {
    // two register sets: each step loads the wavefront's next step before its
    // own arithmetic (a step past the split reads in-bounds or zero tiles that
    // are never used)
    AttnStepLoads l0, l1;
    attn_load(l0, kres, vres, t0, lane);
    int64_t t = t0;
    for (; t + STRIDE < t_end; t += 2 * STRIDE) {
      attn_load(l1, kres, vres, t + STRIDE, lane);
      attn_step(st, l0, qf, a.scale_log2, t, len, kb, n);
      // unconditional: a conditional load would make the compiler wait for
      // every load at the join, this one included
      attn_load(l0, kres, vres, t + 2 * STRIDE, lane);
      attn_step(st, l1, qf, a.scale_log2, t + STRIDE, len, kb, n);
    }
    if (t < t_end) attn_step(st, l0, qf, a.scale_log2, t, len, kb, n);
  }

  // merge the W wavefronts through LDS: lane (kb, n) holds head n's maximum
  // and sum, and rows 4 kb + r (heads) of column n of each 16-dimension block
  if (kb == 0) {
    s_ml[wave][0][n] = st.m;
    s_ml[wave][1][n] = st.l;
  }
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) s_o[wave][4 * kb + r][16 * c + n] = st.o[c][r];
  __syncthreads();
  // thread i: head h = i / 64 (and h + 4, + 8, + 12), dimensions 2 (i % 64), + 1
  const int dp = threadIdx.x % 64;
  for (int h = threadIdx.x / 64; h < a.G; h += W) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; ++w) M = fmaxf(M, s_ml[w][0][h]);
    float L = 0.f, o0 = 0.f, o1 = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const float f = exp2f(s_ml[w][0][h] - M);  // 0 for a wavefront without positions
        L += f * s_ml[w][1][h];
        o0 += f * s_o[w][h][2 * dp];
        o1 += f * s_o[w][h][2 * dp + 1];
      }
    }
    const int64_t bh = int64_t(b) * a.Hq + int64_t(g) * a.G + h;
    if (a.S == 1) {  // the whole context: normalise and store (no merge launch)
      const float inv = M != -INFINITY ? a.out_scale / L : 0.f;
      reinterpret_cast<uint32_t*>(a.out + bh * kHeadDim)[dp] = bf16_pair(o0 * inv, o1 * inv);
    } else {
      const int64_t row = bh * a.S + s;
      if (dp == 0) {
        a.part_ml[2 * row] = M;
        a.part_ml[2 * row + 1] = L;
      }
      reinterpret_cast<float2*>(a.part_o + row * kHeadDim)[dp] = make_float2(o0, o1);
    }
  }
}

// One wavefront per (b, query head): merge the S splits in split order.
__global__ __launch_bounds__(64) void attn_combine_kernel(AttnArgs a) {
  const int lane = threadIdx.x;
  const int64_t bh = int64_t(blockIdx.y) * a.Hq + blockIdx.x;
  const float* ml = a.part_ml + bh * a.S * 2;
  float M = -INFINITY;
  for (int s = 0; s < a.S; ++s) M = fmaxf(M, ml[2 * s]);
  float o0 = 0.f, o1 = 0.f, L = 0.f;
  if (M != -INFINITY) {
    const float* po = a.part_o + bh * a.S * kHeadDim;
    for (int s = 0; s < a.S; ++s) {
      const float w = exp2f(ml[2 * s] - M);  // 0 for an empty split
      L += w * ml[2 * s + 1];
      o0 += w * po[s * kHeadDim + 2 * lane];
      o1 += w * po[s * kHeadDim + 2 * lane + 1];
    }
    const float inv = a.out_scale / L;
    o0 *= inv;
    o1 *= inv;
  }
  reinterpret_cast<uint32_t*>(a.out + bh * kHeadDim)[lane] = bf16_pair(o0, o1);
}

hipError_t launch_attn(const AttnPlan& p, const void* q, const void* k, const void* v, const int32_t* lens,
                       int64_t B, float scale, float k_scale, float v_scale, void* out, void* ws, hipStream_t st) {
  AttnArgs a;
  a.q = reinterpret_cast<const uint16_t*>(q);
  a.k = reinterpret_cast<const uint16_t*>(k);
  a.v = reinterpret_cast<const uint16_t*>(v);
  a.lens = lens;
  a.out = reinterpret_cast<uint16_t*>(out);
  a.part_ml = reinterpret_cast<float*>(ws);
  a.part_o = a.part_ml + B * p.Hq * p.S * 2;
  a.scale_log2 = scale * k_scale * kLog2e;
  a.out_scale = v_scale;
  a.Lmax = p.Lmax;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.G = p.Hq / p.Hkv;
  a.S = p.S;
  a.chunk = p.chunk;
  const dim3 grid(unsigned(p.S), unsigned(p.Hkv), unsigned(B));
  if (p.fp8_kv)
    hipLaunchKernelGGL(attn_split_kernel<true>, grid, dim3(64 * kAttnWaves), 0, st, a);
  else
    hipLaunchKernelGGL(attn_split_kernel<false>, grid, dim3(64 * kAttnWaves), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.S == 1) return e;
  hipLaunchKernelGGL(attn_combine_kernel, dim3(unsigned(p.Hq), unsigned(B)), dim3(64), 0, st, a);
  return hipGetLastError();
}

// ------------------------------------------------------------------ cache writers
// Element offsets (bf16 units) of position t, dimension d inside one (b, g)
// region of the K and V tiles (layout above).
__device__ __forceinline__ int64_t kv_k_index(int64_t t, int d) {
  return ((t / 16) * 4 + d / 32) * 512 + (((d % 32) / 8) * 16 + (t % 16)) * 8 + (d % 8);
}

__device__ __forceinline__ int64_t kv_v_index(int64_t t, int d) {
  const int u = int(t % 32), kb = (u % 16) / 4, e = 4 * (u / 16) + (u % 4);
  return ((t / 32) * 8 + d / 16) * 512 + (kb * 16 + (d % 16)) * 8 + e;
}

// One thread per (b, g, t, dimension pair): logical [B][Hkv][L][128] <-> tiles.
// DIR 0: pack (logical -> tiles), 1: unpack (tiles -> logical).
template <int DIR>
__global__ __launch_bounds__(256) void kv_copy_kernel(const uint16_t* __restrict__ src_k,
                                                      const uint16_t* __restrict__ src_v, uint16_t* __restrict__ dst_k,
                                                      uint16_t* __restrict__ dst_v, int64_t BH, int64_t L,
                                                      int64_t Lmax) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= BH * L * (kHeadDim / 2)) return;
  const int d = int(i % (kHeadDim / 2)) * 2;
  const int64_t t = (i / (kHeadDim / 2)) % L, bh = i / (kHeadDim / 2) / L;
  const int64_t lin = (bh * L + t) * kHeadDim + d;  // logical [bh][t][d] with row stride L
  const int64_t tile = bh * Lmax * kHeadDim;
  if (DIR == 0) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      dst_k[tile + kv_k_index(t, d + e)] = src_k[lin + e];
      dst_v[tile + kv_v_index(t, d + e)] = src_v[lin + e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      dst_k[lin + e] = src_k[tile + kv_k_index(t, d + e)];
      dst_v[lin + e] = src_v[tile + kv_v_index(t, d + e)];
    }
  }
}

// One position per sequence: k_new / v_new [B][Hkv][128] at positions[b]
// (a position outside [0, Lmax) writes nothing).
__global__ __launch_bounds__(256) void kv_append_kernel(const uint16_t* __restrict__ k_new,
                                                        const uint16_t* __restrict__ v_new,
                                                        const int32_t* __restrict__ positions, uint16_t* __restrict__ k,
                                                        uint16_t* __restrict__ v, int64_t B, int64_t Hkv,
                                                        int64_t Lmax) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= B * Hkv * kHeadDim) return;
  const int d = int(i % kHeadDim);
  const int64_t bh = i / kHeadDim, b = bh / Hkv;
  const int64_t t = positions[b];
  if (t < 0 || t >= Lmax) return;
  const int64_t tile = bh * Lmax * kHeadDim;
  k[tile + kv_k_index(t, d)] = k_new[i];
  v[tile + kv_v_index(t, d)] = v_new[i];
}

hipError_t launch_kv_copy(bool pack, const void* src_k, const void* src_v, void* dst_k, void* dst_v, int64_t BH,
                          int64_t L, int64_t Lmax, hipStream_t st) {
  const int64_t n = BH * L * (kHeadDim / 2);
  if (n == 0) return hipSuccess;
  const dim3 grid(unsigned(ceil_div(n, int64_t(256))));
  const auto* sk = reinterpret_cast<const uint16_t*>(src_k);
  const auto* sv = reinterpret_cast<const uint16_t*>(src_v);
  auto* dk = reinterpret_cast<uint16_t*>(dst_k);
  auto* dv = reinterpret_cast<uint16_t*>(dst_v);
  if (pack)
    hipLaunchKernelGGL(kv_copy_kernel<0>, grid, dim3(256), 0, st, sk, sv, dk, dv, BH, L, Lmax);
  else
    hipLaunchKernelGGL(kv_copy_kernel<1>, grid, dim3(256), 0, st, sk, sv, dk, dv, BH, L, Lmax);
  return hipGetLastError();
}

hipError_t launch_kv_append(const void* k_new, const void* v_new, const int32_t* positions, int64_t B, int64_t Hkv,
                            int64_t Lmax, void* k, void* v, hipStream_t st) {
  const int64_t n = B * Hkv * kHeadDim;
  hipLaunchKernelGGL(kv_append_kernel, dim3(unsigned(ceil_div(n, int64_t(256)))), dim3(256), 0, st,
                     reinterpret_cast<const uint16_t*>(k_new), reinterpret_cast<const uint16_t*>(v_new), positions,
                     reinterpret_cast<uint16_t*>(k), reinterpret_cast<uint16_t*>(v), B, Hkv, Lmax);
  return hipGetLastError();
}

// ------------------------------------------------------------ FP8 cache writers
// Byte offsets of position t, dimension d inside one (b, g) region of the FP8
// K and V tiles (layout above).
__device__ __forceinline__ int64_t kv8_k_index(int64_t t, int d) {
  return ((t / 16) * 2 + d / 64) * 1024 + (((d % 32) / 8) * 16 + (t % 16)) * 16 + 8 * ((d % 64) / 32) + (d % 8);
}

__device__ __forceinline__ int64_t kv8_v_index(int64_t t, int d) {
  const int u = int(t % 32), kb = (u % 16) / 4, e = 4 * (u / 16) + (u % 4);
  return ((t / 32) * 4 + d / 32) * 1024 + (kb * 16 + (d % 16)) * 16 + 8 * ((d % 32) / 16) + e;
}

// The E4M3 code of a bf16 value for a per-tensor scale: the nearest E4M3FN
// value of x / scale (float32 division, ties to even, saturating at 448).
__device__ __forceinline__ uint8_t kv8_code(uint16_t x, float scale) {
  return uint8_t(e4m3_encode(__fdiv_rn(bf16_bits_to_f32(x), scale)));
}

// One thread per (b, g, t, dimension pair).  DIR 0: quantise logical bf16
// [BH][L][128] into the tiles; 1: the tiles' codes back to logical uint8
// [BH][L][128].
template <int DIR>
__global__ __launch_bounds__(256) void kv8_copy_kernel(const void* __restrict__ src_k, const void* __restrict__ src_v,
                                                       uint8_t* __restrict__ dst_k, uint8_t* __restrict__ dst_v,
                                                       float k_scale, float v_scale, int64_t BH, int64_t L,
                                                       int64_t Lmax) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= BH * L * (kHeadDim / 2)) return;
  const int d = int(i % (kHeadDim / 2)) * 2;
  const int64_t t = (i / (kHeadDim / 2)) % L, bh = i / (kHeadDim / 2) / L;
  const int64_t lin = (bh * L + t) * kHeadDim + d;
  const int64_t tile = bh * Lmax * kHeadDim;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    if (DIR == 0) {
      dst_k[tile + kv8_k_index(t, d + e)] = kv8_code(static_cast<const uint16_t*>(src_k)[lin + e], k_scale);
      dst_v[tile + kv8_v_index(t, d + e)] = kv8_code(static_cast<const uint16_t*>(src_v)[lin + e], v_scale);
    } else {
      dst_k[lin + e] = static_cast<const uint8_t*>(src_k)[tile + kv8_k_index(t, d + e)];
      dst_v[lin + e] = static_cast<const uint8_t*>(src_v)[tile + kv8_v_index(t, d + e)];
    }
  }
}

// One position per sequence, quantised: k_new / v_new bf16 [B][Hkv][128] at
// positions[b] (a position outside [0, Lmax) writes nothing).
__global__ __launch_bounds__(256) void kv8_append_kernel(const uint16_t* __restrict__ k_new,
                                                         const uint16_t* __restrict__ v_new,
                                                         const int32_t* __restrict__ positions,
                                                         uint8_t* __restrict__ k, uint8_t* __restrict__ v,
                                                         float k_scale, float v_scale, int64_t B, int64_t Hkv,
                                                         int64_t Lmax) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= B * Hkv * kHeadDim) return;
  const int d = int(i % kHeadDim);
  const int64_t bh = i / kHeadDim, b = bh / Hkv;
  const int64_t t = positions[b];
  if (t < 0 || t >= Lmax) return;
  const int64_t tile = bh * Lmax * kHeadDim;
  k[tile + kv8_k_index(t, d)] = kv8_code(k_new[i], k_scale);
  v[tile + kv8_v_index(t, d)] = kv8_code(v_new[i], v_scale);
}

hipError_t launch_kv8_copy(bool pack, const void* src_k, const void* src_v, void* dst_k, void* dst_v, float k_scale,
                           float v_scale, int64_t BH, int64_t L, int64_t Lmax, hipStream_t st) {
  const int64_t n = BH * L * (kHeadDim / 2);
  if (n == 0) return hipSuccess;
  const dim3 grid(unsigned(ceil_div(n, int64_t(256))));
  auto* dk = reinterpret_cast<uint8_t*>(dst_k);
  auto* dv = reinterpret_cast<uint8_t*>(dst_v);
  if (pack)
    hipLaunchKernelGGL(kv8_copy_kernel<0>, grid, dim3(256), 0, st, src_k, src_v, dk, dv, k_scale, v_scale, BH, L,
                       Lmax);
  else
    hipLaunchKernelGGL(kv8_copy_kernel<1>, grid, dim3(256), 0, st, src_k, src_v, dk, dv, k_scale, v_scale, BH, L,
                       Lmax);
  return hipGetLastError();
}

hipError_t launch_kv8_append(const void* k_new, const void* v_new, float k_scale, float v_scale,
                             const int32_t* positions, int64_t B, int64_t Hkv, int64_t Lmax, void* k, void* v,
                             hipStream_t st) {
  const int64_t n = B * Hkv * kHeadDim;
  hipLaunchKernelGGL(kv8_append_kernel, dim3(unsigned(ceil_div(n, int64_t(256)))), dim3(256), 0, st,
                     reinterpret_cast<const uint16_t*>(k_new), reinterpret_cast<const uint16_t*>(v_new), positions,
                     reinterpret_cast<uint8_t*>(k), reinterpret_cast<uint8_t*>(v), k_scale, v_scale, B, Hkv, Lmax);
  return hipGetLastError();
}

}  // namespace wqd
