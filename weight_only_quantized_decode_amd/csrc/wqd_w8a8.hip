// W8A8-FP8: activations quantised to FP8-E4M3 with one dynamic scale per
// tensor, multiplied against the FP8 packed weights on the FP8 matrix cores.
//
// The pages prescribe this variant once the matrix product, not the weight
// bytes, sets the time: large batches, wide verify passes, prefill ("Making
// each token cheaper", section "What quantization saves": only a format whose
// product runs at lower precision, FP8 or INT8 W8A8 on hardware that has it,
// reduces that arithmetic; "Weight quantization / Formats": E4M3 for weights
// and activations, a scale applied before the cast, per channel for weights
// and per tensor for activations).  gfx950's v_mfma_f32_16x16x128_f8f6f4
// multiplies two E4M3 operands at twice the bf16 matrix rate, and no operand
// needs converting.
//
// Activation quantisation (two small kernels, no atomics, deterministic):
//   act_absmax_kernel  G workgroups, each the largest |x| of a contiguous
//                      range, to the workspace;
//   act_quant_kernel   every workgroup reduces the G values itself (all get
//                      the same maximum), s_a = max / 448 (float32; 1 for an
//                      all-zero tensor, at least 2^-126), workgroup 0 stores
//                      it, and each thread encodes 8 activations as the
//                      nearest E4M3 of x / s_a (ties to even, saturating;
//                      the hardware conversion after a clamp to +-448).
//
// The product, up to 255 rows (and where the LDS-staged form below would fill
// the compute units' rounds poorly) w8_gemm_kernel<MF, WR>: a workgroup computes a BM x 256 tile
// of y, BM = 16 MF WR, with WR x 4 wavefronts, each 16 MF rows x 4 weight row
// blocks (64 columns); instantiated for MF = 2, 4, 8 and WR = 1 (at WR = 2
// the 128-row wavefront tiles need one register more than the 256 a lane has).  K advances in 128-k chunks, one multiply per (x row
// block, weight row block) and chunk:
//   * B operand: two consecutive packed FP8 tiles of a weight row block, lane
//     16 g + n holding slice g of row n of each: k = 16 g .. 16 g + 15 of the
//     chunk in bytes 0-15, and 64 + 16 g .. 64 + 16 g + 15 in bytes 16-31,
//     loaded straight from memory (the packed tile is already in lane order);
//   * A operand: the activation codes with the same (lane, byte) -> k
//     mapping, row 16 i + n of the block instead of weight row n.  They go
//     from memory straight into LDS (16-byte loads that write LDS, lane l at
//     16 l), half h of fragment i holding the bytes 16 h .. 16 h + 15 of every
//     lane; a lane reads its two halves back with two conflict-free 16-byte
//     LDS reads.  A k-mapping shared by both operands is all the multiply
//     needs: it sums over k whatever the order;
//   * the pipeline, waits and barriers follow the bf16 tiled kernel: NS stage
//     buffers, one LDS array each, every load issued NS - 1 chunks ahead in a
//     fixed order (x, then weights), an explicit wait for this wavefront's x
//     of the next chunk and a bare barrier at the end of each step;
//   * y = bf16(acc * s_a * s_n); with a K split the partials acc * s_a go to
//     the workspace and the shared split-K sum applies s_n.
#include "wqd_device.h"
#include "wqd_internal.h"
#include "wqd_plan.h"

namespace wqd {

typedef int w8_i32x8_t __attribute__((ext_vector_type(8)));
typedef float w8_f32x4_t __attribute__((ext_vector_type(4)));

// acc += A (16 rows x 128 k, E4M3) . B (16 columns x 128 k, E4M3)^T; the
// scale operands of the scaled form are 0, which selects the plain
// instruction (both formats E4M3: cbsz = blgp = 0).
__device__ __forceinline__ w8_f32x4_t w8_mfma(uint4 a0, uint4 a1, uint4 b0, uint4 b1, w8_f32x4_t c) {
  const w8_i32x8_t a = {int(a0.x), int(a0.y), int(a0.z), int(a0.w), int(a1.x), int(a1.y), int(a1.z), int(a1.w)};
  const w8_i32x8_t b = {int(b0.x), int(b0.y), int(b0.z), int(b0.w), int(b1.x), int(b1.y), int(b1.z), int(b1.w)};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// ------------------------------------------------------------------ activation quantisation
__device__ __forceinline__ float block_max_256(float a, float* red) {
  for (int off = 32; off > 0; off >>= 1) a = fmaxf(a, __shfl_xor(a, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ float absmax8(uint4 v) {
  const uint32_t u[4] = {v.x, v.y, v.z, v.w};
  float a = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) a = fmaxf(a, fmaxf(fabsf(bf16_lo(u[e])), fabsf(bf16_hi(u[e]))));
  return a;
}

// part[b] = largest |x| over the b-th of G contiguous ranges of the n16
// 16-byte pieces (8 bf16 each) of x; 8 independent loads per thread in flight.
__global__ __launch_bounds__(256) void act_absmax_kernel(const uint4* __restrict__ x, int64_t n16,
                                                         float* __restrict__ part) {
  __shared__ float red[4];
  const int64_t G = gridDim.x;
  const int64_t per = (n16 + G - 1) / G;
  const int64_t begin = int64_t(blockIdx.x) * per;
  const int64_t end = begin + per < n16 ? begin + per : n16;
  float a = 0.f;
  int64_t i = begin + threadIdx.x;
  for (; i + 7 * 256 < end; i += 8 * 256) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = x[i + u * 256];
#pragma unroll
    for (int u = 0; u < 8; ++u) a = fmaxf(a, absmax8(v[u]));
  }
  for (; i < end; i += 256) a = fmaxf(a, absmax8(x[i]));
  a = block_max_256(a, red);
  if (threadIdx.x == 0) part[blockIdx.x] = a;
}

constexpr int kQuantPieces = 4;  // 16-byte pieces of x per thread in act_quant_kernel

// The codes of the two bf16 activations in `w` (low half first) into bytes
// 0-1 (HI false) or 2-3 (HI true) of `old`: x / s correctly rounded in
// float32, clamped to +-448 (the saturation; the clamp keeps the sign of
// -0), then the hardware's round-to-nearest-even conversion to E4M3FN.
template <bool HI>
__device__ __forceinline__ uint32_t act_code_pair(uint32_t old, uint32_t w, float s) {
  const float a = fminf(fmaxf(__fdiv_rn(bf16_lo(w), s), -448.0f), 448.0f);
  const float b = fminf(fmaxf(__fdiv_rn(bf16_hi(w), s), -448.0f), 448.0f);
  return uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, int(old), HI));
}

// Each workgroup: s_a from the G partial maxima, then kQuantPieces x 256
// consecutive pieces of x (8 activations each) -> 8 codes per piece.
__global__ __launch_bounds__(256) void act_quant_kernel(const uint4* __restrict__ x, int64_t n16,
                                                        const float* __restrict__ part, int G,
                                                        uint2* __restrict__ codes, float* __restrict__ scale_out) {
  __shared__ float red[4];
  const int64_t i0 = int64_t(blockIdx.x) * (256 * kQuantPieces) + threadIdx.x;
  uint4 v[kQuantPieces];
#pragma unroll
  for (int p = 0; p < kQuantPieces; ++p) {
    const int64_t i = i0 + p * 256;
    v[p] = x[i < n16 ? i : n16 - 1];
  }
  float pm = 0.f;
#pragma unroll
  for (int q = 0; q < kActQuantParts / 256; ++q) {
    const int t = threadIdx.x + 256 * q;
    if (t < G) pm = fmaxf(pm, part[t]);
  }
  const float a = block_max_256(pm, red);
  float s = __fdiv_rn(a, 448.0f);
  s = fmaxf(s, 0x1p-126f);
  if (a == 0.f) s = 1.0f;
  if (blockIdx.x == 0 && threadIdx.x == 0) *scale_out = s;
#pragma unroll
  for (int p = 0; p < kQuantPieces; ++p) {
    const int64_t i = i0 + p * 256;
    if (i >= n16) break;
    const uint32_t u[4] = {v[p].x, v[p].y, v[p].z, v[p].w};
    // elements 2e, 2e + 1 of the piece are the halves of u[e]; code byte j is element j
    const uint32_t c0 = act_code_pair<true>(act_code_pair<false>(0u, u[0], s), u[1], s);
    const uint32_t c1 = act_code_pair<true>(act_code_pair<false>(0u, u[2], s), u[3], s);
    codes[i] = make_uint2(c0, c1);
  }
}

hipError_t launch_act_quant(const void* x, int64_t M, int64_t K, int parts, void* codes, float* scale,
                            float* ws_part, hipStream_t st) {
  const int64_t n16 = M * K / 8;
  hipLaunchKernelGGL(act_absmax_kernel, dim3(unsigned(parts)), dim3(256), 0, st, reinterpret_cast<const uint4*>(x),
                     n16, ws_part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(act_quant_kernel, dim3(unsigned(ceil_div(n16, int64_t(256) * kQuantPieces))), dim3(256), 0, st,
                     reinterpret_cast<const uint4*>(x), n16, ws_part, parts, reinterpret_cast<uint2*>(codes), scale);
  return hipGetLastError();
}

// ------------------------------------------------------------------ the product
struct W8Args {
  const uint8_t* xc;     // activation codes [M][K]
  const float* xscale;   // s_a (device, one float)
  uint16_t* y;
  float* part;           // split partials [S][M][N] (S > 1)
  const uint4* w;
  const float* scales;   // s_n
  int64_t M, N, K, KT, NB;
  int NBN, MB, nchunks, cps, S;
};

template <int MF, int WR>
struct W8T {
  static constexpr int RB = 4;            // weight row blocks per wavefront
  static constexpr int WN = 4;            // wavefronts along N: 256 columns
  static constexpr int NW = WR * WN;      // wavefronts per workgroup
  static constexpr int XB = MF * WR;      // x row blocks per workgroup
  static constexpr int FRAGS = 2 * XB;    // 1 KiB fragment halves per chunk
  static constexpr int XPW = FRAGS / NW;  // of which each wavefront stages
  static constexpr int BUF = FRAGS * 64;  // uint4 per stage buffer
  // 128 accumulator registers leave room for two stages of weights only
  static constexpr int NS = MF >= 8 ? 2 : 3;
  static_assert(XPW >= 1 && XPW * NW == FRAGS, "whole fragment halves per wavefront");
};

template <int MF, int WR>
struct W8State {
  using T = W8T<MF, WR>;
  uint4 w[T::NS][T::RB][2];  // weights of chunks c .. c + NS - 1
  w8_f32x4_t acc[MF][T::RB];
  __amdgpu_buffer_rsrc_t wres[T::RB], xres;
  int64_t kt0, m0, nb0;
  int lane, wave, wm;
};

__device__ __forceinline__ void w8_dma(__amdgpu_buffer_rsrc_t r, uint4* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, voff, 0, 0, 0);
}

// x codes of chunk c into buf: this wavefront's halves f = wave XPW + u;
// half f is (x row block i = f / 2, h = f % 2).  Rows past M and k past K are
// outside the resource and write nothing (the buffer then holds zeros or an
// earlier chunk's codes of the same row, always finite, against zero weights).
template <int MF, int WR>
__device__ __forceinline__ void w8_load_x(W8State<MF, WR>& st, const W8Args& a, int c, uint4* buf) {
  using T = W8T<MF, WR>;
  const int g = st.lane >> 4, j = st.lane & 15;
#pragma unroll
  for (int u = 0; u < T::XPW; ++u) {
    const int f = st.wave * T::XPW + u, i = f >> 1, h = f & 1;
    const int64_t row = st.m0 + 16 * i + j;
    const int64_t k = (st.kt0 + 2 * int64_t(c)) * 64 + 16 * g + 64 * h;
    const uint32_t off = row < a.M && k < a.K ? uint32_t(row * a.K + k) : 0x80000000u;
    w8_dma(st.xres, buf + f * 64, off);
  }
}

// Weights of chunk c (tiles 2c, 2c + 1 of the split) into set H; tiles past
// the split are out of range and read zeros.
template <int MF, int WR, int H>
__device__ __forceinline__ void w8_load_w(W8State<MF, WR>& st, int c) {
  using T = W8T<MF, WR>;
#pragma unroll
  for (int b = 0; b < T::RB; ++b)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      // default cache policy: every x row block of the column block reads them
      const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(st.wres[b], st.lane * 16, (2 * c + t) * kTileBytes, 0);
      st.w[H][b][t] = make_uint4(v.x, v.y, v.z, v.w);
    }
}

template <int MF, int WR, int H>
__device__ __forceinline__ void w8_load_group(W8State<MF, WR>& st, const W8Args& a, int c, uint4* buf) {
  w8_load_x<MF, WR>(st, a, c, buf);
  __builtin_amdgcn_sched_barrier(0);
  w8_load_w<MF, WR, H>(st, c);
}

__device__ __forceinline__ void w8_wait_all() {
  __builtin_amdgcn_s_waitcnt(0x7 << 4);  // vmcnt(0) lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// End of step c: this wavefront's x of chunk c + 1 has landed once at most N
// later loads are in flight (chunk c + 1's weights, then whole groups of the
// chunks after it), and its LDS reads of chunk c are done; then meet the
// other wavefronts at a bare barrier.
template <int MF, int WR>
__device__ __forceinline__ void w8_wait_step() {
  using T = W8T<MF, WR>;
  constexpr int N = 2 * T::RB + (T::NS - 2) * (T::XPW + 2 * T::RB);
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | ((N >> 4) << 14));  // vmcnt(N) lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int MF, int WR, int H>
__device__ __forceinline__ void w8_compute(W8State<MF, WR>& st, const uint4* buf) {
  using T = W8T<MF, WR>;
#pragma unroll
  for (int i = 0; i < MF; ++i) {
    const int xb = st.wm * MF + i;
    const uint4 a0 = buf[(2 * xb) * 64 + st.lane];
    const uint4 a1 = buf[(2 * xb + 1) * 64 + st.lane];
#pragma unroll
    for (int b = 0; b < T::RB; ++b) st.acc[i][b] = w8_mfma(a0, a1, st.w[H][b][0], st.w[H][b][1], st.acc[i][b]);
  }
}

// Step for chunk c = NS it + H: request chunk c + NS - 1 into the buffer of
// chunk c - 1 (released at the last barrier), multiply chunk c, wait for
// chunk c + 1.  The steps after the loop (TAIL) request nothing.
template <int MF, int WR, int H, bool TAIL = false>
__device__ __forceinline__ void w8_step(W8State<MF, WR>& st, const W8Args& a, uint4* const* s_x, int c) {
  constexpr int NS = W8T<MF, WR>::NS;
  constexpr int HL = (H + NS - 1) % NS;
  if constexpr (!TAIL) w8_load_group<MF, WR, HL>(st, a, c + NS - 1, s_x[HL]);
  __builtin_amdgcn_sched_barrier(0);
  w8_compute<MF, WR, H>(st, s_x[H]);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (TAIL)
    w8_wait_all();
  else
    w8_wait_step<MF, WR>();
}

template <int MF, int WR>
__global__ __launch_bounds__((64 * W8T<MF, WR>::NW)) void w8_gemm_kernel(W8Args a) {
  using T = W8T<MF, WR>;
  constexpr int NS = T::NS;
  __shared__ uint4 s_x0[T::BUF], s_x1[T::BUF], s_x2[NS > 2 ? T::BUF : 1];
  uint4* const s_x[3] = {s_x0, s_x1, s_x2};

  // XCD-aware order: the workgroups of one XCD sweep the row blocks of x of
  // one column block back to back (dispatch is round-robin over the 8 XCDs)
  const int Lb = blockIdx.x, xcd = Lb & 7, wi = Lb >> 3;
  const int nbn = (wi / a.MB) * 8 + xcd, mb = wi % a.MB;
  if (nbn >= a.NBN) return;  // whole workgroup, before any barrier

  W8State<MF, WR> st;
  st.lane = threadIdx.x & 63;
  st.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  st.wm = st.wave / T::WN;
  const int wn = st.wave % T::WN;
  const int split = blockIdx.y;
  const int c0 = split * a.cps;
  const int nch = a.nchunks - c0 < a.cps ? a.nchunks - c0 : a.cps;  // >= 1: the planner sizes S so
  st.kt0 = 2 * int64_t(c0);
  st.m0 = int64_t(mb) * 16 * MF * WR;
  const int64_t tiles = a.KT - st.kt0 < 2 * int64_t(nch) ? a.KT - st.kt0 : 2 * int64_t(nch);
  st.nb0 = int64_t(nbn) * 16 + wn * T::RB;
#pragma unroll
  for (int b = 0; b < T::RB; ++b) {
    const bool live = st.nb0 + b < a.NB;
    const int64_t nb = live ? st.nb0 + b : 0;
    st.wres[b] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint4*>(a.w + (nb * a.KT + st.kt0) * (kTileBytes / 16)),
                                                   0, live ? uint32_t(tiles) * kTileBytes : 0u, 0x00020000);
#pragma unroll
    for (int i = 0; i < MF; ++i) st.acc[i][b] = w8_f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  st.xres = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.xc), 0, 0x7FFFFFF0, 0x00020000);

  // the stage buffers start as zeros (lanes out of range write nothing)
#pragma unroll
  for (int h = 0; h < NS; ++h)
    for (int i = threadIdx.x; i < T::BUF; i += 64 * T::NW) s_x[h][i] = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();
  w8_load_group<MF, WR, 0>(st, a, 0, s_x[0]);
  if constexpr (NS > 2) w8_load_group<MF, WR, 1>(st, a, 1, s_x[1]);
  __syncthreads();
  int c = 0;
  for (; c + NS <= nch; c += NS) {
    w8_step<MF, WR, 0>(st, a, s_x, c);
    w8_step<MF, WR, 1>(st, a, s_x, c + 1);
    if constexpr (NS > 2) w8_step<MF, WR, 2 % NS>(st, a, s_x, c + 2);
  }
  const int rest = nch - c;
  if (rest > 0) w8_step<MF, WR, 0, true>(st, a, s_x, c);
  if constexpr (NS > 2) {
    if (rest > 1) w8_step<MF, WR, 1, true>(st, a, s_x, c + 1);
  }

  // lane (g, n) holds rows 4 g + r of each x row block, column n of each row block
  const float sa = *a.xscale;
  const int g = st.lane >> 4, n = st.lane & 15;
#pragma unroll
  for (int b = 0; b < T::RB; ++b) {
    const int64_t col = (st.nb0 + b) * kTileRows + n;
    if (st.nb0 + b >= a.NB || col >= a.N) continue;
    const float cs = a.S == 1 ? a.scales[col] : 1.f;
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = st.m0 + (st.wm * MF + i) * 16 + 4 * g + r;
        if (row >= a.M) continue;
        const float v = st.acc[i][b][r] * sa;
        if (a.S > 1)
          a.part[(int64_t(split) * a.M + row) * a.N + col] = v;
        else
          a.y[row * a.N + col] = uint16_t(f32_to_bf16_rne(v * cs));
      }
  }
}

// ------------------------------------------------------------------ the product, LDS-staged form
// For wide verify batches: both operands of a 128-k chunk go from memory
// straight into one LDS stage (16-byte loads that write LDS, every
// wavefront issuing its share), so every operand byte crosses from memory to
// the compute unit once per workgroup.  A workgroup of 8 wavefronts computes
// a tile of WRM wavefront rows of 64 rows by 8 / WRM wavefront columns of RBW
// weight row blocks (256 x 256, 256 x 224 or 128 x 448); a stage holds the
// tile's weight slots (two packed tiles per row block, the B operand's
// halves; slots past the tile's row blocks lie outside the weight resource,
// so their loads read nothing) and its x fragment halves.  Two stages: at the
// start of chunk c the loads of chunk c + 1 are issued into the stage of
// chunk c - 1 (released at the last barrier), the chunk's operands are read
// from its stage and multiplied, and each wavefront then waits for its loads
// and meets the others at a bare barrier.  K is a whole number of chunks.
template <int RBW, int WRM>
struct W8L {
  static constexpr int WN = 8 / WRM;              // wavefront columns
  static constexpr int XR = 4 * WRM;              // x row blocks per tile
  static constexpr int XH = 2 * XR;               // x fragment halves per chunk
  static constexpr int NWS = 2 * WN * RBW;        // weight slots in use
  static constexpr int LPW = (NWS + XH + 7) / 8;  // loads per wavefront and chunk
  static constexpr int DX = XH / 8;               // of which x
  static constexpr int DW = LPW - DX;             // of which weights
  static constexpr int WS = 8 * DW;               // weight slots per stage
  static constexpr int BUF = (WS + XH) * 64;      // uint4 per stage
  static_assert(XH % 8 == 0 && WS >= NWS && 2 * BUF * 16 <= 160 * 1024, "stage layout");
};

template <int RBW, int WRM>
struct W8LState {
  using T = W8L<RBW, WRM>;
  w8_f32x4_t acc[4][RBW];
  __amdgpu_buffer_rsrc_t wres, xres;
  uint32_t wvo[T::DW], xvo[T::DX];
  int64_t c0;
  int lane, wave, wm, wn;
};

__device__ __forceinline__ void w8l_dma(__amdgpu_buffer_rsrc_t r, uint4* dst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, voff, soff, 0, 0);
}

// All loads of chunk c of the split into buf: this wavefront's weight slots,
// then its x halves; the chunk's part of every address is a scalar offset.
template <int RBW, int WRM>
__device__ __forceinline__ void w8l_load_chunk(const W8LState<RBW, WRM>& st, int c, uint4* buf) {
  using T = W8L<RBW, WRM>;
  const uint32_t ch = uint32_t(st.c0) + uint32_t(c);
#pragma unroll
  for (int u = 0; u < T::DW; ++u) w8l_dma(st.wres, buf + (T::DW * st.wave + u) * 64, st.wvo[u], ch * 2 * kTileBytes);
#pragma unroll
  for (int u = 0; u < T::DX; ++u) w8l_dma(st.xres, buf + (T::WS + T::DX * st.wave + u) * 64, st.xvo[u], ch * 128);
}

template <int N>
__device__ __forceinline__ void w8l_wait_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | ((N >> 4) << 14));  // vmcnt(N) lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Chunk c = (loop body start) + H, in stage H: request chunk c + 1 (if the
// split has one) into the other stage, multiply chunk c, wait for chunk
// c + 1 and meet the others.
template <int H, int RBW, int WRM>
__device__ __forceinline__ void w8l_chunk(W8LState<RBW, WRM>& st, uint4* const* sb, int c, int nch) {
  using T = W8L<RBW, WRM>;
  if (c + 1 < nch) w8l_load_chunk(st, c + 1, sb[1 - H]);
  const uint4* buf = sb[H];
  uint4 a[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h) a[i][h] = buf[(T::WS + 2 * (4 * st.wm + i) + h) * 64 + st.lane];
#pragma unroll
  for (int b = 0; b < RBW; ++b) {
    const int rb = RBW * st.wn + b;
    const uint4 b0 = buf[(2 * rb) * 64 + st.lane], b1 = buf[(2 * rb + 1) * 64 + st.lane];
#pragma unroll
    for (int i = 0; i < 4; ++i) st.acc[i][b] = w8_mfma(a[i][0], a[i][1], b0, b1, st.acc[i][b]);
  }
  __builtin_amdgcn_sched_barrier(0);
  w8l_wait_barrier<0>();
}

template <int RBW, int WRM>
__global__ __launch_bounds__(512) void w8_lds_kernel(W8Args a) {
  using T = W8L<RBW, WRM>;
  __shared__ uint4 s0[T::BUF], s1[T::BUF];
  uint4* const sb[2] = {s0, s1};
  // XCD-aware order: the workgroups of one XCD sweep the row blocks of x of
  // one column block back to back
  const int Lb = blockIdx.x, xcd = Lb & 7, wi = Lb >> 3;
  const int nbn = (wi / a.MB) * 8 + xcd, mb = wi % a.MB;
  if (nbn >= a.NBN) return;  // whole workgroup, before any barrier

  W8LState<RBW, WRM> st;
  st.lane = threadIdx.x & 63;
  st.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  st.wm = st.wave % WRM;
  st.wn = st.wave / WRM;
  const int split = blockIdx.y;
  const int c0 = split * a.cps;
  const int nch = a.nchunks - c0 < a.cps ? a.nchunks - c0 : a.cps;  // >= 1: the planner sizes S so
  st.c0 = c0;
  const int64_t nb0 = int64_t(nbn) * (T::WN * RBW), m0 = int64_t(mb) * (64 * WRM);
  const int64_t nbl = a.NB - nb0 < T::WN * RBW ? a.NB - nb0 : T::WN * RBW;
  st.wres = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint4*>(a.w + nb0 * a.KT * (kTileBytes / 16)), 0,
                                              uint32_t(nbl * a.KT * kTileBytes), 0x00020000);
  st.xres = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.xc), 0, uint32_t(a.M * a.K), 0x00020000);
  {
    const int g = st.lane >> 4, j = st.lane & 15;
#pragma unroll
    for (int u = 0; u < T::DW; ++u) {
      // slot q: tile q % 2 of the chunk of the tile's weight row block q / 2
      const int q = T::DW * st.wave + u;
      st.wvo[u] = uint32_t((q / 2) * a.KT * kTileBytes + (q % 2) * kTileBytes) + st.lane * 16;
    }
#pragma unroll
    for (int u = 0; u < T::DX; ++u) {
      // half f = (x row block i, h): lane (g, j) holds the codes k = 16 g ..
      // 16 g + 15 (h = 0) or 64 + 16 g .. (h = 1) of the chunk of row 16 i + j
      const int f = T::DX * st.wave + u, i = f / 2, h = f % 2;
      const int64_t row = m0 + 16 * i + j;
      st.xvo[u] = row < a.M ? uint32_t(row * a.K + 16 * g + 64 * h) : 0x80000000u;
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int b = 0; b < RBW; ++b) st.acc[i][b] = w8_f32x4_t{0.f, 0.f, 0.f, 0.f};
  // the stages start as zeros (lanes out of range write nothing)
#pragma unroll
  for (int h = 0; h < 2; ++h)
    for (int i = threadIdx.x; i < T::BUF; i += 512) sb[h][i] = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();

  w8l_load_chunk(st, 0, sb[0]);
  w8l_wait_barrier<0>();
  int c = 0;
  for (; c + 2 <= nch; c += 2) {
    w8l_chunk<0>(st, sb, c, nch);
    w8l_chunk<1>(st, sb, c + 1, nch);
  }
  if (c < nch) w8l_chunk<0>(st, sb, c, nch);

  // lane (g, n) holds rows 4 g + r of each x row block, column n of each row block
  const float sa = *a.xscale;
  const int g = st.lane >> 4, n = st.lane & 15;
#pragma unroll
  for (int b = 0; b < RBW; ++b) {
    const int64_t nb = nb0 + RBW * st.wn + b;
    const int64_t col = nb * kTileRows + n;
    if (nb >= a.NB || col >= a.N) continue;
    const float cs = a.S == 1 ? a.scales[col] : 1.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = m0 + (4 * st.wm + i) * 16 + 4 * g + r;
        if (row >= a.M) continue;
        const float v = st.acc[i][b][r] * sa;
        if (a.S > 1)
          a.part[(int64_t(split) * a.M + row) * a.N + col] = v;
        else
          a.y[row * a.N + col] = uint16_t(f32_to_bf16_rne(v * cs));
      }
  }
}

template <int MF, int WR>
static void launch_w8_tile(const W8Args& a, const W8Plan& p, hipStream_t st) {
  const unsigned grid = unsigned(ceil_div(p.NBN, 8) * 8 * p.MB);
  hipLaunchKernelGGL((w8_gemm_kernel<MF, WR>), dim3(grid, unsigned(p.S)), dim3(64 * W8T<MF, WR>::NW), 0, st, a);
}

hipError_t launch_w8a8(const W8Plan& p, const void* xc, const float* xscale, int64_t M, int64_t N, int64_t K,
                       const void* wp, const void* scales, void* y, void* ws, hipStream_t st) {
  W8Args a;
  a.xc = reinterpret_cast<const uint8_t*>(xc);
  a.xscale = xscale;
  a.y = reinterpret_cast<uint16_t*>(y);
  a.part = reinterpret_cast<float*>(ws);
  a.w = reinterpret_cast<const uint4*>(wp);
  a.scales = reinterpret_cast<const float*>(scales);
  a.M = M;
  a.N = N;
  a.K = K;
  a.KT = p.KT;
  a.NB = p.NB;
  a.NBN = int(p.NBN);
  a.MB = int(p.MB);
  a.nchunks = int(p.nchunks);
  a.cps = int(p.cps);
  a.S = p.S;
  if (p.lds) {
    if (K != p.nchunks * 128 || !((p.rbw == 8 && p.lwr == 4) || (p.rbw == 7 && (p.lwr == 4 || p.lwr == 2))) ||
        p.NBN != ceil_div(p.NB, int64_t(8 / p.lwr * p.rbw)) || p.MB != ceil_div(M, int64_t(64 * p.lwr)))
      return hipErrorInvalidValue;
    const dim3 grid(unsigned(ceil_div(p.NBN, int64_t(8)) * 8 * p.MB), unsigned(p.S));
    if (p.lwr == 2)
      hipLaunchKernelGGL((w8_lds_kernel<7, 2>), grid, dim3(512), 0, st, a);
    else if (p.rbw == 7)
      hipLaunchKernelGGL((w8_lds_kernel<7, 4>), grid, dim3(512), 0, st, a);
    else
      hipLaunchKernelGGL((w8_lds_kernel<8, 4>), grid, dim3(512), 0, st, a);
  } else if (p.wr == 1 && p.mf == 8)
    launch_w8_tile<8, 1>(a, p, st);
  else if (p.wr == 1 && p.mf == 4)
    launch_w8_tile<4, 1>(a, p, st);
  else if (p.wr == 1 && p.mf == 2)
    launch_w8_tile<2, 1>(a, p, st);
  else
    return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.S == 1) return e;
  return launch_splitk_reduce(kFmtFP8, a.part, p.S, M, N, scales, y, false, st);
}

}  // namespace wqd
