// Tiled matrix-core kernel with both operands staged in LDS, for BF16
// weights at wide verify batches (a few hundred activation rows and up):
// y = x . dequant(W)^T as a dense contraction ("Making each token cheaper",
// the lab on verify width: the layer multiplies batch x (k + 1) rows, and
// from about a hundred rows the matrix cores, not HBM, set the time).
//
// Why a second tiled kernel: in the one that takes weights straight from
// memory into registers (wqd_gemm.hip), both wavefront rows of a 256-row
// tile fetch every weight fragment, and the fetch path, not the matrix
// cores, sets its pace.  Here a workgroup of 8 wavefronts computes a
// 256 x 256 tile of y, and every operand byte of a K chunk crosses from
// memory to the compute unit once:
//   * a chunk is one packed tile along K (32 k): the 16 weight fragments of
//     the tile's 256 weight rows (each the packed 1 KiB tile, already in
//     B-operand order) and the 16 x fragments of its 256 rows (1 KiB each,
//     lane 16 kb + j holding the 8 k of row j that pair with slice kb of the
//     weights) go from memory straight into one LDS stage (16-byte loads
//     that write LDS, each wavefront issuing its share);
//   * wavefront (wm, wn) owns 64 rows x 128 columns of the tile: per chunk it
//     reads 4 x fragments and 8 weight fragments from LDS and issues 32
//     v_mfma_f32_16x16x32_bf16;
//   * operands are double-buffered in registers: while a chunk's multiplies
//     run, the next chunk's fragments are read from LDS, spread between them
//     (measured on gate at 1024 rows: all operand traffic from memory to the
//     compute unit, not the multiplies or the LDS reads, sets the pace);
//   * 4 LDS stages of 32 KiB (one array each, so that reads of one stage do not wait
//     for loads into another): at the start of chunk c the loads of chunk
//     c + NS - 1 are issued; at its end each wavefront waits until its loads
//     of chunk c + 2 have landed (loads complete in issue order, so the count
//     of later loads is exact) and a bare barrier follows;
//   * split-K over grid y when the tiles alone leave compute units idle; the
//     float32 partials go to the workspace and the fixed-order split-K sum
//     finishes them.
// Every load is unconditional: rows past M, weight row blocks past N and k
// past K lie outside their buffer resources (or get an out-of-range offset)
// and read zero without touching memory; loads past a split's last chunk
// fill stages that are never multiplied.
#include "wqd_device.h"
#include "wqd_internal.h"
#include "wqd_plan.h"

namespace wqd {

typedef __bf16 gl_bf16x8_t __attribute__((ext_vector_type(8)));
typedef float gl_f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ gl_f32x4_t gl_mfma(uint4 a, uint4 b, gl_f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(gl_bf16x8_t, a),
                                                 __builtin_bit_cast(gl_bf16x8_t, b), c, 0, 0, 0);
}

struct GlArgs {
  const uint16_t* x;
  uint16_t* y;
  float* part;  // split partials [S][M][N] (S > 1)
  const uint4* w;
  int64_t M, N, K, KT, NB;
  int NBN, MB;  // 256-column blocks, 256-row blocks
  int cps;      // chunks (tiles along K) per split
  int S;
  int swiglu;
};

// BF16 only: FP8 weights in this form (64-k chunks, three 48 KiB stages)
// measured slower than the tiled kernel that takes them into registers.
struct GlF {
  static constexpr int TK = 32;            // K per packed tile = per chunk
  static constexpr int SLK = TK / 4;       // K per lane slice of a tile
  static constexpr int BUF = (16 + 16) * 64;  // uint4 per LDS stage: weight then x fragments
  static constexpr int DX = 2;             // x loads per wavefront and chunk
  static constexpr int DPC = 2 + DX;       // loads per wavefront and chunk
  static constexpr int NS = 4;             // stages (128 KiB of LDS)
};

template <int RBW>
struct GlState {
  gl_f32x4_t acc[4][RBW];  // [x row block][weight row block]
  uint4 w[2][RBW];         // weight fragments of the current and the next chunk
  uint4 x[2][4];         // x fragments of the current and the next chunk
  __amdgpu_buffer_rsrc_t wres, xres;
  uint32_t wvo[2];         // this lane's byte offsets of its two weight loads (chunk 0 of the matrix)
  uint32_t xvo[GlF::DX];   // this lane's byte offsets of its x loads (chunk 0; out of range past M)
  int64_t kt0;
  int lane, wave, wm, wn;
};

// 16 bytes per lane from r into LDS: lane i's bytes land at dst + 16 i.
__device__ __forceinline__ void gl_dma(__amdgpu_buffer_rsrc_t r, uint4* dst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, voff, soff, 0, 0);
}

// All loads of chunk c of the split into buf: this wavefront's two weight
// fragments (row blocks 2 w, 2 w + 1), then its two x fragments (row blocks
// 2 w, 2 w + 1).  The chunk's part of each address is a scalar offset (K is
// a whole number of tiles on this kernel's shapes, so no x piece of a chunk
// inside the matrix lies past K; chunks past the matrix read weights of the
// next row block, or nothing past the last one, into stages that are never
// multiplied).
template <int RBW>
__device__ __forceinline__ void gl_load_chunk(const GlState<RBW>& st, int c, uint4* buf) {
  const uint32_t kt = uint32_t(st.kt0) + uint32_t(c);
#pragma unroll
  for (int u = 0; u < 2; ++u) gl_dma(st.wres, buf + (2 * st.wave + u) * 64, st.wvo[u], kt * kTileBytes);
#pragma unroll
  for (int u = 0; u < GlF::DX; ++u)
    gl_dma(st.xres, buf + (16 + GlF::DX * st.wave + u) * 64, st.xvo[u], kt * (GlF::TK * 2));
}

// The operands of the chunk in buf into set H: weight fragments of row blocks
// 8 wn .. 8 wn + 7, x fragments of row blocks 4 wm .. 4 wm + 3.
template <int H, int RBW>
__device__ __forceinline__ void gl_read_ops(GlState<RBW>& st, const uint4* buf) {
#pragma unroll
  for (int b = 0; b < RBW; ++b) st.w[H][b] = buf[(RBW * st.wn + b) * 64 + st.lane];
#pragma unroll
  for (int i = 0; i < 4; ++i) st.x[H][i] = buf[(16 + 4 * st.wm + i) * 64 + st.lane];
}

// The 32 multiplies of the operands in set H.
template <int H, int RBW>
__device__ __forceinline__ void gl_mfmas(GlState<RBW>& st) {
#pragma unroll
  for (int b = 0; b < RBW; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) st.acc[i][b] = gl_mfma(st.x[H][i], st.w[H][b], st.acc[i][b]);
}

template <int N>
__device__ __forceinline__ void gl_wait_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | ((N >> 4) << 14));  // vmcnt(N) lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Chunk c = (loop body start) + H of the split, its operands in set H % 2:
// issue the loads of chunk c + NS - 1 (into the stage of chunk c - 1,
// released by the last barrier), multiply while reading chunk c + 1's
// operands (landed before the last barrier) into the other set, then wait
// for chunk c + 2 and meet the other wavefronts.
template <int H, int RBW>
__device__ __forceinline__ void gl_chunk(GlState<RBW>& st, uint4* const* sb, int c) {
  constexpr int NS = GlF::NS, P = H % 2;
  gl_load_chunk(st, c + NS - 1, sb[(H + NS - 1) % NS]);
  gl_read_ops<1 - P>(st, sb[(H + 1) % NS]);
  gl_mfmas<P>(st);
  // spread the RBW + 4 LDS reads and 4 loads over the 4 RBW multiplies (left
  // to itself the scheduler reads the next operands into the registers of the
  // current ones after their last multiply, and waits for them at once)
  static_assert(RBW >= 7 && RBW <= 8, "pattern for 7 or 8 weight row blocks");
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // 2 MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, RBW - 6, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // 1 load into LDS
  }
  __builtin_amdgcn_sched_barrier(0);
  gl_wait_barrier<GlF::DPC * (NS - 3)>();
}

template <int RBW>
__global__ __launch_bounds__(512) void gemm_lds_kernel(GlArgs a) {
  constexpr int NS = GlF::NS;
  __shared__ uint4 s0[GlF::BUF], s1[GlF::BUF], s2[GlF::BUF], s3[GlF::BUF];
  uint4* const sb[4] = {s0, s1, s2, s3};

  // XCD-aware order: the workgroups of one XCD sweep the row blocks of x of
  // one column block back to back, so its weights are fetched into that
  // XCD's L2 once
  const int Lb = blockIdx.x, xcd = Lb & 7, wi = Lb >> 3;
  const int nbn = (wi / a.MB) * 8 + xcd, mb = wi % a.MB;
  if (nbn >= a.NBN) return;  // whole workgroup, before any barrier

  GlState<RBW> st;
  st.lane = threadIdx.x & 63;
  st.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  st.wm = st.wave & 3;
  st.wn = st.wave >> 2;
  const int split = blockIdx.y;
  const int c0 = split * a.cps;
  const int nch = int(a.KT) - c0 < a.cps ? int(a.KT) - c0 : a.cps;  // >= 1: the planner sizes S so
  st.kt0 = c0;
  const int64_t nb0 = int64_t(nbn) * (2 * RBW), m0 = int64_t(mb) * 256;
  // the tile's 2 RBW weight row blocks (slots past them, and row blocks past
  // the matrix, are out of range: their loads read nothing)
  const int64_t nbl = a.NB - nb0 < 2 * RBW ? a.NB - nb0 : 2 * RBW;
  st.wres = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint4*>(a.w + nb0 * a.KT * (kTileBytes / 16)), 0,
                                              uint32_t(nbl * a.KT * kTileBytes), 0x00020000);
  st.xres = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.x), 0, uint32_t(a.M * a.K * 2), 0x00020000);
  {
    const int kb = st.lane >> 4, j = st.lane & 15;
#pragma unroll
    for (int u = 0; u < 2; ++u) st.wvo[u] = uint32_t((2 * st.wave + u) * a.KT * kTileBytes) + st.lane * 16;
#pragma unroll
    for (int u = 0; u < GlF::DX; ++u) {
      // x row block i: lane (kb, j) holds the 8 k of row 16 i + j that pair
      // with slice kb of the weight tile; rows past M are out of range
      const int64_t row = m0 + 16 * (GlF::DX * st.wave + u) + j;
      st.xvo[u] = row < a.M ? uint32_t((row * a.K + kb * GlF::SLK) * 2) : 0x80000000u;
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int b = 0; b < RBW; ++b) st.acc[i][b] = gl_f32x4_t{0.f, 0.f, 0.f, 0.f};

  // the stages start as zeros: lanes out of range of their resource may leave
  // their LDS bytes unwritten (those bytes then only ever hold zeros)
#pragma unroll
  for (int h = 0; h < NS; ++h)
    for (int i = threadIdx.x; i < GlF::BUF; i += 512) sb[h][i] = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();

  // prologue: chunks 0 .. NS - 2 requested; chunk 0's operands in set 0,
  // chunk 1 landed
#pragma unroll
  for (int h = 0; h < NS - 1; ++h) gl_load_chunk(st, h, sb[h]);
  gl_wait_barrier<GlF::DPC * (NS - 2)>();
  gl_read_ops<0>(st, sb[0]);
  gl_wait_barrier<GlF::DPC * (NS - 3)>();

  // loop bodies of NS chunks (stage and register-set indices compile-time),
  // then the split's last nch % NS chunks one by one
  int c = 0;
  for (; c + NS <= nch; c += NS) {
    gl_chunk<0>(st, sb, c);
    gl_chunk<1>(st, sb, c + 1);
    gl_chunk<2>(st, sb, c + 2);
    gl_chunk<3>(st, sb, c + 3);
  }
  const int rest = nch - c;
  if (rest > 0) gl_chunk<0>(st, sb, c);
  if (rest > 1) gl_chunk<1>(st, sb, c + 1);
  if (rest > 2) gl_chunk<2>(st, sb, c + 2);
  __builtin_amdgcn_s_waitcnt(0x7 << 4);  // vmcnt(0) lgkmcnt(0): no load into LDS outlives the workgroup

  // lane (kb, n) holds rows 4 kb + r of each x row block, column n of each weight row block
  const int kb = st.lane >> 4, n = st.lane & 15;
#pragma unroll
  for (int b = 0; b < RBW; ++b) {
    const int64_t nb = nb0 + RBW * st.wn + b;
    const int64_t col = nb * kTileRows + n;
    if (nb >= a.NB || col >= a.N) continue;  // the same for lanes n and n ^ 8 (N % 16 == 0 with SwiGLU)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = m0 + (4 * st.wm + i) * 16 + 4 * kb + r;
        if (row >= a.M) continue;  // the same for lanes n and n ^ 8
        if (a.S > 1)
          a.part[(int64_t(split) * a.M + row) * a.N + col] = st.acc[i][b][r];
        else
          store_out<8>(a.y, a.N, a.swiglu, row, col, st.acc[i][b][r], true);  // lane ^ 8: column ^ 8
      }
  }
}

// ---------------------------------------------------------------- FP8 weights
// The same tile and wavefront layout, 256 columns (RBW = 8 weight row blocks
// per wavefront) or 224 (RBW = 7, where those fill the compute units' rounds
// better: the loads of the two unused weight slots lie outside the weight
// resource and read nothing); a chunk is one packed FP8 tile along K
// (64 k, two matrix-core steps): 16 weight fragments (one per row block,
// bytes 8 s .. 8 s + 7 of each lane's 16 codes are step s's 8 k) and 32 x
// fragments (row block i, step s) in one 48 KiB stage, 3 stages.  With three
// stages a chunk's operands are read from LDS at its start (no register copy
// of the next chunk), so that each wavefront waits at the end of chunk c for
// its loads of chunk c + 1, issued a whole chunk earlier.
struct GlF8 {
  static constexpr int TK = 64;
  static constexpr int BUF = 48 * 64;  // uint4 per stage: weight slots, then x fragments
  static constexpr int DPC = 6;        // loads per wavefront and chunk
  static constexpr int NS = 3;
};

// Tile shapes: WRM wavefront rows of 64 rows (4: 256-row tiles, 2: 128-row
// tiles) by 8 / WRM wavefront columns of RBW weight row blocks.  A stage holds
// WS weight slots (the tile's WN RBW row blocks, the rest out of range) and
// the 2 XR x fragments of the tile's rows, filled by DW weight and DX x loads
// per wavefront.
template <int RBW, int WRM>
struct GlT8 {
  static constexpr int WN = 8 / WRM;
  static constexpr int XR = 4 * WRM;         // x row blocks per tile
  static constexpr int DX = XR / 4;          // x loads per wavefront and chunk (XR blocks x 2 steps)
  static constexpr int DW = GlF8::DPC - DX;  // weight loads per wavefront and chunk
  static constexpr int WS = 8 * DW;          // weight slots per stage
  static_assert(WN * RBW <= WS && (WS + 2 * XR) * 64 == GlF8::BUF, "stage layout");
};

template <int RBW, int WRM>
struct GlState8 {
  using T = GlT8<RBW, WRM>;
  gl_f32x4_t acc[4][RBW];
  uint4 w[RBW];
  uint4 x[2][4];  // steps 0 and 1
  __amdgpu_buffer_rsrc_t wres, xres;
  uint32_t wvo[T::DW];
  uint32_t xvo[T::DX];
  int64_t kt0;
  int lane, wave, wm, wn;
};

template <int RBW, int WRM>
__device__ __forceinline__ void gl8_load_chunk(const GlState8<RBW, WRM>& st, int c, uint4* buf) {
  using T = GlT8<RBW, WRM>;
  const uint32_t kt = uint32_t(st.kt0) + uint32_t(c);
#pragma unroll
  for (int u = 0; u < T::DW; ++u) gl_dma(st.wres, buf + (T::DW * st.wave + u) * 64, st.wvo[u], kt * kTileBytes);
#pragma unroll
  for (int u = 0; u < T::DX; ++u)
    gl_dma(st.xres, buf + (T::WS + T::DX * st.wave + u) * 64, st.xvo[u], kt * (GlF8::TK * 2));
}

template <int S, int RBW, int WRM>
__device__ __forceinline__ void gl8_read_x(GlState8<RBW, WRM>& st, const uint4* buf) {
  using T = GlT8<RBW, WRM>;
#pragma unroll
  for (int i = 0; i < 4; ++i) st.x[S][i] = buf[(T::WS + (4 * st.wm + i) * 2 + S) * 64 + st.lane];
}

template <int S, int RBW, int WRM>
__device__ __forceinline__ void gl8_mfmas(GlState8<RBW, WRM>& st) {
#pragma unroll
  for (int b = 0; b < RBW; ++b) {
    const uint4 wv = st.w[b];
    const uint32_t w0 = S == 0 ? wv.x : wv.z, w1 = S == 0 ? wv.y : wv.w;
    const uint4 bm = make_uint4(__builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<false>(w0)),
                                __builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<true>(w0)),
                                __builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<false>(w1)),
                                __builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<true>(w1)));
#pragma unroll
    for (int i = 0; i < 4; ++i) st.acc[i][b] = gl_mfma(st.x[S][i], bm, st.acc[i][b]);
  }
}

// Chunk c = (loop body start) + H: issue the loads of chunk c + 2 (into the
// stage of chunk c - 1), read this chunk's weights and step-0 x, multiply
// step 0 while reading step 1's x, multiply step 1, then wait for chunk c + 1
// and meet the other wavefronts.
template <int H, int RBW, int WRM>
__device__ __forceinline__ void gl8_chunk(GlState8<RBW, WRM>& st, uint4* const* sb, int c) {
  constexpr int NS = GlF8::NS;
  gl8_load_chunk(st, c + NS - 1, sb[(H + NS - 1) % NS]);
  const uint4* buf = sb[H % NS];
#pragma unroll
  for (int b = 0; b < RBW; ++b) st.w[b] = buf[(RBW * st.wn + b) * 64 + st.lane];
  gl8_read_x<0>(st, buf);
  gl8_read_x<1>(st, buf);
  gl8_mfmas<0>(st);
  gl8_mfmas<1>(st);
  __builtin_amdgcn_sched_barrier(0);
  gl_wait_barrier<GlF8::DPC * (NS - 2)>();
}

template <int RBW, int WRM>
__global__ __launch_bounds__(512) void gemm_lds8_kernel(GlArgs a, const float* __restrict__ scales) {
  using T = GlT8<RBW, WRM>;
  constexpr int NS = GlF8::NS;
  __shared__ uint4 s0[GlF8::BUF], s1[GlF8::BUF], s2[GlF8::BUF];
  uint4* const sb[3] = {s0, s1, s2};
  const int Lb = blockIdx.x, xcd = Lb & 7, wi = Lb >> 3;
  const int nbn = (wi / a.MB) * 8 + xcd, mb = wi % a.MB;
  if (nbn >= a.NBN) return;

  GlState8<RBW, WRM> st;
  st.lane = threadIdx.x & 63;
  st.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  st.wm = st.wave % WRM;
  st.wn = st.wave / WRM;
  const int split = blockIdx.y;
  const int c0 = split * a.cps;
  const int nch = int(a.KT) - c0 < a.cps ? int(a.KT) - c0 : a.cps;
  st.kt0 = c0;
  // the tile's WN RBW weight row blocks (slots past them, and row blocks past
  // the matrix, are out of range of the resource: their loads read nothing
  // and their LDS slots are never multiplied)
  const int64_t nb0 = int64_t(nbn) * (T::WN * RBW), m0 = int64_t(mb) * (64 * WRM);
  const int64_t nbl = a.NB - nb0 < T::WN * RBW ? a.NB - nb0 : T::WN * RBW;
  st.wres = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint4*>(a.w + nb0 * a.KT * (kTileBytes / 16)), 0,
                                              uint32_t(nbl * a.KT * kTileBytes), 0x00020000);
  st.xres = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.x), 0, uint32_t(a.M * a.K * 2), 0x00020000);
  {
    const int kb = st.lane >> 4, j = st.lane & 15;
#pragma unroll
    for (int u = 0; u < T::DW; ++u) st.wvo[u] = uint32_t((T::DW * st.wave + u) * a.KT * kTileBytes) + st.lane * 16;
#pragma unroll
    for (int u = 0; u < T::DX; ++u) {
      // fragment f = (x row block i, step s): lane (kb, j) holds the 8 k of
      // row 16 i + j that pair with bytes 8 s .. 8 s + 7 of weight slice kb
      const int f = T::DX * st.wave + u, i = f / 2, sx = f % 2;
      const int64_t row = m0 + 16 * i + j;
      st.xvo[u] = row < a.M ? uint32_t((row * a.K + kb * 16 + 8 * sx) * 2) : 0x80000000u;
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int b = 0; b < RBW; ++b) st.acc[i][b] = gl_f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int h = 0; h < NS; ++h)
    for (int i = threadIdx.x; i < GlF8::BUF; i += 512) sb[h][i] = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();

  // prologue: chunks 0 and 1 requested, chunk 0 landed
  gl8_load_chunk(st, 0, sb[0]);
  gl8_load_chunk(st, 1, sb[1]);
  gl_wait_barrier<GlF8::DPC>();
  int c = 0;
  for (; c + NS <= nch; c += NS) {
    gl8_chunk<0>(st, sb, c);
    gl8_chunk<1>(st, sb, c + 1);
    gl8_chunk<2>(st, sb, c + 2);
  }
  const int rest = nch - c;
  if (rest > 0) gl8_chunk<0>(st, sb, c);
  if (rest > 1) gl8_chunk<1>(st, sb, c + 1);
  __builtin_amdgcn_s_waitcnt(0x7 << 4);

  const int kb = st.lane >> 4, n = st.lane & 15;
#pragma unroll
  for (int b = 0; b < RBW; ++b) {
    const int64_t nb = nb0 + RBW * st.wn + b;
    const int64_t col = nb * kTileRows + n;
    if (nb >= a.NB || col >= a.N) continue;
    const float cs = a.S == 1 ? scales[col] : 1.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = m0 + (4 * st.wm + i) * 16 + 4 * kb + r;
        if (row >= a.M) continue;
        if (a.S > 1)
          a.part[(int64_t(split) * a.M + row) * a.N + col] = st.acc[i][b][r];
        else
          store_out<8>(a.y, a.N, a.swiglu, row, col, st.acc[i][b][r] * cs, true);
      }
  }
}

hipError_t launch_gemm_lds(int fmt, const GmPlan& p, const void* x, int64_t M, int64_t N, int64_t K, const void* wp,
                           const void* scales, void* y, void* part, bool swiglu, hipStream_t st) {
  if (p.wm != 3 || (fmt != kFmtBF16 && fmt != kFmtFP8) || K != p.KT * (fmt == kFmtFP8 ? GlF8::TK : GlF::TK))
    return hipErrorInvalidValue;
  // tiles of 64 lwr rows by (8 / lwr) rbw weight row blocks: BF16 256 x 256,
  // FP8 256 x 256, 256 x 224 or 128 x 448
  const bool shape_ok = fmt == kFmtBF16 ? ((p.rbw == 8 || p.rbw == 7) && p.lwr == 4)
                                        : ((p.rbw == 8 && p.lwr == 4) || (p.rbw == 7 && (p.lwr == 4 || p.lwr == 2)));
  if (!shape_ok || p.NBN != ceil_div(p.NB, int64_t(8 / p.lwr * p.rbw)) || p.MB != ceil_div(M, int64_t(64 * p.lwr)))
    return hipErrorInvalidValue;
  GlArgs a;
  a.x = reinterpret_cast<const uint16_t*>(x);
  a.y = reinterpret_cast<uint16_t*>(y);
  a.part = reinterpret_cast<float*>(part);
  a.w = reinterpret_cast<const uint4*>(wp);
  a.M = M;
  a.N = N;
  a.K = K;
  a.KT = p.KT;
  a.NB = p.NB;
  a.NBN = int(p.NBN);
  a.MB = int(p.MB);
  a.cps = int(p.cps);
  a.S = p.S;
  a.swiglu = swiglu;
  const dim3 grid(unsigned(ceil_div(p.NBN, int64_t(8)) * 8 * p.MB), unsigned(p.S));
  const float* sc = reinterpret_cast<const float*>(scales);
  if (fmt == kFmtFP8 && p.lwr == 4 && p.rbw == 7)
    hipLaunchKernelGGL((gemm_lds8_kernel<7, 4>), grid, dim3(512), 0, st, a, sc);
  else if (fmt == kFmtFP8 && p.lwr == 4)
    hipLaunchKernelGGL((gemm_lds8_kernel<8, 4>), grid, dim3(512), 0, st, a, sc);
  else if (fmt == kFmtFP8)
    hipLaunchKernelGGL((gemm_lds8_kernel<7, 2>), grid, dim3(512), 0, st, a, sc);
  else if (p.rbw == 7)
    hipLaunchKernelGGL(gemm_lds_kernel<7>, grid, dim3(512), 0, st, a);
  else
    hipLaunchKernelGGL(gemm_lds_kernel<8>, grid, dim3(512), 0, st, a);
  return hipGetLastError();
}

}  // namespace wqd
