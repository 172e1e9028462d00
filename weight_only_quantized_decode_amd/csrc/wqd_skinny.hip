// Skinny matrix-core decode kernel for 9 to 32 activation rows:
// y = x . dequant(W)^T.
//
// Between a handful of rows and the compute-bound verify widths the layer is
// still bound by the weight stream ("Making each token cheaper", sections
// "Speculative decoding" and the lab on verify width: each extra row adds
// work, not weight bytes), but x is now as large per tile as the weights
// (16 rows x 128 k x 2 bytes = 4 KiB of x per 1 KiB W4A16 tile), so it has to
// be read once per workgroup and shared, not re-read per tile by every
// wavefront.  Design for gfx950:
//   * a workgroup owns WN x RB consecutive 16-row blocks over a range of K.
//     WN consumer wavefronts each stream RB row blocks; one producer
//     wavefront stages x;
//   * x is staged per chunk of CT tiles in LDS (NX buffers: the producer
//     runs NX - 1 chunks ahead) by the producer
//     with direct-to-LDS buffer loads, already in matrix-core fragment order:
//     fragment (tile t, row block of x i, K-step s) is 1 KiB, lane
//     16 kb + j holding the 8 k of activation row 16 i + j that the bf16
//     instruction v_mfma_f32_16x16x32_bf16 pairs with slice kb of the weight
//     tile.  Consumers read it back as one conflict-free 16-byte LDS read
//     per lane.  Rows at or past M read zeros (out-of-range buffer offsets),
//     and only feed output rows that are never stored;
//   * the producer waits on its own load counter before each chunk barrier.
//     Consumers never issue x loads, so their in-order load counter holds
//     weights only and the arithmetic waits for exactly the tile it needs;
//   * consumers keep R weight tiles per row block in a register ring, R - 1
//     of them in flight (loads past the range are out of range of their
//     buffer resource: no traffic, zeros); the loop body is one ring (a whole
//     number of chunks), so every ring slot is a compile-time constant;
//   * products and dequantisation as in the streaming matrix-core kernel:
//     W4A16 nibble pairs become bf16 (128 + q) with one AND-OR, a tile
//     contributes s * (P - (128 + z) * X) with X = x . 1 from a chain of the
//     same shape (exact cancellation for q == z == 0); FP8 codes convert
//     exactly, the row scale is applied once at the end; BF16 feeds as is;
//   * when the row blocks alone give too few workgroups, K is split S ways
//     over grid y; the float32 partials go to the workspace and the fixed-order
//     split-K sum of the matrix-core path finishes them (deterministic, no
//     device-scope fences).
#include "wqd_device.h"
#include "wqd_internal.h"
#include "wqd_plan.h"

namespace wqd {

typedef __bf16 sk_bf16x8_t __attribute__((ext_vector_type(8)));
typedef float sk_f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ sk_f32x4_t sk_mfma(uint4 a, uint4 b, sk_f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(sk_bf16x8_t, a),
                                                 __builtin_bit_cast(sk_bf16x8_t, b), c, 0, 0, 0);
}

struct SkArgs {
  const uint16_t* x;
  uint16_t* y;
  float* part;  // split partials [S][M][N] (S > 1)
  const uint4* w;
  const void* scales;
  const uint16_t* zeros;
  int64_t M, N, K, KT, G4, NB;
  int per_split;  // tiles per split, a multiple of the ring size
  int S;
};

template <int FMT>
struct SkF {
  static constexpr int TK = FMT == kFmtBF16 ? 32 : FMT == kFmtFP8 ? 64 : 128;  // K per tile
  static constexpr int SLK = TK / 4;                                             // K per slice
  static constexpr int STEPS = SLK / 8;  // 32-k matrix-core steps per tile
};

template <int FMT, int MF, int CT>
struct SkL {
  static constexpr int FRAGS = CT * MF * SkF<FMT>::STEPS;  // 1 KiB fragments per chunk
  static constexpr int BUF = FRAGS * 64;                    // uint4 per LDS buffer
};

// Producer: stage the x fragments of tiles kt .. kt + CT - 1 into buf.
template <int FMT, int MF, int CT>
__device__ __forceinline__ void sk_stage(const SkArgs& a, __amdgpu_buffer_rsrc_t xres, uint4* buf, int64_t kt,
                                         int lane) {
  using F = SkF<FMT>;
  const int kb = lane >> 4, j = lane & 15;
#pragma unroll
  for (int f = 0; f < SkL<FMT, MF, CT>::FRAGS; ++f) {
    const int t = f / (MF * F::STEPS), i = (f / F::STEPS) % MF, s = f % F::STEPS;
    const int64_t row = 16 * i + j;
    const int64_t k = (kt + t) * F::TK + kb * F::SLK + 8 * s;
    const uint32_t off = row < a.M && k < a.K ? uint32_t((row * a.K + k) * 2) : 0x80000000u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(xres, (__attribute__((address_space(3))) void*)(buf + f * 64), 16, off,
                                             0, 0, 0);
  }
}

template <int FMT, int MF, int RB, int R>
struct SkState {
  uint4 w[R][RB];                 // ring of R weight tiles per row block
  uint32_t sw[R][RB], zw[R][RB];  // W4A16: fp16 scale bits and zero quad of the tile's group
  sk_f32x4_t acc[MF][RB];
  __amdgpu_buffer_rsrc_t wres[RB], sres[RB], zres[RB];
  const uint4* xb;      // LDS buffer of the current chunk
  uint32_t soff, zoff;  // this lane's byte offsets inside a scale / zero quad column
  int64_t kt0;
  int lane, total;
};

// Weights (and W4A16 scale / zero) of tile T into ring slot SLOT = T % R.
template <int FMT, int MF, int RB, int R, int SLOT>
__device__ __forceinline__ void sk_load(SkState<FMT, MF, RB, R>& st, int T) {
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    // cache policy 2: non-temporal (weights are read once per step)
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(st.wres[b], uint32_t(T) * kTileBytes + st.lane * 16, 0, 2);
    st.w[SLOT][b] = make_uint4(v.x, v.y, v.z, v.w);
    if constexpr (FMT == kFmtW4) {
      const int64_t kt = st.kt0 + T;
      const uint32_t q = uint32_t(kt / kScaleQuad);
      st.sw[SLOT][b] = __builtin_amdgcn_raw_buffer_load_b16(
          st.sres[b], (q * kTileRows) * (kScaleQuad * 2) + st.soff + uint32_t(kt % kScaleQuad) * 2, 0, 0);
      st.zw[SLOT][b] = __builtin_amdgcn_raw_buffer_load_b16(st.zres[b], q * (kTileRows * 2) + st.zoff, 0, 0);
    }
  }
}

// Multiply the tile in ring slot SLOT: tile SLOT % CT of the chunk in st.xb.
template <int FMT, int MF, int RB, int R, int CT, int SLOT>
__device__ __forceinline__ void sk_compute(SkState<FMT, MF, RB, R>& st) {
  using F = SkF<FMT>;
  constexpr int t = SLOT % CT;
  const uint4* xf = st.xb + (t * MF) * F::STEPS * 64 + st.lane;  // fragment (t, i, s) at xf[(i * STEPS + s) * 64]
  if constexpr (FMT == kFmtW4) {
    const uint32_t mask = vgpr_const(0x000F000Fu), magic = vgpr_const(0x43004300u);
    const uint4 ones = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);
    sk_f32x4_t X[MF], P[MF][RB];
#pragma unroll
    for (int i = 0; i < MF; ++i) {
      X[i] = sk_f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int b = 0; b < RB; ++b) P[i][b] = sk_f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint4 bm[RB];
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        const uint4 wv = st.w[SLOT][b];
        const uint32_t wd = s == 0 ? wv.x : s == 1 ? wv.y : s == 2 ? wv.z : wv.w;
        bm[b] = make_uint4(and_or_v(wd, mask, magic), and_or_v(wd >> 4, mask, magic), and_or_v(wd >> 8, mask, magic),
                           and_or_v(wd >> 12, mask, magic));
      }
#pragma unroll
      for (int i = 0; i < MF; ++i) {
        const uint4 af = xf[(i * 4 + s) * 64];
        X[i] = sk_mfma(af, ones, X[i]);
#pragma unroll
        for (int b = 0; b < RB; ++b) P[i][b] = sk_mfma(af, bm[b], P[i][b]);
      }
    }
    // splits start on a scale quad and R is a multiple of 4, so the tile's
    // place in its quad is SLOT % 4
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      const float sc = __half2float(__ushort_as_half(uint16_t(st.sw[SLOT][b])));
      const float zc = 128.0f + float((st.zw[SLOT][b] >> (4 * (SLOT % kScaleQuad))) & 0xFu);
#pragma unroll
      for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) st.acc[i][b][r] = fmaf(sc, fmaf(-zc, X[i][r], P[i][b][r]), st.acc[i][b][r]);
    }
  } else if constexpr (FMT == kFmtFP8) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      uint4 bm[RB];
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        const uint4 wv = st.w[SLOT][b];
        const uint32_t w0 = s == 0 ? wv.x : wv.z, w1 = s == 0 ? wv.y : wv.w;
        bm[b] = make_uint4(__builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<false>(w0)),
                           __builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<true>(w0)),
                           __builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<false>(w1)),
                           __builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<true>(w1)));
      }
#pragma unroll
      for (int i = 0; i < MF; ++i) {
        const uint4 af = xf[(i * 2 + s) * 64];
#pragma unroll
        for (int b = 0; b < RB; ++b) st.acc[i][b] = sk_mfma(af, bm[b], st.acc[i][b]);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < MF; ++i) {
      const uint4 af = xf[i * 64];
#pragma unroll
      for (int b = 0; b < RB; ++b) st.acc[i][b] = sk_mfma(af, st.w[SLOT][b], st.acc[i][b]);
    }
  }
}

// Steps I .. R - 1 of a loop body starting at tile T0.  Step T waits at the
// chunk barrier when T starts a chunk, loads tile T + R - 1 into the slot tile
// T - 1 has freed, then multiplies tile T; tiles past the range load zeros
// and are not multiplied.
template <int FMT, int MF, int RB, int R, int CT, int NX, int I>
__device__ __forceinline__ void sk_steps(SkState<FMT, MF, RB, R>& st, uint4* s_x, int T0) {
  if constexpr (I < R) {
    const int T = T0 + I;
    if constexpr (I % CT == 0) {
      __syncthreads();  // chunk T / CT staged; everyone is done with the buffer it replaces
      st.xb = s_x + ((T / CT) % NX) * SkL<FMT, MF, CT>::BUF;
    }
    sk_load<FMT, MF, RB, R, (I + R - 1) % R>(st, T + R - 1);
    // keep the loads here: left to itself the scheduler sinks them to just
    // before their use, which would leave nothing in flight during the math
    __builtin_amdgcn_sched_barrier(0);
    if (T < st.total) sk_compute<FMT, MF, RB, R, CT, I>(st);
    sk_steps<FMT, MF, RB, R, CT, NX, I + 1>(st, s_x, T0);
  }
}

template <int FMT, int MF, int RB, int R, int T>
__device__ __forceinline__ void sk_prologue(SkState<FMT, MF, RB, R>& st) {
  if constexpr (T < R - 1) {
    sk_load<FMT, MF, RB, R, T>(st, T);
    __builtin_amdgcn_sched_barrier(0);
    sk_prologue<FMT, MF, RB, R, T + 1>(st);
  }
}

// Producer wait: at most N loads of this wavefront still in flight.
template <int N>
__device__ __forceinline__ void sk_wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt holds 0 .. 63");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int FMT, int MF, int RB, int WN, int R, int CT, int NX>
__global__ __launch_bounds__(64 * (WN + 1)) void gemv_sk_kernel(SkArgs a) {
  using L = SkL<FMT, MF, CT>;
  static_assert(R % CT == 0 && R % 4 == 0 && NX >= 2 && NX <= 3, "ring, chunk and buffer counts");
  __shared__ uint4 s_x[NX * L::BUF];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int split = blockIdx.y;
  const int64_t kt0 = int64_t(split) * a.per_split;
  const int64_t rem = a.KT - kt0;
  const int total = rem < a.per_split ? int(rem) : a.per_split;  // >= 1: the planner sizes S so
  const int nbody = (total + R - 1) / R;
  const int nch = nbody * (R / CT);

  if (wave == WN) {
    // producer: chunks 0 .. NX - 2 up front, then chunk c + NX - 1 once
    // barrier c has freed the buffer of chunk c - 1
    const __amdgpu_buffer_rsrc_t xres =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.x), 0, 0x7FFFFFF0, 0x00020000);
    for (int q = 0; q < NX - 1 && q < nch; ++q) sk_stage<FMT, MF, CT>(a, xres, s_x + q * L::BUF, kt0 + q * CT, lane);
    for (int c = 0; c < nch; ++c) {
      // chunk c has landed before its barrier opens it (at most chunk c + 1,
      // issued later, is still in flight)
      if (NX == 3 && c + 1 < nch)
        sk_wait_vm<(NX - 2) * L::FRAGS>();
      else
        sk_wait_vm<0>();
      // a bare barrier: __syncthreads() would add a release fence, which waits
      // for every direct-to-LDS load in flight (the next chunk's included)
      asm volatile("s_barrier" ::: "memory");
      const int nc = c + NX - 1;
      if (nc < nch) sk_stage<FMT, MF, CT>(a, xres, s_x + (nc % NX) * L::BUF, kt0 + int64_t(nc) * CT, lane);
    }
    return;
  }

  SkState<FMT, MF, RB, R> st;
  const int n = lane & 15, kb = lane >> 4;
  st.lane = lane;
  st.total = total;
  st.kt0 = kt0;
  st.xb = s_x;
  const int64_t nb0 = (int64_t(blockIdx.x) * WN + wave) * RB;
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    // a row block past the matrix gets empty resources: its loads read zeros
    // and its outputs are never stored
    const bool live = nb0 + b < a.NB;
    const int64_t nb = live ? nb0 + b : 0;
    st.wres[b] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint4*>(a.w + (nb * a.KT + kt0) * (kTileBytes / 16)), 0,
                                                   live ? uint32_t(total) * kTileBytes : 0u, 0x00020000);
    if constexpr (FMT == kFmtW4) {
      const uint16_t* sb = reinterpret_cast<const uint16_t*>(a.scales) + nb * a.G4 * kTileRows * kScaleQuad;
      const uint16_t* zb = a.zeros + nb * a.G4 * kTileRows;
      st.sres[b] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(sb), 0,
                                                     live ? uint32_t(a.G4 * kTileRows * kScaleQuad * 2) : 0u,
                                                     0x00020000);
      st.zres[b] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(zb), 0,
                                                     live ? uint32_t(a.G4 * kTileRows * 2) : 0u, 0x00020000);
    }
#pragma unroll
    for (int i = 0; i < MF; ++i) st.acc[i][b] = sk_f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  st.soff = uint32_t(n) * (kScaleQuad * 2);
  st.zoff = uint32_t(n) * 2;

  // prologue: tiles 0 .. R - 2 into slots 0 .. R - 2, in tile order (the
  // waits of the first loop pass assume it)
  sk_prologue<FMT, MF, RB, R, 0>(st);
  for (int it = 0; it < nbody; ++it) sk_steps<FMT, MF, RB, R, CT, NX, 0>(st, s_x, it * R);

  // lane (kb, n) holds activation rows 16 i + 4 kb + r of column n of each block
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    const int64_t col = (nb0 + b) * kTileRows + n;
    if (nb0 + b >= a.NB || col >= a.N) continue;
    const float cs = FMT == kFmtFP8 && a.S == 1 ? reinterpret_cast<const float*>(a.scales)[col] : 1.f;
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = 16 * i + 4 * kb + r;
        if (row >= a.M) continue;
        if (a.S > 1)
          a.part[(int64_t(split) * a.M + row) * a.N + col] = st.acc[i][b][r];
        else
          a.y[row * a.N + col] = uint16_t(f32_to_bf16_rne(st.acc[i][b][r] * cs));
      }
  }
}

template <int FMT, int MF, int RB, int R, int CT, int NX>
static hipError_t launch_sk_cfg(const SkArgs& a, const SkPlan& p, hipStream_t st) {
  constexpr int WN = 4;
  if (p.waves != WN) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemv_sk_kernel<FMT, MF, RB, WN, R, CT, NX>), dim3(unsigned(p.groups), unsigned(p.S)),
                     dim3(64 * (WN + 1)), 0, st, a);
  return hipGetLastError();
}

// The configurations the planner chooses from (mf, rb, ring, chunk, buffers).
template <int FMT>
static hipError_t launch_sk_fmt(const SkArgs& a, const SkPlan& p, hipStream_t st) {
#define WQD_SK_CFG(MF, RB, R, CT, NX)                                                  \
  if (p.mf == MF && p.rb == RB && p.ring == R && p.ct == CT && p.nx == NX) \
    return launch_sk_cfg<FMT, MF, RB, R, CT, NX>(a, p, st);
  WQD_SK_CFG(1, 2, 8, 4, 3)
  WQD_SK_CFG(2, 2, 8, 4, 2)
#undef WQD_SK_CFG
  return hipErrorInvalidValue;
}

hipError_t launch_gemv_sk(int fmt, const SkPlan& p, const void* x, int64_t M, int64_t N, int64_t K, const void* wp,
                          const void* scales, const void* zeros, void* y, void* ws, hipStream_t st) {
  SkArgs a;
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
  a.G4 = fmt == kFmtW4 ? ceil_div(K / kGroup, kScaleQuad) : 0;
  a.NB = p.NB;
  a.per_split = p.per_split;
  a.S = p.S;
  hipError_t e;
  if (fmt == kFmtBF16)
    e = launch_sk_fmt<kFmtBF16>(a, p, st);
  else if (fmt == kFmtFP8)
    e = launch_sk_fmt<kFmtFP8>(a, p, st);
  else
    e = launch_sk_fmt<kFmtW4>(a, p, st);
  if (e != hipSuccess || p.S == 1) return e;
  return launch_splitk_reduce(fmt, a.part, p.S, M, N, scales, y, st);
}

}  // namespace wqd
