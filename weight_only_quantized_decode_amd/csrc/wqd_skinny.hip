// Skinny matrix-core decode kernel for 9 to 64 activation rows:
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
//     wavefront does everything else;
//   * the producer stages x per chunk of CT tiles in LDS (NX = 3 buffers)
//     with direct-to-LDS buffer loads, already in matrix-core fragment order:
//     fragment (tile t, row block of x i, K-step s) is 1 KiB, lane
//     16 kb + j holding the 8 k of activation row 16 i + j that the bf16
//     instruction v_mfma_f32_16x16x32_bf16 pairs with slice kb of the weight
//     tile, read back by the consumers as one conflict-free 16-byte LDS read
//     per lane.  Rows at or past M read zeros (out-of-range buffer offsets)
//     and only feed output rows that are never stored;
//   * W4A16: the producer also stages the fp16 scales and uint4 zero points
//     of the workgroup's row blocks (one 4-group quad at a time) and computes
//     X = x . 1 per tile with the all-ones B operand, so that a tile
//     contributes s * (P - (128 + z) * X) with P = x . (128 + q) from the
//     consumers' identical chain of matrix-core steps (q == z == 0 cancels
//     exactly).  Consumers thus issue nothing but weight loads: their in-order
//     load counter holds weights only, so the arithmetic waits for exactly the
//     tile it needs;
//   * the producer works one chunk ahead: between the barriers that open
//     chunks c - 1 and c it computes X of chunk c (landed) and issues the
//     loads of chunk c + 1;
//   * consumers keep R weight tiles per row block in a register ring, R - 1
//     of them in flight (loads past the range are out of range of their
//     buffer resource: no traffic, zeros; the tile offset rides in the scalar
//     offset, so a load costs no vector arithmetic); the loop body is one
//     ring (a whole number of chunks), so every ring slot is a compile-time
//     constant;
//   * FP8 codes convert exactly to bf16 and the row scale is applied once at
//     the end; BF16 feeds the matrix cores as loaded;
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

typedef __attribute__((address_space(3))) void* sk_lds_ptr;

struct SkArgs {
  const uint16_t* x;
  uint16_t* y;
  float* part;  // split partials [S][M][N] (S > 1)
  const uint4* w;
  const void* scales;
  const uint16_t* zeros;
  int64_t M, N, K, KT, G4, NB;
  int per_split;  // tiles per split, a multiple of the ring size and of 4
  int S;
  int swiglu;     // packed gate/up pairs: store silu(gate) * up (store_out)
};

template <int FMT>
struct SkF {
  static constexpr int TK = FMT == kFmtBF16 ? 32 : FMT == kFmtFP8 ? 64 : 128;  // K per tile
  static constexpr int SLK = TK / 4;                                             // K per slice
  static constexpr int STEPS = SLK / 8;  // 32-k matrix-core steps per tile
};

// LDS layout, in uint4 units: NX x chunks, then (W4A16) NX x-sum buffers
// (16 bytes per tile, x row block and slice) and 3 scale / zero quad buffers
// (BR = WN * RB row blocks x 16 rows: 8 bytes of scales, 2 of zeros; room
// for a whole number of 8-row-block groups, one staging load each).
template <int FMT, int MF, int CT, int NX, int BR>
struct SkL {
  static constexpr int FRAGS = CT * MF * SkF<FMT>::STEPS;  // 1 KiB fragments per chunk
  static constexpr int XBUF = FRAGS * 64;
  static constexpr int SBUF = CT * MF * 4;
  static constexpr int QG = (BR + 7) / 8;  // groups of 8 row blocks
  static constexpr int QS = QG * 64, QZ = QG * 16, QBUF = QS + QZ;
  static constexpr int X0 = 0, XS0 = NX * XBUF, Q0 = XS0 + (FMT == kFmtW4 ? NX * SBUF : 0);
  static constexpr int TOTAL = Q0 + (FMT == kFmtW4 ? 3 * QBUF : 0);
};

template <int FMT, int MF, int RB, int R>
struct SkState {
  uint4 w[R][RB];  // ring of R weight tiles per row block
  sk_f32x4_t acc[MF][RB];
  __amdgpu_buffer_rsrc_t wres[RB];
  const uint4* xb;      // LDS: x fragments of the current chunk
  const uint4* xs;      // LDS: x sums of the current chunk
  const uint16_t* sq;   // LDS: scale quads of the current chunk's quad, [BR][16][4] fp16
  const uint16_t* zq;   // LDS: zero quads, [BR][16] (4 nibbles)
  int lane, rbl, total;  // rbl: this wavefront's first row block inside the workgroup
};

template <int FMT, int MF, int RB, int R, int SLOT>
__device__ __forceinline__ void sk_load(SkState<FMT, MF, RB, R>& st, int T) {
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    // cache policy 2: non-temporal (weights are read once per step)
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(st.wres[b], st.lane * 16, T * kTileBytes, 2);
    st.w[SLOT][b] = make_uint4(v.x, v.y, v.z, v.w);
  }
}

// Multiply tile T in ring slot SLOT: tile SLOT % CT of the current chunk.
template <int FMT, int MF, int RB, int R, int CT, int SLOT>
__device__ __forceinline__ void sk_compute(SkState<FMT, MF, RB, R>& st, int T) {
  using F = SkF<FMT>;
  constexpr int t = SLOT % CT;
  const int kb = st.lane >> 4, n = st.lane & 15;
  const uint4* xf = st.xb + (t * MF) * F::STEPS * 64 + st.lane;  // fragment (t, i, s) at xf[(i * STEPS + s) * 64]
  if constexpr (FMT == kFmtW4) {
    const uint32_t mask = vgpr_const(0x000F000Fu), magic = vgpr_const(0x43004300u);
    sk_f32x4_t P[MF][RB];
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
      for (int b = 0; b < RB; ++b) P[i][b] = sk_f32x4_t{0.f, 0.f, 0.f, 0.f};
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
#pragma unroll
        for (int b = 0; b < RB; ++b) P[i][b] = sk_mfma(af, bm[b], P[i][b]);
      }
    }
    // splits start on a scale quad and R is a multiple of 4, so the tile's
    // place in its quad is SLOT % 4; tiles past the range get scale 0
    const bool live = T < st.total;
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      const int row = (st.rbl + b) * 16 + n;
      const float s0 = __half2float(__ushort_as_half(st.sq[row * kScaleQuad + SLOT % kScaleQuad]));
      const float sc = live ? s0 : 0.f;
      const float zc = 128.0f + float((uint32_t(st.zq[row]) >> (4 * (SLOT % kScaleQuad))) & 0xFu);
#pragma unroll
      for (int i = 0; i < MF; ++i) {
        const uint4 xq = st.xs[(t * MF + i) * 4 + kb];
        const sk_f32x4_t X = __builtin_bit_cast(sk_f32x4_t, xq);
#pragma unroll
        for (int r = 0; r < 4; ++r) st.acc[i][b][r] = fmaf(sc, fmaf(-zc, X[r], P[i][b][r]), st.acc[i][b][r]);
      }
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
// T - 1 has freed, then multiplies tile T.  Tiles past the range load zeros
// and multiply to zero (W4A16: scale 0).
template <int FMT, int MF, int RB, int R, int CT, int NX, int BR, int I>
__device__ __forceinline__ void sk_steps(SkState<FMT, MF, RB, R>& st, uint4* lds, int T0) {
  using L = SkL<FMT, MF, CT, NX, BR>;
  if constexpr (I < R) {
    const int T = T0 + I;
    if constexpr (I % CT == 0) {
      __syncthreads();  // chunk T / CT staged; everyone is done with the buffers it replaces
      const int c = T / CT, xbuf = c % NX;
      st.xb = lds + L::X0 + xbuf * L::XBUF;
      if constexpr (FMT == kFmtW4) {
        st.xs = lds + L::XS0 + xbuf * L::SBUF;
        const uint4* qb = lds + L::Q0 + ((T / kScaleQuad) % 3) * L::QBUF;
        st.sq = reinterpret_cast<const uint16_t*>(qb);
        st.zq = reinterpret_cast<const uint16_t*>(qb + L::QS);
      }
    }
    sk_load<FMT, MF, RB, R, (I + R - 1) % R>(st, T + R - 1);
    // keep the loads here: left to itself the scheduler sinks them to just
    // before their use, which would leave nothing in flight during the math
    __builtin_amdgcn_sched_barrier(0);
    sk_compute<FMT, MF, RB, R, CT, I>(st, T);
    sk_steps<FMT, MF, RB, R, CT, NX, BR, I + 1>(st, lds, T0);
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

// Producer: issue the direct-to-LDS loads of chunk c (tiles kt0 + c CT ..):
// its x fragments and, when it starts a scale quad, the workgroup's scale
// and zero quads.
template <int FMT, int MF, int CT, int NX, int BR>
__device__ __forceinline__ void sk_stage(const SkArgs& a, __amdgpu_buffer_rsrc_t xres, __amdgpu_buffer_rsrc_t sres,
                                         __amdgpu_buffer_rsrc_t zres, uint4* lds, int64_t kt0, int c, int64_t nbw,
                                         int lane) {
  using F = SkF<FMT>;
  using L = SkL<FMT, MF, CT, NX, BR>;
  const int kb = lane >> 4, j = lane & 15;
  const int64_t kt = kt0 + int64_t(c) * CT;
  uint4* xb = lds + L::X0 + (c % NX) * L::XBUF;
#pragma unroll
  for (int f = 0; f < L::FRAGS; ++f) {
    const int t = f / (MF * F::STEPS), i = (f / F::STEPS) % MF, s = f % F::STEPS;
    const int64_t row = 16 * i + j;
    const int64_t k = (kt + t) * F::TK + kb * F::SLK + 8 * s;
    const uint32_t off = row < a.M && k < a.K ? uint32_t((row * a.K + k) * 2) : 0x80000000u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(xres, (sk_lds_ptr)(xb + f * 64), 16, off, 0, 0, 0);
  }
  if constexpr (FMT == kFmtW4) {
    if ((c * CT) % kScaleQuad == 0) {
      const int64_t q = kt / kScaleQuad;
      uint4* qb = lds + L::Q0 + (int((c * CT) / kScaleQuad) % 3) * L::QBUF;
#pragma unroll
      for (int h = 0; h < L::QG; ++h) {
        // lane l: row block 8 h + l / 8 of the workgroup, rows 2 (l % 8) and 2 (l % 8) + 1
        const int rb = 8 * h + (lane >> 3);
        const int64_t nb = nbw + rb, r0 = (lane & 7) * 2;
        const int64_t e = (nb * a.G4 + q) * kTileRows + r0;  // (row block, quad, row) element
        const bool ok = rb < BR && nb < a.NB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(sres, (sk_lds_ptr)(qb + 64 * h), 16, ok ? uint32_t(e * 8) : 0x80000000u,
                                                 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(zres, (sk_lds_ptr)(qb + L::QS + 16 * h), 4,
                                                 ok ? uint32_t(e * 2) : 0x80000000u, 0, 0, 0);
      }
    }
  }
}

// Producer (W4A16): X = x . 1 of every tile and x row block of chunk c, by the
// same chain of matrix-core steps the consumers use for P; lanes 16 kb store
// rows 4 kb .. 4 kb + 3.
template <int FMT, int MF, int CT, int NX, int BR>
__device__ __forceinline__ void sk_xsums(uint4* lds, int c, int lane) {
  using L = SkL<FMT, MF, CT, NX, BR>;
  const uint4* xb = lds + L::X0 + (c % NX) * L::XBUF + lane;
  uint4* xs = lds + L::XS0 + (c % NX) * L::SBUF;
  const uint4 ones = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);
#pragma unroll
  for (int t = 0; t < CT; ++t)
#pragma unroll
    for (int i = 0; i < MF; ++i) {
      sk_f32x4_t X = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) X = sk_mfma(xb[((t * MF + i) * 4 + s) * 64], ones, X);
      if ((lane & 15) == 0) xs[(t * MF + i) * 4 + (lane >> 4)] = __builtin_bit_cast(uint4, X);
    }
}

template <int FMT, int MF, int RB, int WN, int R, int CT, int NX>
__global__ __launch_bounds__(64 * (WN + 1)) void gemv_sk_kernel(SkArgs a) {
  constexpr int BR = WN * RB;
  using L = SkL<FMT, MF, CT, NX, BR>;
  static_assert(R % CT == 0 && R % 4 == 0 && NX == 3 && (FMT != kFmtW4 || kScaleQuad % CT == 0),
                "ring, chunk and buffer counts");
  __shared__ uint4 lds[L::TOTAL];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int split = blockIdx.y;
  const int64_t kt0 = int64_t(split) * a.per_split;
  const int64_t rem = a.KT - kt0;
  const int total = rem < a.per_split ? int(rem) : a.per_split;  // >= 1: the planner sizes S so
  const int nbody = (total + R - 1) / R;
  const int nch = nbody * (R / CT);
  const int64_t nbw = int64_t(blockIdx.x) * BR;  // the workgroup's first row block

  if (wave == WN) {
    // producer.  Between the barriers that open chunks c - 1 and c: wait for
    // chunk c (the only loads in flight), compute its x sums, issue chunk c + 1
    // into the buffers of chunk c - 2 (free: the consumers are on c - 1)
    const __amdgpu_buffer_rsrc_t xres =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.x), 0, 0x7FFFFFF0, 0x00020000);
    __amdgpu_buffer_rsrc_t sres = xres, zres = xres;
    if constexpr (FMT == kFmtW4) {
      sres = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.scales), 0,
                                               uint32_t(a.NB * a.G4 * kTileRows * kScaleQuad * 2), 0x00020000);
      zres = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.zeros), 0, uint32_t(a.NB * a.G4 * kTileRows * 2),
                                               0x00020000);
    }
    sk_stage<FMT, MF, CT, NX, BR>(a, xres, sres, zres, lds, kt0, 0, nbw, lane);
    // chunk 0 is requested before the consumers' weights, which would
    // otherwise queue ahead of it and leave them waiting for x
    asm volatile("s_barrier" ::: "memory");
    for (int c = 0; c < nch; ++c) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if constexpr (FMT == kFmtW4) sk_xsums<FMT, MF, CT, NX, BR>(lds, c, lane);
      if (c + 1 < nch) sk_stage<FMT, MF, CT, NX, BR>(a, xres, sres, zres, lds, kt0, c + 1, nbw, lane);
      // a bare barrier: __syncthreads() would add a release fence, which waits
      // for the direct-to-LDS loads of chunk c + 1 just issued
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
    return;
  }

  SkState<FMT, MF, RB, R> st;
  const int n = lane & 15, kb = lane >> 4;
  st.lane = lane;
  st.total = total;
  st.rbl = wave * RB;
  st.xb = st.xs = lds;
  st.sq = st.zq = reinterpret_cast<const uint16_t*>(lds);
  const int64_t nb0 = nbw + wave * RB;
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    // a row block past the matrix gets an empty resource: its loads read
    // zeros and its outputs are never stored
    const bool live = nb0 + b < a.NB;
    const int64_t nb = live ? nb0 + b : 0;
    st.wres[b] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint4*>(a.w + (nb * a.KT + kt0) * (kTileBytes / 16)), 0,
                                                   live ? uint32_t(total) * kTileBytes : 0u, 0x00020000);
#pragma unroll
    for (int i = 0; i < MF; ++i) st.acc[i][b] = sk_f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // prologue: tiles 0 .. R - 2 into slots 0 .. R - 2, in tile order (the
  // waits of the first loop pass assume it)
  asm volatile("s_barrier" ::: "memory");  // the producer has requested x of chunk 0
  sk_prologue<FMT, MF, RB, R, 0>(st);
  for (int it = 0; it < nbody; ++it) sk_steps<FMT, MF, RB, R, CT, NX, BR, 0>(st, lds, it * R);

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
        if (row >= a.M) continue;  // the same for lanes n and n ^ 8
        if (a.S > 1)
          a.part[(int64_t(split) * a.M + row) * a.N + col] = st.acc[i][b][r];
        else
          store_out<8>(a.y, a.N, a.swiglu, row, col, st.acc[i][b][r] * cs, true);  // lane ^ 8: column ^ 8
      }
  }
}

template <int FMT, int MF, int RB, int WN>
static hipError_t launch_sk_cfg(const SkArgs& a, const SkPlan& p, hipStream_t st) {
  constexpr int CT = (FMT == kFmtW4 && MF >= 2) || MF >= 3 ? 2 : 4;
  if (p.ring != 8 || p.ct != CT || p.nx != 3) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemv_sk_kernel<FMT, MF, RB, WN, 8, CT, 3>), dim3(unsigned(p.groups), unsigned(p.S)),
                     dim3(64 * (WN + 1)), 0, st, a);
  return hipGetLastError();
}

// Every configuration the planner chooses from (kSkCfg: consumers, weight row
// blocks per consumer), for 1 to 4 x row blocks.
template <int FMT, int MF, int I>
static hipError_t launch_sk_try(const SkArgs& a, const SkPlan& p, hipStream_t st) {
  if constexpr (I == kSkCfgCount) {
    return hipErrorInvalidValue;
  } else {
    constexpr int WN = kSkCfg[I][0], RB = kSkCfg[I][1];
    if (p.waves == WN && p.rb == RB) return launch_sk_cfg<FMT, MF, RB, WN>(a, p, st);
    return launch_sk_try<FMT, MF, I + 1>(a, p, st);
  }
}

template <int FMT>
static hipError_t launch_sk_fmt(const SkArgs& a, const SkPlan& p, hipStream_t st) {
  switch (p.mf) {
    case 1: return launch_sk_try<FMT, 1, 0>(a, p, st);
    case 2: return launch_sk_try<FMT, 2, 0>(a, p, st);
    case 3: return launch_sk_try<FMT, 3, 0>(a, p, st);
    case 4: return launch_sk_try<FMT, 4, 0>(a, p, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemv_sk(int fmt, const SkPlan& p, const void* x, int64_t M, int64_t N, int64_t K, const void* wp,
                          const void* scales, const void* zeros, void* y, void* ws, bool swiglu, hipStream_t st) {
  SkArgs a;
  a.swiglu = swiglu;
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
  return launch_splitk_reduce(fmt, a.part, p.S, M, N, scales, y, swiglu, st);
}

}  // namespace wqd
