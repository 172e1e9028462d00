// Matrix-core decode kernel for M >= 9 activation rows: y = x . dequant(W)^T.
//
// At speculative-verify widths (M = batch x (k + 1), up to 1024 rows) the
// layer uses up the compute slack of a decode step and becomes a dense
// contraction ("Making each token cheaper", sections "Speculative decoding"
// and the lab on verify width; CS336 lecture 10 notes, 3.2-3.3: MLP
// arithmetic intensity grows with the batch).  This kernel runs it on the
// gfx950 bf16 matrix cores (v_mfma_f32_16x16x32_bf16), dequantising the
// weights on load:
//   * the packed 1 KiB tile (16 output rows x 4 slices x 16 bytes, lane
//     l = 16 kb + n) is already the MFMA B-operand order: lane l supplies
//     column n and K block kb.  BF16 tiles feed the matrix core as loaded;
//     FP8 codes go through the hardware E4M3 -> bf16 conversion (exact);
//     W4A16 nibble pairs become bf16 (128 + q) with one AND-OR.  A W4A16
//     tile carries 4 K-steps of 32: step s uses word s of every lane's
//     slice, and the A operand is read with the same K permutation;
//   * every W4A16 group (128 K = one tile) is accumulated on its own; its
//     zero point is removed with sum x, taken from an MFMA of the same x
//     fragments against an all-ones B (same instruction sequence, so
//     q == z == 0 cancels exactly), and its fp16 scale is applied in fp32:
//     acc += s * (acc_g - (128 + z) * sum x);  FP8 applies the row scale
//     once in the epilogue.  Dequantised weights are never rounded;
//   * x is staged per workgroup in LDS (double-buffered chunks, one barrier
//     per chunk); each wavefront streams its own 16 * BNT output columns
//     straight from HBM into registers, one chunk ahead;
//   * when the tiles alone give fewer than ~2 workgroups per compute unit,
//     K is split over workgroups (grid y); the float32 partial tiles go to
//     the caller's workspace and a second small kernel adds them in split
//     order.  Deterministic, and no device-scope fence is needed: the two
//     launches are ordered on the stream;
//   * XCD-aware dispatch: the workgroups of all M-blocks of one column block
//     go to the same XCD back to back (dispatch is round-robin over the 8
//     XCDs), so its weights are read from HBM once and then hit that XCD's L2.
#include "wqd_device.h"
#include "wqd_internal.h"
#include "wqd_plan.h"

namespace wqd {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

struct MfmaArgs {
  const uint16_t* x;
  uint16_t* y;
  const uint4* w;
  const void* scales;
  const uint16_t* zeros;
  float* part;  // split-K partials [S][M][N] (S > 1)
  int64_t M, N, K, NB, KT, G4;
  int NBB, MB;  // column blocks (4 waves x BNT tiles), M-blocks
  int S;        // K splits
  int64_t cps;  // chunks per split
  int swiglu;   // packed gate/up pairs: store silu(gate) * up (store_out)
};

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ f32x4_t mfma16(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

template <int FMT>
struct MfC {
  static constexpr int TK = FMT == kFmtBF16 ? 32 : FMT == kFmtFP8 ? 64 : 128;  // K per tile
  static constexpr int STEPS = TK / 32;                                          // MFMA K-steps per tile
};

// Chunk of x staged per barrier: 16 KiB (8 KiB for BF16), whole tiles.
template <int FMT, int BMS>
struct MfPlan {
  static constexpr int BM = 16 * BMS;
  static constexpr int raw = 8192 / (BM * MfC<FMT>::TK);
  static constexpr int TPC = raw > 8 ? 8 : (raw < 1 ? 1 : raw);  // tiles per chunk
  static constexpr int KC = TPC * MfC<FMT>::TK;                   // K per chunk
  static constexpr int ROWU = KC / 8 + 1;                         // uint4 per LDS row (+1: bank spread)
  static constexpr int XU = BM * (KC / 8);                        // uint4 of x per chunk
  static constexpr int XPT = (XU + 255) / 256;                    // uint4 each thread stages
};

template <int FMT, int BMS, int BNT>
__global__ __launch_bounds__(256) void mfma_kernel(MfmaArgs a) {
  using C = MfC<FMT>;
  using P = MfPlan<FMT, BMS>;
  constexpr int BM = P::BM, TPC = P::TPC, KC = P::KC, ROWU = P::ROWU;
  __shared__ uint4 s_x[2][BM * ROWU];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, kb = lane >> 4;
  // XCD-aware block order: consecutive workgroups of one XCD sweep the
  // M-blocks of one column block.
  const int L = blockIdx.x, xcd = L & 7, wi = L >> 3;
  const int nbb = (wi / a.MB) * 8 + xcd, mb = wi % a.MB;
  if (nbb >= a.NBB) return;  // whole workgroup, before any barrier
  const int64_t m0 = int64_t(mb) * BM;
  const int split = blockIdx.y;

  // this wavefront's tile rows (16 output columns each), clamped for loads
  int64_t nbj[BNT];
  bool colv[BNT];
#pragma unroll
  for (int j = 0; j < BNT; ++j) {
    const int64_t t = (int64_t(nbb) * 4 + wave) * BNT + j;
    colv[j] = t < a.NB;
    nbj[j] = colv[j] ? t : a.NB - 1;
  }

  f32x4_t acc[BMS][BNT];
#pragma unroll
  for (int i = 0; i < BMS; ++i)
#pragma unroll
    for (int j = 0; j < BNT; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // ---- staging helpers; this workgroup's K range is chunks [c_begin, c_end)
  const int64_t total_chunks = (a.K + KC - 1) / KC;
  const int64_t c_begin = int64_t(split) * a.cps;
  const int64_t c_end = min(total_chunks, c_begin + a.cps);
  uint4 xr[P::XPT];
  auto load_x = [&](int64_t c) {
#pragma unroll
    for (int u = 0; u < P::XPT; ++u) {
      const int idx = tid + 256 * u;
      const int r = idx / (KC / 8), col = idx % (KC / 8);
      const int64_t k = c * KC + int64_t(col) * 8;
      xr[u] = make_uint4(0, 0, 0, 0);
      if (idx < P::XU && m0 + r < a.M && k < a.K)
        xr[u] = *reinterpret_cast<const uint4*>(a.x + (m0 + r) * a.K + k);
    }
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int u = 0; u < P::XPT; ++u) {
      const int idx = tid + 256 * u;
      if (idx < P::XU) {
        const int r = idx / (KC / 8), col = idx % (KC / 8);
        s_x[buf][r * ROWU + col] = xr[u];
      }
    }
  };
  uint4 wcur[BNT][TPC], wnxt[BNT][TPC];
  uint32_t scur[BNT][TPC], snxt[BNT][TPC];  // W4A16: fp16 scale bits | zero << 16
  auto load_w = [&](int64_t c, uint4 (&wv)[BNT][TPC], uint32_t (&sv)[BNT][TPC]) {
#pragma unroll
    for (int j = 0; j < BNT; ++j)
#pragma unroll
      for (int t = 0; t < TPC; ++t) {
        const int64_t kt = min(c * TPC + t, a.KT - 1);
        wv[j][t] = load_nt(a.w + (nbj[j] * a.KT + kt) * (kTileBytes / 16) + lane);
        if (FMT == kFmtW4) {
          const int64_t q = (nbj[j] * a.G4 + kt / kScaleQuad) * kTileRows + n;
          const uint32_t sb = reinterpret_cast<const uint16_t*>(a.scales)[q * kScaleQuad + kt % kScaleQuad];
          const uint32_t zb = (uint32_t(a.zeros[q]) >> (4 * (kt % kScaleQuad))) & 0xFu;
          sv[j][t] = sb | (zb << 16);
        }
      }
  };

  // ---- prologue: first chunk staged, its weights in flight
  load_w(c_begin, wcur, scur);
  load_x(c_begin);
  store_x(0);
  __syncthreads();

  for (int64_t c = c_begin; c < c_end; ++c) {
    const int buf = int((c - c_begin) & 1);
    const bool more = c + 1 < c_end;
    if (more) {
      load_x(c + 1);
      load_w(c + 1, wnxt, snxt);
    }
    const uint4* xs = s_x[buf];
#pragma unroll
    for (int t = 0; t < TPC; ++t) {
      if (FMT == kFmtW4) {
        const uint32_t mask = vgpr_const(0x000F000Fu), magic = vgpr_const(0x43004300u);
        f32x4_t ag[BMS][BNT], xsum[BMS];
#pragma unroll
        for (int i = 0; i < BMS; ++i) {
          xsum[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int j = 0; j < BNT; ++j) ag[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        const uint4 ones = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          uint4 bf[BNT];
#pragma unroll
          for (int j = 0; j < BNT; ++j) {
            const uint32_t wd = s == 0 ? wcur[j][t].x : s == 1 ? wcur[j][t].y : s == 2 ? wcur[j][t].z : wcur[j][t].w;
            bf[j] = make_uint4(and_or_v(wd, mask, magic), and_or_v(wd >> 4, mask, magic),
                               and_or_v(wd >> 8, mask, magic), and_or_v(wd >> 12, mask, magic));
          }
#pragma unroll
          for (int i = 0; i < BMS; ++i) {
            // A: row 16 i + n, k = tile t, slice kb, step s  (uint4 index t*16 + 4 kb + s)
            const uint4 af = xs[(16 * i + n) * ROWU + t * 16 + 4 * kb + s];
            xsum[i] = mfma16(af, ones, xsum[i]);
#pragma unroll
            for (int j = 0; j < BNT; ++j) ag[i][j] = mfma16(af, bf[j], ag[i][j]);
          }
        }
#pragma unroll
        for (int j = 0; j < BNT; ++j) {
          const float sc = __half2float(__ushort_as_half(uint16_t(scur[j][t] & 0xFFFFu)));
          const float zc = 128.0f + float(scur[j][t] >> 16);
#pragma unroll
          for (int i = 0; i < BMS; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][j][r] = fmaf(sc, fmaf(-zc, xsum[i][r], ag[i][j][r]), acc[i][j][r]);
        }
      } else if (FMT == kFmtFP8) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          uint4 bf[BNT];
#pragma unroll
          for (int j = 0; j < BNT; ++j) {
            const uint32_t w0 = s == 0 ? wcur[j][t].x : wcur[j][t].z;
            const uint32_t w1 = s == 0 ? wcur[j][t].y : wcur[j][t].w;
            bf[j] = make_uint4(__builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<false>(w0)),
                               __builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<true>(w0)),
                               __builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<false>(w1)),
                               __builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<true>(w1)));
          }
#pragma unroll
          for (int i = 0; i < BMS; ++i) {
            // A: k = tile t, slice kb (16 k), half s  (uint4 index t*8 + 2 kb + s)
            const uint4 af = xs[(16 * i + n) * ROWU + t * 8 + 2 * kb + s];
#pragma unroll
            for (int j = 0; j < BNT; ++j) acc[i][j] = mfma16(af, bf[j], acc[i][j]);
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < BMS; ++i) {
          // A: k = tile t, slice kb (8 k)  (uint4 index t*4 + kb)
          const uint4 af = xs[(16 * i + n) * ROWU + t * 4 + kb];
#pragma unroll
          for (int j = 0; j < BNT; ++j) acc[i][j] = mfma16(af, wcur[j][t], acc[i][j]);
        }
      }
    }
    if (more) {
      store_x(buf ^ 1);
#pragma unroll
      for (int j = 0; j < BNT; ++j)
#pragma unroll
        for (int t = 0; t < TPC; ++t) {
          wcur[j][t] = wnxt[j][t];
          scur[j][t] = snxt[j][t];
        }
    }
    __syncthreads();
  }

  // ---- epilogue: lane holds rows 4 kb + r of each 16-row subtile, column n
#pragma unroll
  for (int j = 0; j < BNT; ++j) {
    if (!colv[j]) continue;
    const int64_t col = nbj[j] * kTileRows + n;
    if (col >= a.N) continue;
    float sc = 1.f;
    if (FMT == kFmtFP8) sc = reinterpret_cast<const float*>(a.scales)[col];
#pragma unroll
    for (int i = 0; i < BMS; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = m0 + 16 * i + 4 * kb + r;
        if (row < a.M) {  // the same for lanes n and n ^ 8
          float v = acc[i][j][r];
          if (a.S > 1) {
            a.part[(int64_t(split) * a.M + row) * a.N + col] = v;
          } else {
            if (FMT == kFmtFP8) v *= sc;
            store_out<8>(a.y, a.N, a.swiglu, row, col, v, true);  // lane ^ 8: column ^ 8
          }
        }
      }
  }
}

// y = sum of the S split partials, added in split order; FP8 applies the
// per-column scale after the sum, as the single-pass epilogue does.  Each
// thread owns 4 consecutive outputs and requests all S partials before the
// first add, so the kernel costs one memory round trip, not S.
constexpr int kMaxSplits = 16;

template <int FMT>
__device__ __forceinline__ float reduce_scale(float v, const float* __restrict__ colscale, int64_t i, int64_t N) {
  return FMT == kFmtFP8 ? v * colscale[i % N] : v;
}

template <int FMT>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int S, int64_t M,
                                                            int64_t N, const float* __restrict__ colscale,
                                                            uint16_t* __restrict__ y, int swiglu) {
  const int64_t MN = M * N;
  const int64_t i0 = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (i0 >= MN) return;  // SwiGLU: N % 16 == 0, so a thread and its partner (^ 2) return together
  if ((MN & 3) == 0) {
    float4 v[kMaxSplits];
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s)
      if (s < S) v[s] = *reinterpret_cast<const float4*>(part + int64_t(s) * MN + i0);
    float4 a = v[0];
#pragma unroll
    for (int s = 1; s < kMaxSplits; ++s)
      if (s < S) {
        a.x += v[s].x;
        a.y += v[s].y;
        a.z += v[s].z;
        a.w += v[s].w;
      }
    const float f[4] = {reduce_scale<FMT>(a.x, colscale, i0, N), reduce_scale<FMT>(a.y, colscale, i0 + 1, N),
                        reduce_scale<FMT>(a.z, colscale, i0 + 2, N), reduce_scale<FMT>(a.w, colscale, i0 + 3, N)};
    if (swiglu) {
      // outputs i and i ^ 8 (columns n and n ^ 8 of one row) are 2 threads apart
#pragma unroll
      for (int e = 0; e < 4; ++e) store_out<2>(y, N, true, (i0 + e) / N, (i0 + e) % N, f[e], true);
      return;
    }
    const uint32_t lo = f32_to_bf16_rne(f[0]) | (f32_to_bf16_rne(f[1]) << 16);
    const uint32_t hi = f32_to_bf16_rne(f[2]) | (f32_to_bf16_rne(f[3]) << 16);
    *reinterpret_cast<uint2*>(y + i0) = make_uint2(lo, hi);
    return;
  }
  const int n = MN - i0 < 4 ? int(MN - i0) : 4;
  for (int e = 0; e < n; ++e) {
    float v[kMaxSplits];
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s)
      if (s < S) v[s] = part[int64_t(s) * MN + i0 + e];
    float a = v[0];
#pragma unroll
    for (int s = 1; s < kMaxSplits; ++s)
      if (s < S) a += v[s];
    y[i0 + e] = uint16_t(f32_to_bf16_rne(reduce_scale<FMT>(a, colscale, i0 + e, N)));
  }
}

// The common case (N a multiple of 8, plain store): eight outputs of one row
// per thread, every split's 32 bytes requested before the first add (twice
// the bytes in flight per thread of the four-output form, and one column
// index per thread).  The sum runs in split order, as above.
template <int FMT>
__global__ __launch_bounds__(256) void splitk_reduce8_kernel(const float* __restrict__ part, int S, int64_t MN,
                                                             int64_t N, const float* __restrict__ colscale,
                                                             uint16_t* __restrict__ y) {
  const int64_t i0 = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 8;
  if (i0 >= MN) return;
  float4 v[kMaxSplits][2];
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s)
    if (s < S) {
      v[s][0] = *reinterpret_cast<const float4*>(part + int64_t(s) * MN + i0);
      v[s][1] = *reinterpret_cast<const float4*>(part + int64_t(s) * MN + i0 + 4);
    }
  float4 a = v[0][0], b = v[0][1];
#pragma unroll
  for (int s = 1; s < kMaxSplits; ++s)
    if (s < S) {
      a.x += v[s][0].x;
      a.y += v[s][0].y;
      a.z += v[s][0].z;
      a.w += v[s][0].w;
      b.x += v[s][1].x;
      b.y += v[s][1].y;
      b.z += v[s][1].z;
      b.w += v[s][1].w;
    }
  float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  if constexpr (FMT == kFmtFP8) {
    const int64_t n0 = i0 % N;  // the eight outputs share a row: N % 8 == 0
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] *= colscale[n0 + e];
  }
  uint32_t o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = f32_to_bf16_rne(f[2 * e]) | (f32_to_bf16_rne(f[2 * e + 1]) << 16);
  *reinterpret_cast<uint4*>(y + i0) = make_uint4(o[0], o[1], o[2], o[3]);
}

hipError_t launch_splitk_reduce(int fmt, const float* part, int S, int64_t M, int64_t N, const void* scales, void* y,
                                bool swiglu, hipStream_t st) {
  if (S < 1 || S > kMaxSplits) return hipErrorInvalidValue;
  if (swiglu && N % 16 != 0) return hipErrorInvalidValue;
  if (!swiglu && N % 8 == 0) {
    const dim3 grid8(unsigned((M * N / 8 + 255) / 256));
    const float* cs8 = reinterpret_cast<const float*>(scales);
    uint16_t* yo8 = reinterpret_cast<uint16_t*>(y);
    if (fmt == kFmtFP8)
      hipLaunchKernelGGL(splitk_reduce8_kernel<kFmtFP8>, grid8, dim3(256), 0, st, part, S, M * N, N, cs8, yo8);
    else
      hipLaunchKernelGGL(splitk_reduce8_kernel<kFmtBF16>, grid8, dim3(256), 0, st, part, S, M * N, N, cs8, yo8);
    return hipGetLastError();
  }
  const int64_t quads = (M * N + 3) / 4;
  const dim3 grid(unsigned((quads + 255) / 256));
  const float* cs = reinterpret_cast<const float*>(scales);
  uint16_t* yo = reinterpret_cast<uint16_t*>(y);
  if (fmt == kFmtFP8)
    hipLaunchKernelGGL(splitk_reduce_kernel<kFmtFP8>, grid, dim3(256), 0, st, part, S, M, N, cs, yo, int(swiglu));
  else
    hipLaunchKernelGGL(splitk_reduce_kernel<kFmtBF16>, grid, dim3(256), 0, st, part, S, M, N, cs, yo, int(swiglu));
  return hipGetLastError();
}

template <int FMT, int BMS, int BNT>
static hipError_t launch_mf(MfmaArgs a, hipStream_t st) {
  const int64_t nbb8 = ceil_div(a.NBB, 8) * 8;
  const int64_t grid = nbb8 * a.MB;
  hipLaunchKernelGGL((mfma_kernel<FMT, BMS, BNT>), dim3(unsigned(grid), unsigned(a.S)), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.S == 1) return e;
  return launch_splitk_reduce(FMT, a.part, a.S, a.M, a.N, a.scales, a.y, a.swiglu != 0, st);
}

template <int FMT>
static hipError_t launch_mf_fmt(const MfmaArgs& a, int bms, int bnt, hipStream_t st) {
  if (bms == 1) return launch_mf<FMT, 1, 1>(a, st);
  if (bms == 2) return launch_mf<FMT, 2, 1>(a, st);
  if (bnt == 1) return launch_mf<FMT, 4, 1>(a, st);
  return launch_mf<FMT, 4, (FMT == kFmtBF16 ? 1 : 2)>(a, st);
}

hipError_t launch_mfma(int fmt, const MfmaPlan& p, int64_t M, int64_t N, int64_t K, const void* x, const void* wp,
                       const void* scales, const void* zeros, void* y, void* ws, bool swiglu, hipStream_t st) {
  MfmaArgs a;
  a.swiglu = swiglu;
  a.x = reinterpret_cast<const uint16_t*>(x);
  a.y = reinterpret_cast<uint16_t*>(y);
  a.w = reinterpret_cast<const uint4*>(wp);
  a.scales = scales;
  a.zeros = reinterpret_cast<const uint16_t*>(zeros);
  a.part = reinterpret_cast<float*>(ws);
  a.M = M;
  a.N = N;
  a.K = K;
  a.NB = p.NB;
  a.KT = p.KT;
  a.G4 = fmt == kFmtW4 ? ceil_div(K / kGroup, kScaleQuad) : 0;
  a.NBB = int(p.NBB);
  a.MB = int(p.MB);
  a.S = p.S;
  a.cps = p.chunks_per_split;
  if (fmt == kFmtBF16) return launch_mf_fmt<kFmtBF16>(a, p.BMS, p.BNT, st);
  if (fmt == kFmtFP8) return launch_mf_fmt<kFmtFP8>(a, p.BMS, p.BNT, st);
  return launch_mf_fmt<kFmtW4>(a, p.BMS, p.BNT, st);
}

}  // namespace wqd
