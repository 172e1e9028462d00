// Setup and parity kernels: quantise + pre-shuffle (pack), dequantise, unpack
// to logical codes, and the raw E4M3 decode.
#include "wqd_device.h"
#include "wqd_internal.h"
#include "wqd_plan.h"

namespace wqd {

// Thread mapping of the pack / dequant / unpack kernels: one thread per
// (16-row block nb, K tile kt, row r), t = (nb * KT + kt) * 16 + r.  It owns
// the 64 bytes of row r inside the tile, i.e. slice j at uint4 index 16 j + r.
struct RowTile {
  int64_t nb, kt, n, tile;
  int r;
};

__device__ __forceinline__ bool row_tile(int64_t t, int64_t NB, int64_t KT, RowTile& rt) {
  if (t >= NB * KT * kTileRows) return false;
  rt.r = int(t % kTileRows);
  rt.tile = t / kTileRows;
  rt.nb = rt.tile / KT;
  rt.kt = rt.tile % KT;
  rt.n = rt.nb * kTileRows + rt.r;
  return true;
}

__device__ __forceinline__ void store_row_slices(uint4* wp, const RowTile& rt, const uint32_t (&words)[16]) {
  uint4* base = wp + rt.tile * (kTileBytes / 16);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    base[j * kTileRows + rt.r] = make_uint4(words[4 * j], words[4 * j + 1], words[4 * j + 2], words[4 * j + 3]);
}

// ------------------------------------------------------------------ BF16 pack
__global__ __launch_bounds__(256) void pack_bf16_kernel(const float* __restrict__ W, int64_t N, int64_t K,
                                                        int64_t NB, int64_t KT, uint4* __restrict__ wp, int64_t F) {
  RowTile rt;
  if (!row_tile(int64_t(blockIdx.x) * 256 + threadIdx.x, NB, KT, rt)) return;
  const int64_t k0 = rt.kt * 32;
  uint32_t words[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {  // 8 x 4 consecutive k
    float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
    const int64_t k = k0 + 4 * i;
    if (rt.n < N && k < K) f = *reinterpret_cast<const float4*>(W + src_row(rt.n, F) * K + k);
    words[2 * i + 0] = f32_to_bf16_rne(f.x) | (f32_to_bf16_rne(f.y) << 16);
    words[2 * i + 1] = f32_to_bf16_rne(f.z) | (f32_to_bf16_rne(f.w) << 16);
  }
  store_row_slices(wp, rt, words);
}

// ------------------------------------------------------------------ FP8 pack
// Row scale s_n = max|W[n, :]| / 448 in float32 (1 for an all-zero row,
// floored at 2^-126); one workgroup per (padded) row.
__global__ __launch_bounds__(256) void fp8_rowscale_kernel(const float* __restrict__ W, int64_t N, int64_t K,
                                                           float* __restrict__ scales, int64_t F) {
  __shared__ float red[4];
  const int64_t n = blockIdx.x;
  float a = 0.f;
  if (n < N) {
    for (int64_t k = int64_t(threadIdx.x) * 4; k < K; k += 1024) {
      float4 f = *reinterpret_cast<const float4*>(W + src_row(n, F) * K + k);
      a = fmaxf(a, fmaxf(fmaxf(fabsf(f.x), fabsf(f.y)), fmaxf(fabsf(f.z), fabsf(f.w))));
    }
  }
  for (int off = 32; off > 0; off >>= 1) a = fmaxf(a, __shfl_xor(a, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
  __syncthreads();
  if (threadIdx.x == 0) {
    a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    float s = 0.f;
    if (n < N) {
      s = __fdiv_rn(a, 448.0f);
      s = fmaxf(s, 0x1p-126f);
      if (a == 0.f) s = 1.0f;
    }
    scales[n] = s;
  }
}

__global__ __launch_bounds__(256) void pack_fp8_kernel(const float* __restrict__ W, int64_t N, int64_t K,
                                                       int64_t NB, int64_t KT, const float* __restrict__ scales,
                                                       uint4* __restrict__ wp, int64_t F) {
  RowTile rt;
  if (!row_tile(int64_t(blockIdx.x) * 256 + threadIdx.x, NB, KT, rt)) return;
  const int64_t k0 = rt.kt * 64;
  const float s = rt.n < N ? scales[rt.n] : 1.0f;
  uint32_t words[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {  // word i = codes of k0 + 4i .. 4i+3
    const int64_t k = k0 + 4 * i;
    uint32_t w = 0;
    if (rt.n < N && k < K) {
      float4 f = *reinterpret_cast<const float4*>(W + src_row(rt.n, F) * K + k);
      w = e4m3_encode(__fdiv_rn(f.x, s)) | (e4m3_encode(__fdiv_rn(f.y, s)) << 8) |
          (e4m3_encode(__fdiv_rn(f.z, s)) << 16) | (e4m3_encode(__fdiv_rn(f.w, s)) << 24);
    }
    words[i] = w;
  }
  store_row_slices(wp, rt, words);
}

// ------------------------------------------------------------------ W4A16 pack
// One thread per (row, 128-wide K group): lo = min(0, min W), hi = max(0, max W),
// s = fp16(fp32(hi - lo) / 15), z = clamp(rint(-lo/s)), q = clamp(rint(W/s) + z)
// (CS336 lecture 10 notes, 5.2: a scale and a zero point; "Making each token
// cheaper", Formats: one scale per group of 128).  Thread t =
// ((nb * G4 + g4) * 16 + r) * 4 + gq handles group g = 4 g4 + gq of row
// 16 nb + r, which is also the index of its scale; the four groups of a
// (row, g4) are consecutive lanes and merge their zero nibbles into one uint16.
__global__ __launch_bounds__(256) void pack_w4_kernel(const float* __restrict__ W, int64_t N, int64_t K,
                                                      int64_t NB, int64_t G, int64_t G4, uint4* __restrict__ wp,
                                                      uint16_t* __restrict__ scales, uint16_t* __restrict__ zeros,
                                                      int64_t F) {
  const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int64_t total = NB * G4 * kTileRows * kScaleQuad;
  const bool in_range = t < total;  // the grid is a multiple of 4 threads, so quads stay together
  const int gq = int(t & 3);
  const int r = int((t >> 2) % kTileRows);
  const int64_t g4 = (t >> 2) / kTileRows % (G4 > 0 ? G4 : 1);
  const int64_t nb = (t >> 2) / kTileRows / (G4 > 0 ? G4 : 1);
  const int64_t g = g4 * kScaleQuad + gq;
  const int64_t n = nb * kTileRows + r;
  const bool valid = in_range && g < G && n < N;
  float v[128];
  float lo = 0.f, hi = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
    if (valid) f = *reinterpret_cast<const float4*>(W + src_row(n, F) * K + g * kGroup + 4 * i);
    v[4 * i + 0] = f.x;
    v[4 * i + 1] = f.y;
    v[4 * i + 2] = f.z;
    v[4 * i + 3] = f.w;
    lo = fminf(lo, fminf(fminf(f.x, f.y), fminf(f.z, f.w)));
    hi = fmaxf(hi, fmaxf(fmaxf(f.x, f.y), fmaxf(f.z, f.w)));
  }
  const float span = __fsub_rn(hi, lo);
  __half s16 = __float2half_rn(__fdiv_rn(span, 15.0f));
  uint16_t sb = __half_as_ushort(s16);
  if ((sb & 0x7FFFu) == 0) sb = 0x0001;        // 2^-24, the smallest fp16 step
  if ((sb & 0x7FFFu) == 0x7C00u) sb = 0x7BFF;  // infinite scale -> 65504
  if (span == 0.f) sb = 0x3C00;                // all-zero group: s = 1
  const float s = __half2float(__ushort_as_half(sb));
  const float zf = fminf(fmaxf(rintf(__fdiv_rn(-lo, s)), 0.f), 15.f);
  uint32_t words[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    uint32_t w = 0;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float qf = fminf(fmaxf(rintf(__fdiv_rn(v[8 * i + nib_elem(q)], s)) + zf, 0.f), 15.f);
      w |= uint32_t(qf) << (4 * q);
    }
    words[i] = w;
  }
  if (in_range && g < G) {
    RowTile rt;
    rt.r = r;
    rt.tile = nb * G + g;
    store_row_slices(wp, rt, words);  // padded rows (n >= N) store zero codes
  }
  const uint32_t z = valid ? uint32_t(zf) : 0u;
  if (in_range) scales[t] = valid ? sb : uint16_t(0);
  // merge the four zero nibbles of this (row, g4)
  uint32_t zq = z << (4 * gq);
  zq |= __shfl_xor(zq, 1);
  zq |= __shfl_xor(zq, 2);
  if (in_range && gq == 0) zeros[t >> 2] = uint16_t(zq);
}

// ------------------------------------------------------------------ dequant / unpack
// Logical element e (0..tile_k-1) of row r in a tile, read back from the
// packed slices: the code (bf16 bits, e4m3 code or uint4 q).
template <int FMT>
__device__ __forceinline__ uint32_t tile_code(const uint4* base, int r, int e) {
  if (FMT == kFmtBF16) {
    const int j = e >> 3, w = (e & 7) >> 1;
    const uint4 v = base[j * kTileRows + r];
    const uint32_t word = w == 0 ? v.x : w == 1 ? v.y : w == 2 ? v.z : v.w;
    return (word >> (16 * (e & 1))) & 0xFFFFu;
  } else if (FMT == kFmtFP8) {
    const int j = e >> 4, w = (e & 15) >> 2;
    const uint4 v = base[j * kTileRows + r];
    const uint32_t word = w == 0 ? v.x : w == 1 ? v.y : w == 2 ? v.z : v.w;
    return (word >> (8 * (e & 3))) & 0xFFu;
  } else {
    const int j = e >> 5, w = (e & 31) >> 3, el = e & 7;
    const uint4 v = base[j * kTileRows + r];
    const uint32_t word = w == 0 ? v.x : w == 1 ? v.y : w == 2 ? v.z : v.w;
    const int q = (el & 1) * 4 + (el >> 1);  // inverse of nib_elem
    return (word >> (4 * q)) & 0xFu;
  }
}

__device__ __forceinline__ uint32_t w4_scale_bits(const uint16_t* scales, int64_t nb, int64_t G4, int r, int64_t g) {
  return scales[((nb * G4 + g / kScaleQuad) * kTileRows + r) * kScaleQuad + g % kScaleQuad];
}

__device__ __forceinline__ uint32_t w4_zero(const uint16_t* zeros, int64_t nb, int64_t G4, int r, int64_t g) {
  return (uint32_t(zeros[(nb * G4 + g / kScaleQuad) * kTileRows + r]) >> (4 * (g % kScaleQuad))) & 0xFu;
}

template <int FMT>
__global__ __launch_bounds__(256) void dequant_kernel(const uint4* __restrict__ wp, const void* __restrict__ scales,
                                                      const uint16_t* __restrict__ zeros, int64_t N, int64_t K,
                                                      int64_t NB, int64_t KT, int64_t G4, float* __restrict__ out) {
  constexpr int TK = FMT == kFmtBF16 ? 32 : FMT == kFmtFP8 ? 64 : 128;
  RowTile rt;
  if (!row_tile(int64_t(blockIdx.x) * 256 + threadIdx.x, NB, KT, rt)) return;
  if (rt.n >= N) return;
  const uint4* base = wp + rt.tile * (kTileBytes / 16);
  float s = 1.f;
  float z = 0.f;
  if (FMT == kFmtFP8) s = reinterpret_cast<const float*>(scales)[rt.n];
  if (FMT == kFmtW4) {
    s = __half2float(__ushort_as_half(
        uint16_t(w4_scale_bits(reinterpret_cast<const uint16_t*>(scales), rt.nb, G4, rt.r, rt.kt))));
    z = float(w4_zero(zeros, rt.nb, G4, rt.r, rt.kt));
  }
  for (int e = 0; e < TK; ++e) {
    const int64_t k = rt.kt * TK + e;
    if (k >= K) break;
    const uint32_t c = tile_code<FMT>(base, rt.r, e);
    float v;
    if (FMT == kFmtBF16) v = bf16_bits_to_f32(c);
    else if (FMT == kFmtFP8) v = __fmul_rn(e4m3_to_f32(c), s);
    else v = __fmul_rn(__fsub_rn(float(c), z), s);
    out[rt.n * K + k] = v;
  }
}

template <int FMT>
__global__ __launch_bounds__(256) void unpack_kernel(const uint4* __restrict__ wp, const void* __restrict__ scales,
                                                     const uint16_t* __restrict__ zeros, int64_t N, int64_t K,
                                                     int64_t NB, int64_t KT, int64_t G4, void* __restrict__ codes_out,
                                                     void* __restrict__ scales_out, uint8_t* __restrict__ zeros_out) {
  constexpr int TK = FMT == kFmtBF16 ? 32 : FMT == kFmtFP8 ? 64 : 128;
  RowTile rt;
  if (!row_tile(int64_t(blockIdx.x) * 256 + threadIdx.x, NB, KT, rt)) return;
  if (rt.n >= N) return;
  const uint4* base = wp + rt.tile * (kTileBytes / 16);
  for (int e = 0; e < TK; ++e) {
    const int64_t k = rt.kt * TK + e;
    if (k >= K) break;
    const uint32_t c = tile_code<FMT>(base, rt.r, e);
    if (FMT == kFmtBF16) reinterpret_cast<uint16_t*>(codes_out)[rt.n * K + k] = uint16_t(c);
    else reinterpret_cast<uint8_t*>(codes_out)[rt.n * K + k] = uint8_t(c);
  }
  if (FMT == kFmtFP8 && rt.kt == 0 && scales_out)
    reinterpret_cast<float*>(scales_out)[rt.n] = reinterpret_cast<const float*>(scales)[rt.n];
  if (FMT == kFmtW4) {
    const int64_t G = K / kGroup;
    if (scales_out)
      reinterpret_cast<uint16_t*>(scales_out)[rt.n * G + rt.kt] =
          uint16_t(w4_scale_bits(reinterpret_cast<const uint16_t*>(scales), rt.nb, G4, rt.r, rt.kt));
    if (zeros_out) zeros_out[rt.n * G + rt.kt] = uint8_t(w4_zero(zeros, rt.nb, G4, rt.r, rt.kt));
  }
}

__global__ __launch_bounds__(256) void decode_e4m3_kernel(const uint8_t* __restrict__ codes, float* __restrict__ out,
                                                          int64_t n) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) out[i] = e4m3_to_f32(codes[i]);
}

// ------------------------------------------------------------------ launchers
static inline unsigned grid_for(int64_t threads) { return unsigned((threads + 255) / 256); }

hipError_t launch_pack(int fmt, const float* W, int64_t N, int64_t K, const PackedSizes& ps, void* wp, void* scales,
                       void* zeros, int64_t F, hipStream_t st) {
  uint4* w4 = reinterpret_cast<uint4*>(wp);
  const int64_t rows_tiles = ps.NB * ps.KT * kTileRows;
  if (fmt == kFmtBF16) {
    hipLaunchKernelGGL(pack_bf16_kernel, dim3(grid_for(rows_tiles)), dim3(256), 0, st, W, N, K, ps.NB, ps.KT, w4, F);
  } else if (fmt == kFmtFP8) {
    float* sc = reinterpret_cast<float*>(scales);
    hipLaunchKernelGGL(fp8_rowscale_kernel, dim3(unsigned(ps.NB * kTileRows)), dim3(256), 0, st, W, N, K, sc, F);
    hipLaunchKernelGGL(pack_fp8_kernel, dim3(grid_for(rows_tiles)), dim3(256), 0, st, W, N, K, ps.NB, ps.KT, sc, w4,
                       F);
  } else {
    const int64_t threads = ps.NB * ps.G4 * kTileRows * kScaleQuad;
    hipLaunchKernelGGL(pack_w4_kernel, dim3(grid_for(threads)), dim3(256), 0, st, W, N, K, ps.NB, ps.KT, ps.G4, w4,
                       reinterpret_cast<uint16_t*>(scales), reinterpret_cast<uint16_t*>(zeros), F);
  }
  return hipGetLastError();
}

hipError_t launch_dequant(int fmt, const void* wp, const void* scales, const void* zeros, int64_t N, int64_t K,
                          const PackedSizes& ps, float* out, hipStream_t st) {
  const uint4* w4 = reinterpret_cast<const uint4*>(wp);
  const uint16_t* z = reinterpret_cast<const uint16_t*>(zeros);
  dim3 grid(grid_for(ps.NB * ps.KT * kTileRows));
  if (fmt == kFmtBF16)
    hipLaunchKernelGGL(dequant_kernel<kFmtBF16>, grid, dim3(256), 0, st, w4, scales, z, N, K, ps.NB, ps.KT, ps.G4, out);
  else if (fmt == kFmtFP8)
    hipLaunchKernelGGL(dequant_kernel<kFmtFP8>, grid, dim3(256), 0, st, w4, scales, z, N, K, ps.NB, ps.KT, ps.G4, out);
  else
    hipLaunchKernelGGL(dequant_kernel<kFmtW4>, grid, dim3(256), 0, st, w4, scales, z, N, K, ps.NB, ps.KT, ps.G4, out);
  return hipGetLastError();
}

hipError_t launch_unpack(int fmt, const void* wp, const void* scales, const void* zeros, int64_t N, int64_t K,
                         const PackedSizes& ps, void* codes, void* scales_out, void* zeros_out, hipStream_t st) {
  const uint4* w4 = reinterpret_cast<const uint4*>(wp);
  const uint16_t* z = reinterpret_cast<const uint16_t*>(zeros);
  uint8_t* zo = reinterpret_cast<uint8_t*>(zeros_out);
  dim3 grid(grid_for(ps.NB * ps.KT * kTileRows));
  if (fmt == kFmtBF16)
    hipLaunchKernelGGL(unpack_kernel<kFmtBF16>, grid, dim3(256), 0, st, w4, scales, z, N, K, ps.NB, ps.KT, ps.G4,
                       codes, scales_out, zo);
  else if (fmt == kFmtFP8)
    hipLaunchKernelGGL(unpack_kernel<kFmtFP8>, grid, dim3(256), 0, st, w4, scales, z, N, K, ps.NB, ps.KT, ps.G4,
                       codes, scales_out, zo);
  else
    hipLaunchKernelGGL(unpack_kernel<kFmtW4>, grid, dim3(256), 0, st, w4, scales, z, N, K, ps.NB, ps.KT, ps.G4,
                       codes, scales_out, zo);
  return hipGetLastError();
}

hipError_t launch_decode_e4m3(const uint8_t* codes, float* out, int64_t n, hipStream_t st) {
  hipLaunchKernelGGL(decode_e4m3_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, st, codes, out, n);
  return hipGetLastError();
}

}  // namespace wqd
