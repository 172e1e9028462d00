// Ceiling kernels: a read-only stream (16-byte loads folded into a checksum
// so the loads cannot be dropped) and a 16-byte copy give the measured HBM
// bandwidth that the decode kernels are compared against; back-to-back
// matrix-core multiplies from registers give the measured matrix-core
// throughput that the wide verify batches are compared against.
#include "wqd_device.h"
#include "wqd_internal.h"

namespace wqd {

static constexpr unsigned kStreamBlocks = 2048;  // 8 workgroups per compute unit on 256 CUs
static constexpr int kUnroll = 8;                // independent 16-byte loads per thread in flight

// Each workgroup reads one contiguous range; per iteration its 256 threads
// issue 8 loads each (32 KiB of the range, 1 KiB contiguous per wavefront
// load), all independent, before folding them into the checksum.
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ src, size_t n16,
                                                          uint32_t* __restrict__ sink) {
  __shared__ uint32_t red[4];
  const size_t per_block = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t begin = size_t(blockIdx.x) * per_block;
  const size_t end = begin + per_block < n16 ? begin + per_block : n16;
  uint32_t acc = 0;
  size_t i = begin + threadIdx.x;
  for (; i + (kUnroll - 1) * 256 < end; i += kUnroll * 256) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = load_nt(src + i + u * 256);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < end; i += 256) {
    const uint4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

// The copy has the read kernel's structure: one contiguous range per
// workgroup, and per iteration 8 independent non-temporal 16-byte loads per
// thread before their 8 non-temporal stores, so that 32 KiB per workgroup are
// in flight in each direction.
__global__ __launch_bounds__(256) void stream_copy_kernel(uint4* __restrict__ dst, const uint4* __restrict__ src,
                                                          size_t n16) {
  const size_t per_block = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t begin = size_t(blockIdx.x) * per_block;
  const size_t end = begin + per_block < n16 ? begin + per_block : n16;
  size_t i = begin + threadIdx.x;
  for (; i + (kUnroll - 1) * 256 < end; i += kUnroll * 256) {
    u32x4_t v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src + i + u * 256));
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) __builtin_nontemporal_store(v[u], reinterpret_cast<u32x4_t*>(dst + i + u * 256));
  }
  for (; i < end; i += 256) dst[i] = src[i];
}

size_t stream_sink_words(size_t bytes) {
  const size_t n16 = bytes / 16;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > kStreamBlocks) blocks = kStreamBlocks;
  return blocks < 1 ? 1 : blocks;
}

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t st) {
  const size_t n16 = bytes / 16;
  hipLaunchKernelGGL(stream_read_kernel, dim3(unsigned(stream_sink_words(bytes))), dim3(256), 0, st,
                     reinterpret_cast<const uint4*>(src), n16, sink);
  return hipGetLastError();
}

// Matrix-core ceiling: every wavefront keeps 16 independent accumulators and
// issues iters x 16 v_mfma_f32_16x16x32_bf16 on operands that stay in
// registers; four wavefronts per SIMD (two 8-wavefront workgroups per compute
// unit).  The accumulators are folded into one float per workgroup so the
// multiplies cannot be dropped.
static constexpr unsigned kPeakBlocks = 2 * 256;  // two workgroups on each of the 256 compute units
static constexpr int kPeakThreads = 512, kPeakAcc = 16;

typedef __bf16 pk_bf16x8_t __attribute__((ext_vector_type(8)));
typedef float pk_f32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kPeakThreads) void mfma_peak_kernel(float* __restrict__ sink, int64_t iters) {
  pk_bf16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = __bf16(float(threadIdx.x & 63) * 0.001f + float(i));
    b[i] = __bf16(float(i) * 0.5f + float(blockIdx.x & 7));
  }
  pk_f32x4_t acc[kPeakAcc];
#pragma unroll
  for (int i = 0; i < kPeakAcc; ++i) acc[i] = pk_f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < kPeakAcc; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[i], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kPeakAcc; ++i) s += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
  if (threadIdx.x == 0) sink[blockIdx.x] = s;
}

size_t mfma_peak_sink_words() { return kPeakBlocks; }

double mfma_peak_flops(int64_t iters) {
  return double(kPeakBlocks) * (kPeakThreads / 64) * double(iters) * kPeakAcc * (2.0 * 16 * 16 * 32);
}

hipError_t launch_mfma_peak(int64_t iters, float* sink, hipStream_t st) {
  hipLaunchKernelGGL(mfma_peak_kernel, dim3(kPeakBlocks), dim3(kPeakThreads), 0, st, sink, iters);
  return hipGetLastError();
}

hipError_t launch_stream_copy(void* dst, const void* src, size_t bytes, hipStream_t st) {
  const size_t n16 = bytes / 16;
  hipLaunchKernelGGL(stream_copy_kernel, dim3(unsigned(stream_sink_words(bytes))), dim3(256), 0, st,
                     reinterpret_cast<uint4*>(dst), reinterpret_cast<const uint4*>(src), n16);
  return hipGetLastError();
}

}  // namespace wqd
