// HBM ceiling kernels: a read-only stream (16-byte loads folded into a
// checksum so the loads cannot be dropped) and a 16-byte copy.  They give the
// measured bandwidth that the decode kernels are compared against.
#include "wqd_internal.h"

namespace wqd {

static constexpr unsigned kStreamBlocks = 2048;  // 8 workgroups per compute unit on 256 CUs

__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ src, size_t n16,
                                                          uint32_t* __restrict__ sink) {
  __shared__ uint32_t red[4];
  uint32_t acc = 0;
  const size_t stride = size_t(gridDim.x) * 256;
  size_t i = size_t(blockIdx.x) * 256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

__global__ __launch_bounds__(256) void stream_copy_kernel(uint4* __restrict__ dst, const uint4* __restrict__ src,
                                                          size_t n16) {
  const size_t stride = size_t(gridDim.x) * 256;
  for (size_t i = size_t(blockIdx.x) * 256 + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
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

hipError_t launch_stream_copy(void* dst, const void* src, size_t bytes, hipStream_t st) {
  const size_t n16 = bytes / 16;
  hipLaunchKernelGGL(stream_copy_kernel, dim3(unsigned(stream_sink_words(bytes))), dim3(256), 0, st,
                     reinterpret_cast<uint4*>(dst), reinterpret_cast<const uint4*>(src), n16);
  return hipGetLastError();
}

}  // namespace wqd
