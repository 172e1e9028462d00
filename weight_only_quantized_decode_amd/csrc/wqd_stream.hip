// HBM ceiling kernels: a read-only stream (16-byte loads folded into a
// checksum so the loads cannot be dropped) and a 16-byte copy.  They give the
// measured bandwidth that the decode kernels are compared against.
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
