// Speculative-sampling accept / reject over the verify pass's distributions
// (CS336 lecture 10 notes, section 6.1: keep draft tokens left to right with
// probability min(1, target / draft), resample the first rejection from the
// normalised positive part of target - draft, or draw one more token from the
// last target row when every draft is kept; section 6.2: the output is then an
// exact sample of the target).
//
// One workgroup of 256 threads per sequence.  The accept tests are a handful
// of loads, taken by every thread alike.  The draw reads one row (two for a
// residual) of V float32 probabilities: each thread owns a contiguous segment
// of V / 256 tokens, sums its weights in integer units of 2^-32, the segment
// sums are scanned in LDS, and the thread whose segment holds the threshold
// walks it to the drawn token.  Integer units make the draw exact and
// independent of the order of summation.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "wqd_internal.h"

namespace wqd {
namespace {

constexpr int kSpecThreads = 256;

// floor(w * 2^32): exact for float32 w in [0, 1] (scaling by 2^32 is exact in double).
__device__ inline uint64_t draw_unit(float w) { return uint64_t(floor(double(w) * 4294967296.0)); }

__device__ inline uint64_t weight_at(const float* tr, const float* dr, int64_t j) {
  return dr ? draw_unit(fmaxf(tr[j] - dr[j], 0.0f)) : draw_unit(tr[j]);
}

__global__ __launch_bounds__(kSpecThreads) void spec_accept_kernel(
    const float* __restrict__ target, const float* __restrict__ draft, const int32_t* __restrict__ tokens,
    const float* __restrict__ u_accept, const float* __restrict__ u_draw, int64_t k, int64_t V,
    int32_t* __restrict__ n_kept, int32_t* __restrict__ out) {
  __shared__ uint64_t s_seg[kSpecThreads];
  __shared__ uint64_t s_total;
  const int tid = threadIdx.x;
  const int64_t b = blockIdx.x;
  const float* t = target + b * (k + 1) * V;
  const float* d = draft ? draft + b * k * V : nullptr;
  int32_t* o = out + b * (k + 1);

  // accept tests, left to right: keep x while u * d(x) < t(x) in float32
  int64_t r = k;
  for (int64_t i = 0; i < k; ++i) {
    const int32_t x = tokens[b * k + i];
    const bool keep = x >= 0 && x < V && u_accept[b * k + i] * d[i * V + x] < t[i * V + x];
    if (!keep) {
      r = i;
      break;
    }
  }
  for (int64_t i = tid; i <= k; i += kSpecThreads)
    if (i != r) o[i] = i < r ? tokens[b * k + i] : -1;
  if (tid == 0) n_kept[b] = int32_t(r);

  // the draw: residual of row r, else (empty residual, or every draft kept) target row r
  const float* tr = t + r * V;
  const float* dr = r < k ? d + r * V : nullptr;
  const int64_t seg = (V + kSpecThreads - 1) / kSpecThreads;
  const int64_t lo = tid * seg < V ? tid * seg : V;
  const int64_t hi = lo + seg < V ? lo + seg : V;
  for (int pass = 0; pass < 2; ++pass) {
    uint64_t mine = 0;
    for (int64_t j = lo; j < hi; ++j) mine += weight_at(tr, dr, j);
    s_seg[tid] = mine;
    __syncthreads();
    if (tid == 0) {
      uint64_t acc = 0;
      for (int i = 0; i < kSpecThreads; ++i) {
        const uint64_t s = s_seg[i];
        s_seg[i] = acc;  // exclusive prefix
        acc += s;
      }
      s_total = acc;
    }
    __syncthreads();
    const uint64_t T = s_total;
    if (T == 0 && dr) {  // empty residual: draw from the target row
      dr = nullptr;
      __syncthreads();
      continue;
    }
    if (T == 0) {
      if (tid == 0) o[r] = -1;
      break;
    }
    const uint64_t U = uint64_t(floor(double(u_draw[b]) * double(T)));
    const uint64_t base = s_seg[tid];
    if (base <= U && U < base + mine) {
      uint64_t acc = base;
      for (int64_t j = lo; j < hi; ++j) {
        acc += weight_at(tr, dr, j);
        if (acc > U) {
          o[r] = int32_t(j);
          break;
        }
      }
    }
    break;
  }
}

}  // namespace

hipError_t launch_spec_accept(const float* target, const float* draft, const int32_t* tokens, const float* u_accept,
                              const float* u_draw, int64_t B, int64_t k, int64_t V, int32_t* n_kept, int32_t* out,
                              hipStream_t st) {
  hipLaunchKernelGGL(spec_accept_kernel, dim3(unsigned(B)), dim3(kSpecThreads), 0, st, target, draft, tokens,
                     u_accept, u_draw, k, V, n_kept, out);
  return hipGetLastError();
}

}  // namespace wqd
