// Speculative-sampling accept / reject over the verify pass's distributions
// (CS336 lecture 10 notes, section 6.1: keep draft tokens left to right with
// probability min(1, target / draft), resample the first rejection from the
// normalised positive part of target - draft, or draw one more token from the
// last target row when every draft is kept; section 6.2: the output is then an
// exact sample of the target).
//
// One workgroup of 16 wavefronts per sequence.  The accept tests are a
// handful of loads, taken by every thread alike.  The draw reads one row (two
// for a residual) of V float32 probabilities in tiles of 256 tokens: a
// wavefront sums a tile's weights in integer units of 2^-32 from four
// coalesced loads per lane and row, the tile sums are scanned in LDS to find
// the tile that holds the threshold, and one wavefront scans that tile's
// tokens in order to the drawn one.  Integer units make the draw exact and
// independent of the order of summation.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "wqd_internal.h"

namespace wqd {

constexpr int kSpecWaves = 16;
constexpr int kSpecThreads = 64 * kSpecWaves;
constexpr int kSpecTile = 256;                                   // tokens per tile, 4 per lane
constexpr int kSpecMaxTiles = (1 << 20) / kSpecTile;             // V <= 2^20
static_assert(kSpecMaxTiles == 4 * kSpecThreads, "each thread scans four tile sums");

typedef unsigned long long u64;

// floor(w * 2^32): exact for float32 w in [0, 1] (scaling by 2^32 is exact in
// double).  A weight outside [0, 1] counts as the nearest end of it, a NaN as
// 0 (fmaxf returns its other operand), so the unit sum cannot overflow.
__device__ inline u64 draw_unit(float w) {
  w = fminf(fmaxf(w, 0.0f), 1.0f);
  return u64(floor(double(w) * 4294967296.0));
}

// The draw's threshold floor(u * T) for T > 0, kept in [0, T - 1]: a u of 1 or
// more (a generator with range (0, 1]) takes the last token of positive
// weight, and a NaN or negative u counts as 0.
__device__ inline u64 draw_threshold(float u, u64 T) {
  const double p = u > 0.0f ? double(u) : 0.0;
  const double f = floor(p * double(T));
  return f >= double(T) ? T - 1 : u64(f);
}

__device__ inline u64 weight_at(const float* tr, const float* dr, int64_t j, int64_t V) {
  if (j >= V) return 0;
  return dr ? draw_unit(fmaxf(tr[j] - dr[j], 0.0f)) : draw_unit(tr[j]);
}

__device__ inline u64 wave_inclusive_scan(u64 v, int lane) {
  for (int o = 1; o < 64; o <<= 1) {
    const u64 n = __shfl_up(v, o);
    if (lane >= o) v += n;
  }
  return v;
}

__global__ __launch_bounds__(kSpecThreads) void spec_accept_kernel(
    const float* __restrict__ target, const float* __restrict__ draft, const int32_t* __restrict__ tokens,
    const float* __restrict__ u_accept, const float* __restrict__ u_draw, int64_t k, int64_t V,
    int32_t* __restrict__ n_kept, int32_t* __restrict__ out) {
  __shared__ u64 s_tile[kSpecMaxTiles];
  __shared__ u64 s_wave[kSpecWaves];
  __shared__ u64 s_pick[2];  // picked tile, units before it
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
  if (tid == 0) {
    n_kept[b] = int32_t(r);
    s_pick[0] = 0;  // read only after a barrier; always overwritten when T > 0
    s_pick[1] = 0;
  }

  // the draw: residual of row r, else (empty residual, or every draft kept) target row r
  const float* tr = t + r * V;
  const float* dr = r < k ? d + r * V : nullptr;
  const int64_t NT = (V + kSpecTile - 1) / kSpecTile;
  for (int pass = 0; pass < 2; ++pass) {
    // tile sums: wavefront w takes tiles w, w + 16, ...
#pragma unroll 4
    for (int64_t ti = wave; ti < NT; ti += kSpecWaves) {
      const int64_t j = ti * kSpecTile + lane;
      u64 s = weight_at(tr, dr, j, V) + weight_at(tr, dr, j + 64, V) + weight_at(tr, dr, j + 128, V) +
              weight_at(tr, dr, j + 192, V);
      for (int m = 32; m > 0; m >>= 1) s += __shfl_xor(s, m);
      if (lane == 0) s_tile[ti] = s;
    }
    __syncthreads();
    // scan of the tile sums: thread t owns tiles 4t .. 4t + 3
    u64 mine = 0;
    for (int q = 0; q < 4; ++q) {
      const int64_t i = 4 * tid + q;
      mine += i < NT ? s_tile[i] : 0;
    }
    const u64 incl = wave_inclusive_scan(mine, lane);
    if (lane == 63) s_wave[wave] = incl;
    __syncthreads();
    u64 wbase = 0, T = 0;
    for (int w = 0; w < kSpecWaves; ++w) {
      const u64 s = s_wave[w];
      if (w < wave) wbase += s;
      T += s;
    }
    if (T == 0 && dr) {  // empty residual: draw from the target row
      dr = nullptr;
      __syncthreads();
      continue;
    }
    if (T == 0) {
      if (tid == 0) o[r] = -1;
      break;
    }
    const u64 U = draw_threshold(u_draw[b], T);
    const u64 base = wbase + incl - mine;
    if (base <= U && U < base + mine) {  // the one thread whose tiles hold the threshold
      u64 acc = base;
      for (int q = 0; q < 4; ++q) {
        const int64_t i = 4 * tid + q;
        const u64 s = i < NT ? s_tile[i] : 0;
        if (acc + s > U) {
          s_pick[0] = u64(i);
          s_pick[1] = acc;
          break;
        }
        acc += s;
      }
    }
    __syncthreads();
    // the picked tile, in token order: lane l holds tokens 4l .. 4l + 3
    if (wave == 0) {
      const int64_t j0 = int64_t(s_pick[0]) * kSpecTile + 4 * lane;
      u64 w4[4], sum = 0;
      for (int q = 0; q < 4; ++q) {
        w4[q] = weight_at(tr, dr, j0 + q, V);
        sum += w4[q];
      }
      u64 acc = s_pick[1] + wave_inclusive_scan(sum, lane) - sum;
      if (acc <= U && U < acc + sum) {
        for (int q = 0; q < 4; ++q) {
          acc += w4[q];
          if (acc > U) {
            o[r] = int32_t(j0 + q);
            break;
          }
        }
      }
    }
    break;
  }
}

hipError_t launch_spec_accept(const float* target, const float* draft, const int32_t* tokens, const float* u_accept,
                              const float* u_draw, int64_t B, int64_t k, int64_t V, int32_t* n_kept, int32_t* out,
                              hipStream_t st) {
  hipLaunchKernelGGL(spec_accept_kernel, dim3(unsigned(B)), dim3(kSpecThreads), 0, st, target, draft, tokens,
                     u_accept, u_draw, k, V, n_kept, out);
  return hipGetLastError();
}

}  // namespace wqd
