// Speculative-sampling accept / reject over the verify pass's distributions
// (CS336 lecture 10 notes, section 6.1: keep draft tokens left to right with
// probability min(1, target / draft), resample the first rejection from the
// normalised positive part of target - draft, or draw one more token from the
// last target row when every draft is kept; section 6.2: the output is then an
// exact sample of the target).
//
// Two launches, so that the row reads spread over the whole GPU:
//   * spec_sums_kernel, P workgroups of 4 wavefronts per sequence: each takes
//     the accept tests (a handful of loads, the same for every thread) and
//     sums its share of the row's tiles of 256 tokens - each wavefront four
//     tiles at a time, from four coalesced loads per lane, tile and row - in integer
//     units of 2^-32, both the residual max(target - draft, 0) and the target
//     itself from the same loads (the residual may be empty), into the
//     workspace; workgroup 0 writes the kept count and tokens;
//   * spec_draw_kernel, one workgroup of 16 wavefronts per sequence: scans
//     the tile sums in LDS to find the tile that holds the threshold, and one
//     wavefront scans that tile's tokens in order to the drawn one.
// Integer units make the draw exact and independent of the order of
// summation.
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

// Accept tests of sequence b, left to right: keep x while u * d(x) < t(x) in
// float32; the first rejected position (k when every draft is kept).
__device__ inline int64_t spec_first_rejection(const float* t, const float* d, const int32_t* tokens,
                                               const float* u_accept, int64_t b, int64_t k, int64_t V) {
  for (int64_t i = 0; i < k; ++i) {
    const int32_t x = tokens[b * k + i];
    const bool keep = x >= 0 && x < V && u_accept[b * k + i] * d[i * V + x] < t[i * V + x];
    if (!keep) return i;
  }
  return k;
}

// Workgroup (b, p): the tile sums of sequence b's draw rows, tiles
// p * 4 + w + 4 P i for wavefront w; ws[b][tile] = {residual units, target units}.
__global__ __launch_bounds__(256) void spec_sums_kernel(const float* __restrict__ target,
                                                        const float* __restrict__ draft,
                                                        const int32_t* __restrict__ tokens,
                                                        const float* __restrict__ u_accept, int64_t k, int64_t V,
                                                        int64_t NT, int32_t* __restrict__ n_kept,
                                                        int32_t* __restrict__ out, u64* __restrict__ ws) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t b = blockIdx.x, P = gridDim.y, p = blockIdx.y;
  const float* t = target + b * (k + 1) * V;
  const float* d = draft ? draft + b * k * V : nullptr;
  const int64_t r = spec_first_rejection(t, d, tokens, u_accept, b, k, V);
  if (p == 0) {
    int32_t* o = out + b * (k + 1);
    for (int64_t i = tid; i <= k; i += 256)
      if (i != r) o[i] = i < r ? tokens[b * k + i] : -1;
    if (tid == 0) n_kept[b] = int32_t(r);
  }
  const float* tr = t + r * V;
  const float* dr = r < k ? d + r * V : nullptr;
  u64* wsb = ws + b * NT * 2;
  // four of the wavefront's tiles per round, all their loads issued before any sum
  for (int64_t t0 = p * 4 + wave; t0 < NT; t0 += 16 * P) {
    float tv[4][4], dv[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t jq = (t0 + 4 * P * u) * kSpecTile + lane + 64 * q;
        const bool in = t0 + 4 * P * u < NT && jq < V;
        tv[u][q] = in ? tr[jq] : 0.0f;
        dv[u][q] = in && dr ? dr[jq] : 0.0f;
      }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t ti = t0 + 4 * P * u;
      u64 sr = 0, st = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        st += draw_unit(tv[u][q]);
        if (dr) sr += draw_unit(fmaxf(tv[u][q] - dv[u][q], 0.0f));
      }
      for (int m = 32; m > 0; m >>= 1) {
        sr += __shfl_xor(sr, m);
        st += __shfl_xor(st, m);
      }
      if (lane == 0 && ti < NT) {
        wsb[2 * ti] = sr;
        wsb[2 * ti + 1] = st;
      }
    }
  }
}

// One workgroup per sequence: the draw from the tile sums.
__global__ __launch_bounds__(kSpecThreads) void spec_draw_kernel(const float* __restrict__ target,
                                                                 const float* __restrict__ draft,
                                                                 const float* __restrict__ u_draw, int64_t k,
                                                                 int64_t V, int64_t NT,
                                                                 const int32_t* __restrict__ n_kept,
                                                                 int32_t* __restrict__ out,
                                                                 const u64* __restrict__ ws) {
  __shared__ u64 s_tile[kSpecMaxTiles];
  __shared__ u64 s_wave[kSpecWaves];
  __shared__ u64 s_pick[2];  // picked tile, units before it
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t b = blockIdx.x;
  const int64_t r = n_kept[b];
  int32_t* o = out + b * (k + 1);
  const float* tr = target + (b * (k + 1) + r) * V;
  const float* dr = r < k ? draft + (b * k + r) * V : nullptr;
  const u64* wsb = ws + b * NT * 2;
  if (tid == 0) {
    s_pick[0] = 0;  // read only after a barrier; always overwritten when T > 0
    s_pick[1] = 0;
  }
  // the residual's sums (rejection), the target's (every draft kept, or an empty residual)
  for (int pass = 0; pass < 2; ++pass) {
    const int which = dr ? 0 : 1;
    for (int64_t i = tid; i < NT; i += kSpecThreads) s_tile[i] = wsb[2 * i + which];
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
      const u64 sw = s_wave[w];
      if (w < wave) wbase += sw;
      T += sw;
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
        const u64 sq = i < NT ? s_tile[i] : 0;
        if (acc + sq > U) {
          s_pick[0] = u64(i);
          s_pick[1] = acc;
          break;
        }
        acc += sq;
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

int64_t spec_tiles(int64_t V) { return (V + kSpecTile - 1) / kSpecTile; }

size_t spec_workspace_bytes(int64_t B, int64_t V) { return size_t(B) * size_t(spec_tiles(V)) * 2 * sizeof(u64); }

hipError_t launch_spec_accept(const float* target, const float* draft, const int32_t* tokens, const float* u_accept,
                              const float* u_draw, int64_t B, int64_t k, int64_t V, int32_t* n_kept, int32_t* out,
                              void* ws, hipStream_t st) {
  const int64_t NT = spec_tiles(V);
  // about 2048 workgroups of 4 wavefronts in all, each at least one tile per wavefront
  int64_t P = (2048 + B - 1) / B;
  const int64_t pmax = (NT + 3) / 4;
  if (P > pmax) P = pmax;
  if (P < 1) P = 1;
  hipLaunchKernelGGL(spec_sums_kernel, dim3(unsigned(B), unsigned(P)), dim3(256), 0, st, target, draft, tokens,
                     u_accept, k, V, NT, n_kept, out, reinterpret_cast<u64*>(ws));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(spec_draw_kernel, dim3(unsigned(B)), dim3(kSpecThreads), 0, st, target, draft, u_draw, k, V, NT,
                     n_kept, out, reinterpret_cast<const u64*>(ws));
  return hipGetLastError();
}

}  // namespace wqd
