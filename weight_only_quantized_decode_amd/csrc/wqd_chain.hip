// A chain of decode linear layers in one persistent launch.
//
// A decode step runs a layer's matrices one after another, each reading the
// previous one's output (CS336 lecture 10 notes, section 3.2: the attention
// projections, then the MLP's gate/up and down), and a step made of many
// small kernels pays a launch cost for each ("Only Accepted Tokens Count"
// reading notes, on why paired experiments turn CUDA graphs on).  Even
// replayed from a graph, every launch of the streaming kernel pays several
// microseconds of fixed cost at decode sizes (dispatch, the first memory
// round trip, the tail).  Here one launch runs the whole chain: the weights
// of the next matrix never depend on the previous output, so they stream
// while the previous matrix finishes, and only the products wait.
//
// Work: items (call c, two 16-row blocks), numbered call by call and dealt to
// the G workgroups round robin (workgroup g takes items g, g + G, ...).  The
// kChainWaves wavefronts of a workgroup split K into contiguous shares (a
// multiple of 8 tiles) and multiply with the broadcast kernel's per-tile
// arithmetic (wqd_bcast_tile.h), each x register serving both row blocks:
// two register groups of 4 tiles of both blocks in flight, each refilled as
// soon as it is consumed.  The last two refills of an item
// load the first two groups of the workgroup's next item: weights, scales and
// zero points always, x too when the next item belongs to the same call.
//
// Dependencies: a call's x may be an earlier call's y (wait_for).  Before the
// first product of such a call, wavefront 0 of the workgroup polls that
// call's completion counters until they sum to its item count, while the
// other wavefronts wait at a barrier.  After its last item of a call, a
// workgroup adds the number of that call's items it finished to counter
// (workgroup % kChainCounters) of the call; spreading the adds over 64
// counters in separate 128-byte lines keeps them from serialising on one
// address.  x is read with agent-scope coherent loads and y written with
// agent-scope coherent stores, so an output stored from one XCD is seen by
// loads on another without a cache write-back or invalidate; the storing
// wavefront waits for its stores to complete before it adds to the counter.
//
// Progress: items are dealt in call order and a call waits only on earlier
// calls, so with every workgroup resident (the grid is at most the resident
// capacity, and the device runs nothing else meanwhile) every wait ends.
// Each wait is also bounded in time: past the bound the waiting wavefront
// sets the workspace's error flag, every workgroup that sees it stops, and
// the host reads the flag (wqd_chain_status).  Counters and flag are cleared
// by a small kernel launched just before the chain (no memset, so the pair
// can be captured in a graph).
#include "wqd_bcast_tile.h"
#include "wqd_device.h"
#include "wqd_internal.h"
#include "wqd_plan.h"

namespace wqd {

// Pointers read from the call table are generic to the compiler, which would
// access them with flat instructions (counted on both the vector-memory and
// the LDS counters, and waited for with vmcnt(0)).  They all point to global
// memory, so they are used through the global address space.
#define WQD_GLOBAL __attribute__((address_space(1)))

template <class T>
__device__ __forceinline__ const WQD_GLOBAL T* gptr(const void* p) {
  return (const WQD_GLOBAL T*)(p);
}

__device__ __forceinline__ uint64_t ld_coherent(const WQD_GLOBAL uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_coherent(const WQD_GLOBAL uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Groups of 4 tiles per wavefront share at most (the straight-line steps):
// shares of up to 64 W4A16, 128 FP8 or 256 BF16 tiles, K <= 32768.
template <int FMT>
struct ChainNG {
  static constexpr int value = FMT == kFmtW4 ? 16 : FMT == kFmtFP8 ? 32 : 64;
};

// One item as one wavefront sees it (uniform over the wavefront except the
// per-lane scale and zero-point bases).
struct CItem {
  const WQD_GLOBAL uint16_t* x;
  const WQD_GLOBAL uint64_t* sbase;  // 4 fp16 scales per (row, scale quad), first row block
  const WQD_GLOBAL uint16_t* zbase;
  __amdgpu_buffer_rsrc_t wres[kChainRB];  // one per row block (range 0 for a block past N)
  int64_t K, KT, kt_begin, nbi;  // nbi: the item's first 16-row block
  int64_t sstride;               // scale / zero entries from one row block to the next
  int total;  // tiles of this wavefront's share (0 .. per_wave)
  int ng;     // groups of 4 tiles per share (even, the same for every wavefront)
  int call;
};

template <int FMT>
__device__ __forceinline__ CItem make_item(const ChainCall* __restrict__ calls, int c, int64_t item, int wave, int n,
                                           bool live) {
  const ChainCall& cc = calls[c];
  CItem it;
  const int64_t nbi = item * kChainRB;
  it.call = c;
  it.nbi = nbi;
  it.x = gptr<uint16_t>(cc.x);
  it.K = cc.K;
  it.KT = cc.KT;
  it.kt_begin = int64_t(wave) * cc.per_wave;
  const int64_t rem = cc.KT - it.kt_begin;
  it.total = rem <= 0 ? 0 : (rem < cc.per_wave ? int(rem) : cc.per_wave);
  it.ng = cc.per_wave / 4;
  // an item that is not there (past the workgroup's last), or a row block
  // past the matrix, reads zeros
#pragma unroll
  for (int b = 0; b < kChainRB; ++b) {
    const bool there = live && nbi + b < cc.nb;
    const uint4* w = reinterpret_cast<const uint4*>(cc.w) +
                     ((there ? nbi + b : 0) * cc.KT + (it.total > 0 ? it.kt_begin : 0)) * (kTileBytes / 16);
    it.wres[b] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint4*>(w), 0, there ? it.total * kTileBytes : 0,
                                                   0x00020000);
  }
  // a second row block past the matrix reads the first one's scales (its
  // products are never stored)
  it.sstride = nbi + 1 < cc.nb ? cc.G4 * kTileRows : 0;
  if (FMT == kFmtW4) {
    const int64_t q0 = (nbi * cc.G4 + (it.total > 0 ? it.kt_begin / kScaleQuad : 0)) * kTileRows + n;
    it.sbase = gptr<uint64_t>(cc.scales) + q0;
    it.zbase = gptr<uint16_t>(cc.zeros) + q0;
  } else {
    it.sbase = nullptr;
    it.zbase = nullptr;
  }
  return it;
}

// The registers of one group of 4 tiles: both row blocks' weights, scales
// and zero points, and the x registers they share.
template <int FMT, int MR>
struct CGroup {
  uint4 w[kChainRB][4];
  XReg<FMT> x[MR][BcC<FMT>::XR];
  uint2 s[kChainRB];
  uint32_t z[kChainRB];
};

// Row block B of a group as the broadcast kernel's register group.
template <int FMT, int MR, int B>
__device__ __forceinline__ BGroup<FMT, MR> block_view(const CGroup<FMT, MR>& g) {
  BGroup<FMT, MR> v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v.w[i] = g.w[B][i];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int r = 0; r < BcC<FMT>::XR; ++r) v.x[m][r] = g.x[m][r];
  v.s = g.s[B];
  v.z = g.z[B];
  return v;
}

// The x registers of tiles t0 .. t0 + 3 (coherent loads, clamped to the
// share's last tile and into the row).  The loaded values are not touched
// here, so the loads stay in flight; dwords past K (a ragged last FP8 / BF16
// tile) are zeroed when the group is multiplied (zero_ragged_x).
template <int FMT, int MR>
__device__ __forceinline__ void load_x(CGroup<FMT, MR>& g, const CItem& it, int t0, int kb, int j) {
  using C = BcC<FMT>;
  const int last = it.total > 0 ? it.total - 1 : 0;
#pragma unroll
  for (int r = 0; r < C::XR; ++r) {
    const int tt = min(t0 + r * C::TPX + j / C::LPS, last);
    const int64_t k = (it.kt_begin + tt) * C::TK + kb * C::SLK + 2 * C::XW * (j % C::LPS);
    const int64_t kc = k < it.K ? k : it.K - 2 * C::XW;
#pragma unroll
    for (int m = 0; m < MR; ++m) g.x[m][r] = ld_coherent((const WQD_GLOBAL XReg<FMT>*)(it.x + int64_t(m) * it.K + kc));
  }
}

// Loads of tiles t0 .. t0 + 3 of item `it`: weights through the share's
// buffer resource (tiles past the share read zero without touching memory),
// the x registers, and the W4A16 scale and zero quad.
// Every index is clamped into the item's rows, so the same loads are issued
// whatever the share holds: the compiler's waits stay exact.
template <int FMT, int MR>
__device__ __forceinline__ void load_group(CGroup<FMT, MR>& g, const CItem& it, int t0, int lane, int kb, int j) {
#pragma unroll
  for (int b = 0; b < kChainRB; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(it.wres[b], (t0 + i) * kTileBytes + lane * 16, 0, 2);
      g.w[b][i] = make_uint4(v.x, v.y, v.z, v.w);
    }
  load_x<FMT, MR>(g, it, t0, kb, j);
  if (FMT == kFmtW4) {
    const int q = min(t0, it.total > 0 ? it.total - 1 : 0) / kScaleQuad;
#pragma unroll
    for (int b = 0; b < kChainRB; ++b) {
      const uint64_t sq = it.sbase[b * it.sstride + q * kTileRows];
      g.s[b] = make_uint2(uint32_t(sq), uint32_t(sq >> 32));
      g.z[b] = it.zbase[b * it.sstride + q * kTileRows];
    }
  }
}

// W4A16 x sums of 16 tiles: lane (kb, n) takes slice kb of tile 16 c + n of
// the share (clamped to the share's last tile and to the row), 32 values per
// row as 8 coherent 8-byte loads.
template <int MR>
__device__ __forceinline__ void load_xs(uint4 (&xs)[MR][4], const CItem& it, int c, int kb, int n) {
  const int last = it.total > 0 ? it.total - 1 : 0;
  const int64_t tile = min(it.kt_begin + min(16 * c + n, last), it.KT - 1);
  const int64_t k0 = tile * kGroup + kb * (kGroup / 4);
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    const WQD_GLOBAL uint64_t* p = (const WQD_GLOBAL uint64_t*)(it.x + int64_t(m) * it.K + k0);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint64_t lo = ld_coherent(p + 2 * u), hi = ld_coherent(p + 2 * u + 1);
      xs[m][u] = make_uint4(uint32_t(lo), uint32_t(lo >> 32), uint32_t(hi), uint32_t(hi >> 32));
    }
  }
}

// x dwords past K read as the row's last dwords; before the multiply they
// are zeroed (a W4A16 row is whole groups of 128, so K is never ragged).
template <int FMT, int MR>
__device__ __forceinline__ void zero_ragged_x(CGroup<FMT, MR>& g, const CItem& it, int t0, int kb, int j) {
  using C = BcC<FMT>;
  if constexpr (FMT != kFmtW4) {
    if (it.K % C::TK != 0) {
      const int last = it.total > 0 ? it.total - 1 : 0;
#pragma unroll
      for (int r = 0; r < C::XR; ++r) {
        const int tt = min(t0 + r * C::TPX + j / C::LPS, last);
        const int64_t k = (it.kt_begin + tt) * C::TK + kb * C::SLK + 2 * C::XW * (j % C::LPS);
#pragma unroll
        for (int m = 0; m < MR; ++m) g.x[m][r] = k < it.K ? g.x[m][r] : XReg<FMT>(0);
      }
    }
  }
}

// Group S of the current item (tiles 4S .. 4S + 3, fewer at the end of a
// ragged share), then the refill of its registers: group S + 2 of this item,
// or past the item's end group S + 2 - ng of the next one (selected, not
// branched on).
template <int FMT, int MR, int XC, int S>
__device__ __forceinline__ void cstep(CGroup<FMT, MR>& g, const CItem& cur, const CItem& nxt,
                                      const float (&X)[MR][XC], float (&acc)[kChainRB][MR], int lane, int kb,
                                      int j) {
  static_assert(kChainRB == 2, "the two row blocks of an item");
  const int left = cur.total - 4 * S;
  zero_ragged_x<FMT, MR>(g, cur, 4 * S, kb, j);
  const BGroup<FMT, MR> g0 = block_view<FMT, MR, 0>(g), g1 = block_view<FMT, MR, 1>(g);
  if (left >= 4) {
    btile<FMT, MR, XC, 0, 4 * S + 0>(g0, X, acc[0]);
    btile<FMT, MR, XC, 0, 4 * S + 0>(g1, X, acc[1]);
    btile<FMT, MR, XC, 1, 4 * S + 1>(g0, X, acc[0]);
    btile<FMT, MR, XC, 1, 4 * S + 1>(g1, X, acc[1]);
    btile<FMT, MR, XC, 2, 4 * S + 2>(g0, X, acc[0]);
    btile<FMT, MR, XC, 2, 4 * S + 2>(g1, X, acc[1]);
    btile<FMT, MR, XC, 3, 4 * S + 3>(g0, X, acc[0]);
    btile<FMT, MR, XC, 3, 4 * S + 3>(g1, X, acc[1]);
  } else if (left > 0) {
    btile<FMT, MR, XC, 0, 4 * S + 0>(g0, X, acc[0]);
    btile<FMT, MR, XC, 0, 4 * S + 0>(g1, X, acc[1]);
    if (left > 1) {
      btile<FMT, MR, XC, 1, 4 * S + 1>(g0, X, acc[0]);
      btile<FMT, MR, XC, 1, 4 * S + 1>(g1, X, acc[1]);
    }
    if (left > 2) {
      btile<FMT, MR, XC, 2, 4 * S + 2>(g0, X, acc[0]);
      btile<FMT, MR, XC, 2, 4 * S + 2>(g1, X, acc[1]);
    }
  }
  const bool in_item = S + 2 < cur.ng;
  CItem src;
  src.x = in_item ? cur.x : nxt.x;
  src.sbase = in_item ? cur.sbase : nxt.sbase;
  src.zbase = in_item ? cur.zbase : nxt.zbase;
#pragma unroll
  for (int b = 0; b < kChainRB; ++b) src.wres[b] = in_item ? cur.wres[b] : nxt.wres[b];
  src.sstride = in_item ? cur.sstride : nxt.sstride;
  src.K = in_item ? cur.K : nxt.K;
  src.KT = in_item ? cur.KT : nxt.KT;
  src.kt_begin = in_item ? cur.kt_begin : nxt.kt_begin;
  src.total = in_item ? cur.total : nxt.total;
  load_group<FMT, MR>(g, src, in_item ? 4 * (S + 2) : 4 * (S + 2 - cur.ng), lane, kb, j);
  // issue the refill here: left to itself the scheduler sinks loads to just
  // before their use, which would leave one group in flight instead of two
  __builtin_amdgcn_sched_barrier(0);
}

// Steps S .. ng - 1 as straight-line code with an early exit (no loop, so the
// compiler's load-counter waits stay exact); groups alternate between g0
// (even) and g1 (odd).  The W4A16 x sums of tiles 16 c .. 16 c + 15 are
// formed just before their first group, from loads issued one register ahead.
template <int FMT, int MR, int XC, int S>
__device__ __forceinline__ void csteps(CGroup<FMT, MR>& g0, CGroup<FMT, MR>& g1, const CItem& cur, const CItem& nxt,
                                       float (&X)[MR][XC], uint4 (&xs)[MR][4], float (&acc)[kChainRB][MR], int lane,
                                       int kb, int n) {
  if constexpr (S < 4 * XC) {
    if constexpr (FMT == kFmtW4 && S % 4 == 0 && S > 0) {
      xsums<FMT, MR, XC>(X, xs, S / 4);
      if constexpr (S / 4 + 1 < XC) load_xs<MR>(xs, cur, S / 4 + 1, kb, n);
    }
    cstep<FMT, MR, XC, S>(S % 2 == 0 ? g0 : g1, cur, nxt, X, acc, lane, kb, n);
    if (S + 1 < cur.ng) csteps<FMT, MR, XC, S + 1>(g0, g1, cur, nxt, X, xs, acc, lane, kb, n);
  }
}

// A workgroup barrier that waits for LDS only: __syncthreads() would also
// wait for every load in flight, the next item's weights included.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Wavefront 0 polls call d's counters until they sum to its item count; the
// others wait at the barrier.  False when the wait was abandoned (time bound
// passed, or another workgroup set the error flag).
__device__ __forceinline__ bool chain_wait(const ChainCall* __restrict__ calls, int d, const int* counters,
                                           int* flag, int* s_flag, int wave, int lane, long long ticks) {
  if (wave == 0) {
    const int target = calls[d].ni;
    const int* cnt = counters + int64_t(d) * kChainCounters * kChainCounterStride;
    const long long start = (long long)__builtin_amdgcn_s_memrealtime();
    int abort = 0;
    while (true) {
      int v = __hip_atomic_load(cnt + lane * kChainCounterStride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
      if (__builtin_amdgcn_readfirstlane(v) >= target) break;
      const int f = __builtin_amdgcn_readfirstlane(__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      if (f != 0 || (long long)__builtin_amdgcn_s_memrealtime() - start > ticks) {
        if (f == 0 && lane == 0) __hip_atomic_store(flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        abort = 1;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (lane == 0) *s_flag = abort;
  }
  lds_barrier();
  return *s_flag == 0;
}

static_assert(kChainCounters == 64, "one counter per lane of the polling wavefront");

template <int FMT, int MR>
__global__ __launch_bounds__(64 * kChainWaves) void chain_kernel(const ChainHeader* __restrict__ hdr,
                                                                 const ChainCall* __restrict__ calls, int ncalls,
                                                                 int total_items, int* counters, int* flag,
                                                                 long long ticks) {
  __shared__ float s_red[2][kChainWaves][kChainRB][MR][kTileRows];
  __shared__ int s_flag;
  const int lane = threadIdx.x & 63, kb = lane >> 4, n = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (hdr->magic != kChainMagic || hdr->fmt != FMT || hdr->M != MR || hdr->ncalls != ncalls ||
      hdr->total_items != total_items || hdr->grid != int(gridDim.x)) {
    if (threadIdx.x == 0) __hip_atomic_store(flag, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  constexpr int XC = ChainNG<FMT>::value / 4;
  const int G = gridDim.x;
  int j = blockIdx.x;
  if (j >= total_items) return;
  int c = 0;
  while (c + 1 < ncalls && j >= calls[c].item0 + calls[c].ni) ++c;
  CItem cur = make_item<FMT>(calls, c, j - calls[c].item0, wave, n, true);
  CGroup<FMT, MR> g0, g1;
  load_group<FMT, MR>(g0, cur, 0, lane, kb, n);
  load_group<FMT, MR>(g1, cur, 4, lane, kb, n);
  __builtin_amdgcn_sched_barrier(0);
  bool x_ready = false;  // x in g0, g1 (and xs0) was read after this call's wait
  int waited = -1;
  int par = 0;
  int done = 0;  // items of the current call this workgroup has finished
  uint4 xs0[MR][4];  // W4A16: x sums of the first 16 tiles of the current item
  while (true) {
    // wait_for names an earlier call (the table was checked when it was
    // written; the bound keeps a damaged table from indexing past it)
    const int d = calls[cur.call].wait_for;
    if (d >= 0 && d < cur.call && d != waited) {
      if (!chain_wait(calls, d, counters, flag, &s_flag, wave, lane, ticks)) return;
      waited = d;
      x_ready = false;
    }
    if (!x_ready) {
      load_x<FMT, MR>(g0, cur, 0, kb, n);
      load_x<FMT, MR>(g1, cur, 4, kb, n);
      if constexpr (FMT == kFmtW4) load_xs<MR>(xs0, cur, 0, kb, n);
    }
    const int jn = j + G;
    const bool has_next = jn < total_items;
    int cn = cur.call;
    while (cn + 1 < ncalls && jn >= calls[cn].item0 + calls[cn].ni) ++cn;
    const CItem nxt = make_item<FMT>(calls, cn, has_next ? jn - calls[cn].item0 : 0, wave, n, has_next);
    const bool next_same = has_next && cn == cur.call;

    float acc[kChainRB][MR];
    float X[MR][XC];
#pragma unroll
    for (int m = 0; m < MR; ++m) {
#pragma unroll
      for (int b = 0; b < kChainRB; ++b) acc[b][m] = 0.f;
#pragma unroll
      for (int q = 0; q < XC; ++q) X[m][q] = 0.f;
    }
    uint4 xs[MR][4];
    if constexpr (FMT == kFmtW4) {
      // this item's first x sums were loaded during the previous item; the
      // next item's go out now, a whole item ahead of their use (reloaded
      // after a wait when the next item belongs to another call)
      xsums<FMT, MR, XC>(X, xs0, 0);
      load_xs<MR>(xs0, nxt, 0, kb, n);
      if constexpr (XC > 1) load_xs<MR>(xs, cur, 1, kb, n);
    }
    csteps<FMT, MR, XC, 0>(g0, g1, cur, nxt, X, xs, acc, lane, kb, n);

    // the 4 slices of a row (lanes n, n+16, n+32, n+48), then the wavefronts
    // in order through LDS (two buffers: the next item's writes never meet
    // this item's reads, which end before the next barrier)
#pragma unroll
    for (int b = 0; b < kChainRB; ++b)
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        float v = acc[b][m];
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        if (kb == 0) s_red[par][wave][b][m][n] = v;
      }
    lds_barrier();
    if (wave == 0) {
      const ChainCall& cc = calls[cur.call];
      if (lane < kChainRB * MR * kTileRows) {
        const int b = lane / (MR * kTileRows), m = (lane / kTileRows) % MR, r = lane % kTileRows;
        float v = s_red[par][0][b][m][r];
#pragma unroll
        for (int w = 1; w < kChainWaves; ++w) v += s_red[par][w][b][m][r];
        const int64_t row = (cur.nbi + b) * kTileRows + r;
        const bool live = row < cc.N;
        if (FMT == kFmtFP8 && live) v *= gptr<float>(cc.scales)[row];
        WQD_GLOBAL uint16_t* y = (WQD_GLOBAL uint16_t*)(cc.y);
        // as store_out<8>, with coherent stores (lane ^ 8 holds row ^ 8)
        if (!cc.swiglu) {
          if (live)
            __hip_atomic_store(y + m * cc.N + row, uint16_t(f32_to_bf16_rne(v)), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        } else {
          const float u = __shfl_xor(v, 8);
          if (live && (row & 8) == 0) {
            const float h = v / (1.0f + expf(-v)) * u;
            __hip_atomic_store(y + m * (cc.N / 2) + (row >> 4) * 8 + (row & 7), uint16_t(f32_to_bf16_rne(h)),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      }
      // After the workgroup's last item of this call, once every store of its
      // items has completed (and with them this wavefront's loads in flight),
      // the items count as done: one add per workgroup and call.
      ++done;
      if (!next_same) {
        __builtin_amdgcn_s_waitcnt(0);
        if (lane == 0)
          __hip_atomic_fetch_add(counters + (int64_t(cur.call) * kChainCounters + blockIdx.x % kChainCounters) *
                                                kChainCounterStride,
                                 done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        done = 0;
      }
    }
    if (!has_next) break;
    cur = nxt;
    j = jn;
    x_ready = next_same;
    par ^= 1;
  }
}

__global__ void chain_clear_kernel(int* counters, int n, int* flag) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) counters[int64_t(i) * kChainCounterStride] = 0;
  if (i == 0) *flag = 0;
}

template <int FMT, int MR>
static const void* chain_symbol() {
  return reinterpret_cast<const void*>(&chain_kernel<FMT, MR>);
}

static const void* chain_kernel_for(int fmt, int M) {
  if (M == 1) {
    if (fmt == kFmtBF16) return chain_symbol<kFmtBF16, 1>();
    if (fmt == kFmtFP8) return chain_symbol<kFmtFP8, 1>();
    return chain_symbol<kFmtW4, 1>();
  }
  if (fmt == kFmtBF16) return chain_symbol<kFmtBF16, 2>();
  if (fmt == kFmtFP8) return chain_symbol<kFmtFP8, 2>();
  return chain_symbol<kFmtW4, 2>();
}

hipError_t chain_resident_workgroups(int fmt, int M, int* out) {
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, chain_kernel_for(fmt, M), 64 * kChainWaves, 0);
  if (e != hipSuccess) return e;
  *out = cus * per_cu;
  return hipSuccess;
}

hipError_t chain_compute_units(int* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  return hipDeviceGetAttribute(out, hipDeviceAttributeMultiprocessorCount, dev);
}

template <int FMT, int MR>
static void launch_chain_t(unsigned grid, const ChainHeader* hdr, const ChainCall* calls, int ncalls, int total,
                           int* counters, int* flag, long long ticks, hipStream_t st) {
  hipLaunchKernelGGL((chain_kernel<FMT, MR>), dim3(grid), dim3(64 * kChainWaves), 0, st, hdr, calls, ncalls, total,
                     counters, flag, ticks);
}

hipError_t launch_chain(int fmt, int M, int ncalls, int total_items, int grid, long long ticks, void* ws,
                        hipStream_t st) {
  if (M < 1 || M > kChainMaxM || grid < 1 || ncalls < 1) return hipErrorInvalidValue;
  char* base = reinterpret_cast<char*>(ws);
  const ChainHeader* hdr = reinterpret_cast<const ChainHeader*>(base);
  int* flag = reinterpret_cast<int*>(base + 128);
  const ChainCall* calls = reinterpret_cast<const ChainCall*>(base + chain_table_offset());
  int* counters = reinterpret_cast<int*>(base + chain_counters_offset(ncalls));
  const int nctr = ncalls * kChainCounters;
  hipLaunchKernelGGL(chain_clear_kernel, dim3(unsigned((nctr + 255) / 256)), dim3(256), 0, st, counters, nctr, flag);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned g = unsigned(grid);
  if (M == 1) {
    if (fmt == kFmtBF16) launch_chain_t<kFmtBF16, 1>(g, hdr, calls, ncalls, total_items, counters, flag, ticks, st);
    else if (fmt == kFmtFP8) launch_chain_t<kFmtFP8, 1>(g, hdr, calls, ncalls, total_items, counters, flag, ticks, st);
    else launch_chain_t<kFmtW4, 1>(g, hdr, calls, ncalls, total_items, counters, flag, ticks, st);
  } else {
    if (fmt == kFmtBF16) launch_chain_t<kFmtBF16, 2>(g, hdr, calls, ncalls, total_items, counters, flag, ticks, st);
    else if (fmt == kFmtFP8) launch_chain_t<kFmtFP8, 2>(g, hdr, calls, ncalls, total_items, counters, flag, ticks, st);
    else launch_chain_t<kFmtW4, 2>(g, hdr, calls, ncalls, total_items, counters, flag, ticks, st);
  }
  return hipGetLastError();
}

}  // namespace wqd
