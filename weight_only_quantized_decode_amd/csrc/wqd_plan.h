// Packed layout geometry, argument validation and launch planning.
// Pure host C++: no HIP headers, so it is the same code on a GPU-less host.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace wqd {

// A tile is 16 output rows x 4 slices x 16 bytes = 1 KiB.  Inside a tile,
// slice j of row r sits at byte (16 j + r) * 16, so lane l = 16 j + r of a
// 64-wide wavefront loads 16 bytes at l * 16: one fully contiguous 1 KiB load
// per wavefront.  The same lane order is the B-operand order of the bf16
// matrix-core instructions (lane = 16 * k_block + column).  Each row holds
// 64 bytes of K per tile; tiles of one 16-row block are consecutive along K.
constexpr int kTileRows = 16;
constexpr int kSlices = 4;
constexpr int kSliceBytes = 16;
constexpr int kTileBytes = kTileRows * kSlices * kSliceBytes;  // 1024
constexpr int kGroup = 128;  // W4A16 group length along K (= one tile's K extent)
constexpr int kScaleQuad = 4;  // W4A16 scales / zeros are stored 4 groups per row together

constexpr int kFmtBF16 = 0;
constexpr int kFmtFP8 = 1;
constexpr int kFmtW4 = 2;

// K elements covered by one tile: 64 bytes per row.
inline int tile_k(int fmt) { return fmt == kFmtBF16 ? 32 : fmt == kFmtFP8 ? 64 : 128; }
inline bool fmt_ok(int fmt) { return fmt == kFmtBF16 || fmt == kFmtFP8 || fmt == kFmtW4; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct PackedSizes {
  int64_t NB;     // 16-row blocks
  int64_t KT;     // tiles along K
  int64_t G4;     // W4A16: groups of 4 K-groups (scale / zero storage unit)
  size_t w_bytes, s_bytes, z_bytes;
};

// Status codes mirror enum wqd_status in include/wqd.h.
enum { kOK = 0, kEArg = 1, kEShape = 2, kEAlign = 3, kEWorkspace = 4, kEHip = 5, kEUnsupported = 6 };

int packed_sizes(int fmt, int64_t N, int64_t K, PackedSizes* out);

// Streaming kernel (M <= 8): one workgroup per 16-row block over all of K.
constexpr int kGemvMaxM = 8;

struct GemvPlan {
  int64_t NB, KT;
  int mrows;    // rows per launch (M, or kGemvMaxM when M is processed in chunks)
  int nchunks;  // launches over M
  int waves;    // wavefronts per workgroup (each takes a contiguous share of K)
};

int plan_gemv(int fmt, int64_t M, int64_t N, int64_t K, GemvPlan* out);

// Row-broadcast streaming kernel (M <= 2 for W4A16, M <= 8 for FP8 and
// BF16): like the above, but x is read from L2 per tile and broadcast across
// the lanes of a DPP row, so no LDS staging.  W wavefronts (4, 8 or 16) per
// 16-row block, each on a share of per_wave tiles (a multiple of 4, at most
// 32: straight-line code over `groups` = 4 or 8 groups of 4 tiles; at most 16
// tiles for three or more rows, or two W4A16 rows); kEUnsupported when K is
// too long for that.
constexpr int kBcastMaxM = 8;
constexpr int kBcastMaxMW4 = 2;

struct BcastPlan {
  int64_t NB, KT;
  int waves, per_wave, groups;
};

int plan_bcast(int fmt, int64_t M, int64_t N, int64_t K, BcastPlan* out);

// Streaming matrix-core kernel (M <= 16): the same work split (4, 8 or 16
// wavefronts per workgroup), with the products on bf16 matrix cores (x
// fragments read from L2 per tile).  Shares of at most 32 tiles; kEUnsupported when K is too long for that or the x
// rows span 2 GiB or more.
constexpr int kMcMaxM = 16;

struct McPlan {
  int64_t NB, KT;
  int waves, per_wave;
  int rb;  // 16-row blocks per wavefront (1, 2 or 3): x fragments shared by rb weight tiles
};

int plan_mc(int fmt, int64_t M, int64_t N, int64_t K, McPlan* out);

// Skinny matrix-core kernel (9 to 64 rows): a workgroup of `waves` consumer
// wavefronts (plus a producer that stages x, scales and zero points in LDS
// and computes the W4A16 x sums) owns waves x rb 16-row blocks
// (`groups` workgroups cover the matrix), mf 16-row blocks of x, and chunks
// of ct tiles.  K is split S ways (per_split tiles each, a multiple of ring)
// when the row blocks alone give too few workgroups; the S float32 partials
// then need S * M * N * 4 bytes of workspace.  kEUnsupported above 64 rows,
// for x rows spanning 2 GiB or more, and for K not a whole number of tiles.
constexpr int kSkMaxM = 64;

struct SkPlan {
  int64_t NB, KT, groups;
  int mf, rb, waves;
  int ring, ct, nx;  // weight ring slots (tiles), tiles per x chunk, x chunk buffers
  int S, per_split;
  size_t ws_bytes;
};

// The skinny kernel's (consumer wavefronts, row blocks per consumer)
// configurations: the planner chooses among them and the kernel file
// instantiates every one for 1 to 4 x row blocks.
constexpr int kSkCfgCount = 4;
constexpr int kSkCfg[kSkCfgCount][2] = {{7, 2}, {7, 1}, {4, 2}, {5, 2}};

int plan_skinny(int fmt, int64_t M, int64_t N, int64_t K, SkPlan* out);

// Tiled matrix-core kernel (more than kGmMinM rows and at least kGmMinNBN
// column blocks): wm = 1, a 64 x 256 tile of y (BF16 / FP8 up to 256 rows: 4
// wavefronts of 64 x 64; W4A16: 8 of 64 x 32), or wm = 2, 128-row wavefront
// tiles (BF16 / FP8 above 256 rows: a 256 x 256 tile, 8 wavefronts of
// 128 x 64; W4A16 where the time model puts it faster: 128 x 256, 8 of
// 128 x 32); NBN column blocks x MB row blocks of workgroups (XCD-aware
// order), K in chunks (64; W4A16 128) split S ways (cps chunks per split) as
// the time model picks.
// Workspace: W4A16 x sums, float32 [KT][Mp] (Mp = MB rows per block), xs_bytes
// rounded up to 256; then the S float32 partials, S * M * N * 4 bytes when
// S > 1.  kEUnsupported for x rows spanning 2 GiB or more.
constexpr int kGmMinM = 64;
constexpr int64_t kGmMinNBN = 16;

struct GmPlan {
  int64_t NB, KT, NBN, MB, nchunks, cps, Mp;
  int wm, S;
  int64_t nbn1;  // tail split (S2 > 0, S == 1): column blocks from nbn1 split S2 ways (cps2 chunks each)
  int S2, cps2;
  int rbw;  // LDS-staged form (wm 3): weight row blocks per wavefront ...
  int lwr;  // ... and wavefront rows of 64 rows: tiles of 64 lwr rows by (8 / lwr) rbw row blocks
  size_t xs_bytes, ws_bytes;
};

int plan_gemm(int fmt, int64_t M, int64_t N, int64_t K, GmPlan* out);

// Matrix-core kernel (M > 8): workgroup tile = 16 * BMS rows of x times
// 4 wavefronts x BNT 16-column tiles; the K loop advances in chunks of TPC
// tiles.  When that leaves fewer than ~2 workgroups per compute unit, K is
// split S ways over workgroups; the S float32 partial tiles go to the
// workspace and a second kernel adds them in split order (deterministic, no
// atomics, no device-scope fences).
struct MfmaPlan {
  int BMS, BNT, TPC;
  int64_t NB, KT, NBB, MB, chunks;
  int S;                // K splits
  int64_t chunks_per_split;
  size_t ws_bytes;      // S * M * N * 4 when S > 1
};

int plan_mfma(int fmt, int64_t M, int64_t N, int64_t K, MfmaPlan* out);

// The kernel family for a shape, in order of preference (measured on the
// 70B shapes): the broadcast kernel for 1 W4A16 row or up to 4 FP8 / BF16
// rows (FP8 at 4 rows only where the skinny kernel's shares are not long);
// up to 8 rows the skinny matrix-core kernel where its K shares are
// at least 48 tiles long and unsplit (or split, at 8 rows), else the
// streaming matrix-core kernel; the broadcast kernel again, then the staged
// one, up to 8 rows where those cannot take the shape; from 9 to 16 rows
// the streaming matrix-core kernel on matrices up to 8192 x 8192 that the
// skinny kernel would split over K; the skinny kernel otherwise up to 64
// rows; above that the tiled matrix-core kernel where N has at least
// kGmMinNBN column blocks of 256 (for BF16 and FP8, where its time model
// says so, in the form that stages the weights in LDS as well), else the LDS
// matrix-core kernel.
enum Path { kPathBcast = 0, kPathStaged = 1, kPathMfma = 2, kPathMc = 3, kPathSkinny = 4, kPathGemm = 5, kPathGemmLds = 6 };

struct Choice {
  int path;
  GemvPlan gemv;
  BcastPlan bcast;
  McPlan mc;
  SkPlan sk;
  GmPlan gm;
  MfmaPlan mfma;
};

int choose_path(int fmt, int64_t M, int64_t N, int64_t K, Choice* out);

// Workspace bytes for wqd_qgemm (0: no path needs scratch memory).
int workspace_bytes(int fmt, int64_t M, int64_t N, int64_t K, size_t* out);

// W8A8-FP8 tiled kernel: FP8 activation codes [M, K] times FP8 packed
// weights on v_mfma_f32_16x16x128_f8f6f4.  A workgroup computes a BM x 256
// tile of y with WR x 4 wavefronts of (16 MF rows) x (4 weight row blocks);
// K advances in 128-k chunks (two packed tiles) through NS pipeline stages.
// BM = 16 MF WR: 32 (MF 2), 64 (MF 4) or 128 (MF 8), WR = 1.  K is
// split S ways over grid y when the tiles leave the compute units idle; the
// float32 partials (already times the activation scale) go to the workspace
// and the fixed-order split-K sum applies the row scales.
struct W8Plan {
  int64_t NB, KT, NBN, MB, nchunks, cps;
  int mf, wr, S;
  int lds, rbw, lwr;  // LDS-staged form: tiles of 64 lwr rows by (8 / lwr) rbw weight row blocks
  size_t ws_bytes;
};

int plan_w8a8(int64_t M, int64_t N, int64_t K, W8Plan* out);

// Decode attention split along the context: S splits of `chunk` positions (a
// multiple of the kernel's step: 32 positions over a bf16 cache, 64 over an
// FP8 one) per (sequence, KV head), one workgroup of 4 wavefronts each; with
// S > 1 the partial maxima, sums and outputs take B * Hq * S * (2 + 128)
// floats of workspace.
struct AttnPlan {
  int64_t Lmax;
  int Hq, Hkv, S, chunk;
  int fp8_kv;  // 1: E4M3 codes, one byte per element
  size_t ws_bytes;
};

int plan_attn(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lmax, int64_t D, AttnPlan* out, bool fp8_kv = false);

// The activation quantisation: G workgroups each reduce a contiguous range of
// x to its largest |x| (G <= kActQuantParts, written to the workspace), then
// every workgroup of the quantising kernel reduces the G values itself.
constexpr int kActQuantParts = 1024;
int plan_act_quant(int64_t M, int64_t K, int* parts);

// A chain of decode linear layers in one persistent launch (wqd_chain.hip).
// Items are (call, kChainRB 16-row blocks) pairs, numbered call by call and
// dealt to the workgroups round robin; each workgroup has kChainWaves wavefronts on
// contiguous shares of K (a multiple of 8 tiles, so the two-group register
// ring lines up from one item to the next).  A call whose input is an earlier
// call's output waits for that call's completion counters: kChainCounters
// per call, each in its own 128-byte line, one atomic add per item.
constexpr int kChainWaves = 4;
constexpr int kChainRB = 2;  // 16-row blocks per item, sharing each x register
constexpr int kChainMaxM = 2;
constexpr int kChainCounters = 64;
constexpr int kChainCounterStride = 32;  // ints: 128 bytes
constexpr int kChainMaxCalls = 1 << 16;
constexpr uint32_t kChainMagic = 0x43484e31u;
constexpr size_t kChainHeaderBytes = 256;  // header, then the error flag at byte 128

struct ChainCall {      // one entry of the device table (128 bytes)
  const void* w;        // packed weights, scales, zero points
  const void* scales;
  const void* zeros;
  const void* x;        // bf16 [M][K]
  void* y;              // bf16 [M][N] ([M][N / 2] with swiglu)
  int64_t N, K, KT, G4;
  int32_t per_wave;     // tiles per wavefront share
  int32_t nb;           // 16-row blocks
  int32_t ni;           // items: kChainRB row blocks each (the last may hold fewer)
  int32_t item0;        // number of the call's first item
  int32_t wait_for;     // earlier call whose output x is, or -1
  int32_t swiglu;
  int32_t pad[8];
};
static_assert(sizeof(ChainCall) == 128, "chain table entries are 128 bytes");

struct ChainHeader {
  uint32_t magic;
  int32_t fmt, M, ncalls, total_items, grid;
  int32_t pad[10];
};
static_assert(sizeof(ChainHeader) == 64, "chain header is 64 bytes");

// Fills the shape fields of one call (KT, G4, per_wave, nb) or returns a status.
int plan_chain_call(int fmt, int64_t M, int64_t N, int64_t K, bool swiglu, ChainCall* out);
// Workspace: header and flag, the table, then kChainCounters lines per call.
size_t chain_workspace_bytes(int64_t ncalls);
inline size_t chain_table_offset() { return kChainHeaderBytes; }
inline size_t chain_counters_offset(int64_t ncalls) {
  return (kChainHeaderBytes + size_t(ncalls) * sizeof(ChainCall) + 255) / 256 * 256;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace wqd
