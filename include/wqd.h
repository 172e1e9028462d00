/*
 * wqd.h - C ABI of the weight-only quantized decode linear layer for MI355X (gfx950).
 *
 * The layer is y[M, N] = x[M, K] . W[N, K]^T for the few activation rows of a
 * decode step (M = batch x verify width), with W streamed from HBM in one of
 * three storage formats and dequantised in registers on the fly; activations
 * stay bfloat16 and are never quantised.  Sources for the operation:
 *   - "降低每個 Token 的生成成本" (Making each token cheaper), section
 *     "量化省下什麼" (What quantization saves): a weight-only decode kernel
 *     multiplies the quantised matrix by a full-precision vector, dequantising
 *     the weights on the fly, without quantising activations;
 *   - same page, "權重量化 / 格式" (Weight quantization / Formats): values are
 *     stored in fewer bits with a scale that maps them back; FP8-E4M3 (largest
 *     normal 448); weight-only INT4 with one scale per group of 128 along K,
 *     dequantised to 16 bits before the multiply-accumulate;
 *   - same page, "完整範例" (Worked example: weight bytes per format): one
 *     32-bit scale per row for FP8;
 *   - CS336 lecture 10 notes, section 5.2 "量化": a scale and a zero point per
 *     group; real speed needs kernels that read the low-bit weights directly.
 *
 * Conventions common to every entry point
 *   - Tensor pointers marked "device" are HIP device pointers owned by the
 *     caller.  The library never allocates, frees or retains them.  All must be
 *     16-byte aligned.  Row-major means the last index is contiguous.
 *   - `stream` is a hipStream_t passed as void*; NULL is the default stream.
 *     Every call that touches the device only enqueues work on `stream` and
 *     returns; results are valid once the stream has synchronised.
 *   - Every function returns a wqd_status.  Arguments are validated on the host
 *     before anything is enqueued, so a non-OK return leaves no partial writes.
 *     A failing HIP call returns WQD_E_HIP; wqd_last_hip_error() then gives the
 *     hipError_t of the calling thread.  Nothing prints, throws or aborts.
 *   - Results are bitwise reproducible for the same (fmt, M, N, K) on gfx950:
 *     there are no floating-point atomics.
 *
 * Formats (fmt):
 *   WQD_FMT_BF16       each weight bfloat16 (round to nearest even).
 *   WQD_FMT_FP8_E4M3   OCP E4M3FN codes, one float32 scale per output row:
 *                      s_n = max_k |W[n,k]| / 448 (1 for an all-zero row, at
 *                      least 2^-126), code = nearest E4M3 of W/s_n (ties to
 *                      even, saturating at 448); weight = e4m3(code) * s_n.
 *   WQD_FMT_W4A16_G128 unsigned 4-bit codes q in groups of 128 consecutive k,
 *                      each group with an fp16 scale s and a uint4 zero point z:
 *                      lo = min(0, min W_g), hi = max(0, max W_g),
 *                      s = fp16(fp32(hi - lo) / 15) (2^-24 if that is 0, 65504
 *                      if it overflows, 1 for an all-zero group),
 *                      z = clamp(rint(-lo / s), 0, 15),
 *                      q = clamp(rint(W / s) + z, 0, 15); weight = (q - z) * s.
 *                      All divisions float32, rint ties to even.
 *
 * Packed layout (private to the library; read it back only through
 * wqd_dequant / wqd_unpack): weights are stored in tiles of 16 output rows x
 * 64 bytes of K (1 KiB: 32 bf16, 64 FP8 or 128 W4A16 codes per row), each row's
 * 64 bytes split into four 16-byte slices, slice j of row r at byte
 * (16 j + r) x 16.  Lane l of a 64-wide wavefront loads the 16 bytes at 16 l,
 * so one wavefront load is the whole tile, contiguous, and the lane order is
 * the B-operand order of the bf16 matrix-core multiply.  The tiles of a
 * 16-row block are consecutive along K.  wqd_packed_sizes gives the sizes.
 */
#ifndef WQD_H
#define WQD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum wqd_fmt {
    WQD_FMT_BF16 = 0,
    WQD_FMT_FP8_E4M3 = 1,
    WQD_FMT_W4A16_G128 = 2
};

enum wqd_status {
    WQD_OK = 0,
    WQD_E_ARG = 1,          /* null pointer, unknown fmt, negative size */
    WQD_E_SHAPE = 2,        /* shape not supported by fmt (e.g. K % 128 != 0 for W4A16) */
    WQD_E_ALIGN = 3,        /* a pointer is not 16-byte aligned */
    WQD_E_WORKSPACE = 4,    /* workspace missing or smaller than wqd_workspace_bytes */
    WQD_E_HIP = 5,          /* a HIP runtime call failed; see wqd_last_hip_error() */
    WQD_E_UNSUPPORTED = 6,  /* a valid request the library cannot serve */
    WQD_E_TIMEOUT = 7       /* a chain run abandoned a wait (wqd_chain_status) */
};

/* Library version as major*10000 + minor*100 + patch. */
int wqd_version(void);

/* Static description of a status code (never NULL). */
const char* wqd_status_str(int status);

/* hipError_t of the last failing HIP call made by this thread (0 if none). */
int wqd_last_hip_error(void);

/*
 * Host-only: byte sizes of the three packed buffers for an N x K weight in
 * `fmt` (N padded to whole 16-row blocks and K to whole 1 KiB tiles; W4A16
 * scales and zeros to whole sets of four groups).  scale_bytes and
 * zero_bytes are 0 where the format has none.  Any output pointer may be NULL.
 * Errors: WQD_E_ARG (fmt, N < 1, K < 1), WQD_E_SHAPE (K % 128 != 0 for W4A16,
 * K % 8 != 0 for the others).
 */
int wqd_packed_sizes(int fmt, int64_t N, int64_t K,
                     size_t* w_bytes, size_t* scale_bytes, size_t* zero_bytes);

/*
 * Host-only: bytes of scratch workspace wqd_qgemm needs for this shape (may
 * be 0).  The matrix-core paths use one when they split K over workgroups:
 * it holds their float32 partial tiles (S * M * N * 4 bytes), which a second
 * kernel adds in split order.  W4A16 on the tiled matrix-core kernel also
 * keeps the x sums of each 128-k group there (float32, K / 128 x M rounded
 * up to 64 rows, first), written by a first kernel of the same call.  Its
 * contents on entry do not matter (every byte read is written first in the
 * same call).  One workspace must not be used by two calls that can run at
 * the same time.
 */
int wqd_workspace_bytes(int fmt, int64_t M, int64_t N, int64_t K, size_t* bytes);

/* Kernel families behind wqd_qgemm (wqd_kernel_path).  Which one serves a
 * shape: the broadcast kernel for 1 W4A16 row or up to 4 FP8 / BF16 rows
 * (FP8 at 4 rows only where the skinny kernel's shares are not long); up
 * to 8 rows the skinny matrix-core kernel for long shares of K (large N, or
 * long K at 8 rows), else the streaming matrix-core kernel; otherwise, up to
 * 8 rows, the broadcast kernel, then the staged one; from 9 to 64 rows the skinny
 * matrix-core kernel (K a whole number of tiles: 128 W4A16, 64 FP8, 32 BF16),
 * except up to 16 rows on matrices up to 8192 x 8192 that it would split over
 * K, which take the streaming matrix-core kernel;
 * above 64 rows the tiled matrix-core kernel where N > 3840 (16 or more
 * 256-column blocks), else the LDS matrix-core kernel (also where the others
 * cannot take the shape: x rows spanning 2 GiB or more, or a ragged K below
 * 65 rows).  Each
 * streaming kernel also needs K short enough for its shares (hundreds of
 * 16-row tiles). */
enum wqd_path {
    WQD_PATH_BCAST = 0,   /* streaming, x read per tile and broadcast across DPP rows */
    WQD_PATH_STAGED = 1,  /* streaming, x staged in LDS, dot2 products */
    WQD_PATH_MFMA = 2,    /* bf16 matrix cores, x staged in LDS, dequant on load */
    WQD_PATH_MC = 3,      /* streaming, bf16 matrix cores, x fragments read per tile */
    WQD_PATH_SKINNY = 4,  /* bf16 matrix cores, x staged in LDS by a producer wavefront, shared by 7-14 row blocks */
    WQD_PATH_GEMM = 5,    /* bf16 matrix cores, 64 or 256 x 256 tiles of y, x staged in LDS, dequant on load */
    WQD_PATH_GEMM_LDS = 6 /* bf16 matrix cores, 256 x 256 tiles of y (FP8 also 256 x 224), x and the weights staged in LDS */
};

/*
 * Host-only: which kernel family wqd_qgemm launches for this shape (written
 * to *path), and the wavefronts per workgroup it uses (to *waves; may be
 * NULL).  Same validation as wqd_qgemm's shape checks.
 */
int wqd_kernel_path(int fmt, int64_t M, int64_t N, int64_t K, int* path, int* waves);

/*
 * Host-only: for a shape that wqd_qgemm serves with a tiled matrix-core kernel
 * (WQD_PATH_GEMM or WQD_PATH_GEMM_LDS), the tile of y each workgroup computes
 * (*rows x *cols: 64, 128 or 256 rows; 256 columns, or on the LDS-staged
 * kernel 224 or (FP8) 448 where those fill the compute units' rounds better),
 * the number of K splits (*splits; 1 when K is not split), and a tail split
 * (*tail_cols: the last columns of y, computed as *tail_splits K splits after
 * the others so that they fill the launch's last round; 0 and 0 when there is
 * none).  Any output pointer may be NULL.  Errors: those of wqd_kernel_path,
 * and WQD_E_UNSUPPORTED for a shape served by another kernel family.
 */
int wqd_gemm_tile(int fmt, int64_t M, int64_t N, int64_t K, int* rows, int* cols, int* splits, int* tail_cols,
                  int* tail_splits);

/*
 * Host-only: the tile of y each workgroup of wqd_qgemm_w8a8 computes for this
 * shape (*rows x *cols: 32, 64 or 128 x 256 with the weights taken into
 * registers; 256 x 256, 256 x 224 or 128 x 448 with both operands staged in
 * LDS, from 256 rows where K is a whole number of 128-k chunks) and its
 * number of K splits.  Any output pointer may be NULL.  Errors: those of
 * wqd_w8a8_workspace_bytes.
 */
int wqd_w8a8_tile(int64_t M, int64_t N, int64_t K, int* rows, int* cols, int* splits);

/*
 * Setup (not on the decode hot path): quantise W (device, float32 [N, K]
 * row-major) to `fmt` and write the packed weights, scales and zero points
 * (device buffers of the sizes wqd_packed_sizes gives; scales and zeros may be
 * NULL where the format has none).  Deterministic.  W must be finite: the
 * values are only read on the device, after the call has returned, so a NaN
 * or infinity is not reported, and the codes, scales and zeros of a row (FP8)
 * or group (W4A16) that holds one are unspecified (other rows and groups are
 * unaffected).
 */
int wqd_pack_weights(int fmt, const float* W, int64_t N, int64_t K,
                     void* w_packed, void* scales, void* zeros, void* stream);

/*
 * Hot path: y[M, N] = x[M, K] . dequant(W)^T.
 *   x  device bfloat16 [M, K] row-major;   y  device bfloat16 [M, N] row-major.
 * Products are formed from exactly dequantised weights and accumulated in
 * float32 (each W4A16 group and each FP8 row scale applied in float32); y is
 * the float32 sum rounded to nearest even bfloat16.  M >= 1; any M is
 * accepted, and the kernel family that serves a shape is the one
 * wqd_kernel_path names (see enum wqd_path).  workspace: device, >=
 * wqd_workspace_bytes bytes (may be NULL when that is 0).
 */
int wqd_qgemm(int fmt, const void* x, int64_t M, int64_t N, int64_t K,
              const void* w_packed, const void* scales, const void* zeros,
              void* y, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The fused MLP input projections with a SwiGLU epilogue: the MLP's gate and
 * up projections read the same activations and its next input is
 * silu(gate) * up (CS336 lecture 10 notes, section 3.2: the MLP's three
 * matrices; "Making each token cheaper", "Why decode is usually bandwidth
 * bound": each launch and each activation byte written and read again costs
 * time in a memory-bound step).  One launch streams both matrices and writes
 * h = silu(g) * up once, instead of g and up.
 *
 * wqd_pack_gate_up: W device float32 [2F][K] row-major, gate rows 0 .. F-1
 *   then up rows F .. 2F-1 (finite), packed in `fmt` as a 2F x K matrix whose
 *   rows are interleaved for the epilogue (16-row block b: gate rows
 *   8b .. 8b+7, then up rows 8b .. 8b+7); buffers of wqd_packed_sizes(fmt,
 *   2F, K).  Each row is quantised exactly as wqd_pack_weights quantises it.
 *   F % 8 == 0 (else WQD_E_SHAPE).
 * wqd_qgemm_swiglu: h[M][F] bfloat16 = bf16(silu(g) * u), g = x . gate^T and
 *   u = x . up^T formed exactly as wqd_qgemm forms y (float32 sums of exact
 *   products), silu(g) = g / (1 + exp(-g)) in float32.  workspace >=
 *   wqd_workspace_bytes(fmt, M, 2F, K).  Errors as wqd_qgemm.
 */
int wqd_pack_gate_up(int fmt, const float* W, int64_t F, int64_t K,
                     void* w_packed, void* scales, void* zeros, void* stream);
int wqd_qgemm_swiglu(int fmt, const void* x, int64_t M, int64_t F, int64_t K,
                     const void* w_packed, const void* scales, const void* zeros,
                     void* h, void* workspace, size_t workspace_bytes, void* stream);

/*
 * W8A8-FP8: activations quantised to FP8-E4M3 too, and the product on the
 * FP8 matrix cores, for the shapes where the matrix product, not the weight
 * bytes, sets the time (wide verify passes, large batches, prefill).  Sources:
 * "Making each token cheaper", "Weight quantization / Formats" (E4M3 for
 * weights and activations; a scale applied before the cast, per channel for
 * weights and per tensor for activations) and "What quantization saves"
 * (only a format whose product runs at lower precision, such as FP8 W8A8,
 * reduces that arithmetic); "LLM 推理是怎么变快的", section 4.2 B (W8A8 on the
 * FP8 / INT8 matrix units doubles the arithmetic rate).
 *
 * wqd_act_quant_fp8: x device bfloat16 [M, K] row-major (finite) ->
 *   x_scale  device float32 [1]: s_a = max |x| / 448 over the whole tensor
 *            (float32 division; 1 if x is all zero; at least 2^-126);
 *   x_codes  device uint8 [M, K] row-major: nearest E4M3FN of x / s_a
 *            (float32 division, ties to even, saturating at 448).
 *   workspace: device, >= WQD_ACT_QUANT_WORKSPACE_BYTES, contents on entry
 *   do not matter.  K % 16 == 0 (else WQD_E_SHAPE).  Deterministic.
 *
 * wqd_qgemm_w8a8: y[M, N] bfloat16 = bf16(s_a * s_n * sum_k e4m3(x_codes)
 *   e4m3(W codes)), with x_codes / x_scale as wqd_act_quant_fp8 writes them
 *   (x_scale read on the device) and W packed by wqd_pack_weights in the FP8
 *   format (w_packed, w_scales).  The products are exact and summed in
 *   float32.  workspace: >= wqd_w8a8_workspace_bytes (float32 split-K
 *   partials; may be NULL when that is 0).  K % 16 == 0, M * K < 2^31.
 *   Errors as wqd_qgemm.
 */
#define WQD_ACT_QUANT_WORKSPACE_BYTES 4096u
int wqd_act_quant_fp8(const void* x, int64_t M, int64_t K, void* x_codes, float* x_scale,
                      void* workspace, size_t workspace_bytes, void* stream);
int wqd_w8a8_workspace_bytes(int64_t M, int64_t N, int64_t K, size_t* bytes);
int wqd_qgemm_w8a8(const void* x_codes, const float* x_scale, int64_t M, int64_t N, int64_t K,
                   const void* w_packed, const void* w_scales, void* y,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode attention over a KV cache, split along the context (Flash-Decoding),
 * with grouped-query heads.  Sources: "Making each token cheaper", section
 * "Why kernels matter most for long prefill" (a decode step has one query per
 * sequence; decode attention is dominated by reading the KV cache;
 * Flash-Decoding splits keys and values into chunks processed in parallel,
 * since parallelising over batch and queries alone leaves most of the GPU
 * idle) and "Why decode is usually bandwidth bound" (each sequence's KV bytes
 * are read once per step); "LLM 推理是怎么变快的", section 2.3 (grouped-query
 * attention: several query heads share one KV head).
 *
 * For each sequence b and query head h, with g = h / (Hq / Hkv):
 *   o[b, h] = sum_{t < len[b]} softmax_t(scale * q[b, h] . K[b, g, t]) V[b, g, t]
 * products and sums in float32 from the bf16 inputs (the softmax weights
 * are not rounded to bf16), rounded to bf16; len[b] = 0 gives zeros.
 *   q          device bf16 [B][Hq][D]
 *   k_cache,   device bf16, B * Hkv * Lmax * D elements each, in the
 *   v_cache    library's tiled layout, written by wqd_kv_pack / wqd_kv_append
 *              (per (b, g), 1 KiB tiles in matrix-core operand order so that
 *              every load of the kernel is one contiguous 1 KiB; the element
 *              offsets of position t, dimension d within a (b, g) region of
 *              Lmax * D elements are:
 *                K: ((t / 16) * 4 + d / 32) * 512 + (((d % 32) / 8) * 16 + t % 16) * 8 + d % 8;
 *                V: ((t / 32) * 8 + d / 16) * 512 + (kb * 16 + d % 16) * 8 + e,
 *                   u = t % 32, kb = (u % 16) / 4, e = 4 * (u / 16) + u % 4)
 *   lengths    device int32 [B]: positions used per sequence (clamped to
 *              [0, Lmax]); cache entries at or past a length are never used,
 *              whatever they hold
 *   out        device bf16 [B][Hq][D]
 *   workspace  device, >= wqd_attn_workspace_bytes (partial maxima, sums and
 *              outputs when the context is split over several workgroups;
 *              0 bytes, and NULL allowed, when it is not), contents on entry
 *              do not matter.
 * D = 128, Hq a multiple of Hkv with Hq / Hkv <= 16, Lmax a multiple of 32
 * and Lmax * D * 2 < 2^31 (else WQD_E_SHAPE / WQD_E_UNSUPPORTED).
 * Deterministic.
 *
 * wqd_kv_pack: logical k, v device bf16 [B][Hkv][L][D] (L <= Lmax) into the
 *   caches' positions 0 .. L - 1 (later positions untouched).
 * wqd_kv_append: one new position per sequence, k_new / v_new device bf16
 *   [B][Hkv][D] at positions[b] (device int32 [B]; a position outside
 *   [0, Lmax) writes nothing) - the decode step's cache write.
 * wqd_kv_unpack: the caches back to logical device bf16 [B][Hkv][Lmax][D]
 *   (parity of the layout).
 */
int wqd_attn_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lmax, int64_t D, size_t* bytes);
/* Host only: how many chunks the context of each (sequence, KV head) is split
 * into for these sizes (1: one workgroup per pair writes the output). */
int wqd_attn_splits(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lmax, int64_t D, int* splits);
int wqd_decode_attention(const void* q, const void* k_cache, const void* v_cache, const int32_t* lengths,
                         int64_t B, int64_t Hq, int64_t Hkv, int64_t Lmax, int64_t D, float scale, void* out,
                         void* workspace, size_t workspace_bytes, void* stream);
int wqd_kv_pack(const void* k, const void* v, int64_t B, int64_t Hkv, int64_t L, int64_t Lmax, int64_t D,
                void* k_cache, void* v_cache, void* stream);
int wqd_kv_append(const void* k_new, const void* v_new, const int32_t* positions, int64_t B, int64_t Hkv,
                  int64_t Lmax, int64_t D, void* k_cache, void* v_cache, void* stream);
int wqd_kv_unpack(const void* k_cache, const void* v_cache, int64_t B, int64_t Hkv, int64_t Lmax, int64_t D,
                  void* k_out, void* v_out, void* stream);

/*
 * Decode attention over an FP8-E4M3 KV cache.  Sources: "LLM 推理是怎么变快的",
 * section 4, C (keys and values stored in FP8 halve the cache's bytes);
 * "Making each token cheaper", hands-on lab, exercise 5 (the step bound with
 * a one-byte KV cache).  The pages do not fix the scales; here one float32
 * scale per tensor for K and one for V, chosen by the caller:
 *   code = nearest E4M3FN value of x / scale (float32 division, ties to
 *          even, magnitudes past 448 saturate), value = e4m3(code) * scale,
 * then the attention of wqd_decode_attention on those values:
 *   o[b, h] = sum_{t < len[b]} softmax_t(scale * q[b, h] . K[b, g, t]) V[b, g, t]
 * (products and sums in float32, the dequantised keys and values exact).
 *   q, lengths, out, workspace   as wqd_decode_attention, with the sizes of
 *              wqd_attn_fp8kv_workspace_bytes / wqd_attn_fp8kv_splits
 *   k_cache,   device, B * Hkv * Lmax * D bytes each of E4M3 codes in the
 *   v_cache    library's tiled layout, written by wqd_kv_pack_fp8 /
 *              wqd_kv_append_fp8 (per (b, g), 1 KiB tiles; the byte offsets
 *              of position t, dimension d within a (b, g) region of
 *              Lmax * D bytes are:
 *                K: ((t / 16) * 2 + d / 64) * 1024 + (((d % 32) / 8) * 16 + t % 16) * 16
 *                   + 8 * ((d % 64) / 32) + d % 8;
 *                V: ((t / 32) * 4 + d / 32) * 1024 + (kb * 16 + d % 16) * 16
 *                   + 8 * ((d % 32) / 16) + e,
 *                   u = t % 32, kb = (u % 16) / 4, e = 4 * (u / 16) + u % 4)
 *              entries at or past a length are never used, whatever they hold
 *   k_scale,   the caches' scales: finite and > 0 (else WQD_E_ARG)
 *   v_scale
 * Shapes and errors as wqd_decode_attention.  Deterministic.
 *
 * wqd_kv_pack_fp8: logical k, v device bf16 [B][Hkv][L][D] (L <= Lmax),
 *   quantised with k_scale / v_scale, into positions 0 .. L - 1 (later
 *   positions untouched).  NaN inputs are not meaningful (the code saturates).
 * wqd_kv_append_fp8: one new position per sequence, quantised: k_new / v_new
 *   device bf16 [B][Hkv][D] at positions[b] (device int32 [B]; a position
 *   outside [0, Lmax) writes nothing).
 * wqd_kv_unpack_fp8: the caches' codes back to logical device uint8
 *   [B][Hkv][Lmax][D] (parity of the quantisation and the layout).
 */
int wqd_attn_fp8kv_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lmax, int64_t D, size_t* bytes);
int wqd_attn_fp8kv_splits(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lmax, int64_t D, int* splits);
int wqd_decode_attention_fp8kv(const void* q, const void* k_cache, const void* v_cache, float k_scale, float v_scale,
                               const int32_t* lengths, int64_t B, int64_t Hq, int64_t Hkv, int64_t Lmax, int64_t D,
                               float scale, void* out, void* workspace, size_t workspace_bytes, void* stream);
int wqd_kv_pack_fp8(const void* k, const void* v, float k_scale, float v_scale, int64_t B, int64_t Hkv, int64_t L,
                    int64_t Lmax, int64_t D, void* k_cache, void* v_cache, void* stream);
int wqd_kv_append_fp8(const void* k_new, const void* v_new, float k_scale, float v_scale, const int32_t* positions,
                      int64_t B, int64_t Hkv, int64_t Lmax, int64_t D, void* k_cache, void* v_cache, void* stream);
int wqd_kv_unpack_fp8(const void* k_cache, const void* v_cache, int64_t B, int64_t Hkv, int64_t Lmax, int64_t D,
                      void* k_codes, void* v_codes, void* stream);

/*
 * A chain of decode linear layers in one persistent launch.  Sources: CS336
 * lecture 10 notes, section 3.2 (a layer's matrices run in sequence, each on
 * the previous one's output: the attention projections, then the MLP's
 * gate/up and down); "Only Accepted Tokens Count" reading notes, on why the
 * paired experiments turn CUDA graphs on (a step made of many small kernels
 * pays a launch cost for each); "Making each token cheaper", "Why decode is
 * usually bandwidth bound" (a decode step reads every weight byte once, so
 * the step time is the weight bytes over the bandwidth).
 *
 * Call i computes y_i = x_i . dequant(W_i)^T, or with swiglu the SwiGLU of a
 * wqd_pack_gate_up pair, as wqd_qgemm / wqd_qgemm_swiglu would (the
 * broadcast streaming kernel's per-tile arithmetic, 4 wavefronts splitting K
 * for each pair of 16-row blocks), for 1 <= M <= 2 activation rows.  A call whose x is written by an
 * earlier call j names j in wait_for: its products start once every output
 * of call j is stored, while the weights of later calls stream meanwhile.
 *   wqd_chain_call, per call:
 *     w_packed, scales, zeros  device, from wqd_pack_weights / wqd_pack_gate_up
 *     x   device bf16 [M][K];  y  device bf16 [M][N] ([M][N / 2] with swiglu);
 *         both 16-byte aligned
 *     N, K      as for wqd_qgemm (swiglu: N % 16 == 0)
 *     wait_for  an earlier call whose y x reads (0 <= wait_for < i), or -1
 *               when x is ready before the run starts
 *     swiglu    0, or 1 for a gate/up pair
 *   Memory: a call may overwrite memory that another call reads only when
 *   that reader is among its ancestors through wait_for; the library orders
 *   nothing else.
 *
 * wqd_chain_workspace_bytes: host only; the device workspace a chain of
 *   ncalls needs (the call table, completion counters and a status flag).
 * wqd_chain_prepare (setup; synchronous copy to the device): validates every
 *   call as wqd_qgemm would, writes the table into `workspace` (16-byte
 *   aligned, >= wqd_chain_workspace_bytes; leave it untouched between runs)
 *   and fills *plan (caller-owned).  workgroups: 0 for the library's choice,
 *   else the grid size, at most the workgroups the device keeps resident at
 *   once (WQD_E_UNSUPPORTED beyond).  Errors: as wqd_qgemm for a call;
 *   WQD_E_ARG for M outside 1..2 (WQD_E_UNSUPPORTED above 2), ncalls < 1 or
 *   > 65536, a wait_for outside [-1, i); WQD_E_WORKSPACE; WQD_E_HIP.
 * wqd_chain_run: enqueues two launches on `stream` (counters cleared, then
 *   the chain); may be captured in a graph.  The grid is persistent: nothing
 *   else may run on the device at the same time.  Each wait is bounded by
 *   plan->wait_ticks ticks of the GPU's 100 MHz clock (0.1 s as prepared);
 *   past it the run is abandoned instead of hanging.
 * wqd_chain_status: synchronizes `stream`, then reports the last run:
 *   WQD_OK; WQD_E_TIMEOUT (a wait was abandoned: outputs are incomplete);
 *   WQD_E_ARG (the plan passed to the run did not match the prepared table).
 */
typedef struct {
    const void* w_packed;
    const void* scales;
    const void* zeros;
    const void* x;
    void* y;
    int64_t N, K;
    int32_t wait_for;
    int32_t swiglu;
} wqd_chain_call;

typedef struct {
    int32_t fmt, M, ncalls, total_items, workgroups, reserved;
    int64_t wait_ticks;
} wqd_chain_plan;

int wqd_chain_workspace_bytes(int64_t ncalls, size_t* bytes);
int wqd_chain_prepare(int fmt, int64_t M, int64_t ncalls, const wqd_chain_call* calls, int workgroups,
                      void* workspace, size_t workspace_bytes, wqd_chain_plan* plan);
int wqd_chain_run(const wqd_chain_plan* plan, void* workspace, void* stream);
int wqd_chain_status(const void* workspace, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * product as wqd_qgemm, with the same arguments except the workspace.  The
 * split-K partials and W4A16 group x sums go to a scratch array of
 * WQD_NOALLOC_SCRATCH_BYTES that the library holds in device memory, one copy
 * per GPU, from the first call on that GPU until the process ends.  Nothing
 * is allocated per call (no hipMalloc, no allocating library routine).
 *   - The scratch address is looked up on the first call on each device (the
 *     calling thread's current device, on which `stream` must be); the
 *     lookup makes no stream call.
 *   - Every call on one GPU shares that GPU's array: calls that can overlap
 *     on one GPU (other streams, other threads) race and give undefined
 *     results.  Consecutive calls on one stream are safe; the contents left
 *     by a call never affect the next.
 *   - Errors: as wqd_qgemm; WQD_E_WORKSPACE when the shape needs more than
 *     WQD_NOALLOC_SCRATCH_BYTES of workspace (wqd_workspace_bytes gives the
 *     need; every decode and verify width of the 70B and 7B shapes up to
 *     1024 rows fits, except BF16 above 512 rows); WQD_E_HIP if the lookup
 *     fails.
 */
#define WQD_NOALLOC_SCRATCH_BYTES (64u << 20)
int wqd_qgemm_noalloc(int fmt, const void* x, int64_t M, int64_t N, int64_t K,
                      const void* w_packed, const void* scales, const void* zeros,
                      void* y, void* stream);

/*
 * Parity: dequantised weights in logical order, W_out device float32 [N, K]
 * row-major.  bf16 and W4A16 values are exact; FP8 values are the float32
 * product e4m3(code) * s_n rounded once.
 */
int wqd_dequant(int fmt, const void* w_packed, const void* scales, const void* zeros,
                int64_t N, int64_t K, float* W_out, void* stream);

/*
 * Parity: the logical codes behind a packed weight.
 *   codes_out  device [N, K] row-major: uint16 bf16 bit patterns (BF16), uint8
 *              E4M3 codes (FP8) or uint8 q in [0, 15] (W4A16);
 *   scales_out device float32 [N] (FP8) or float16 bits [N, K/128] (W4A16);
 *   zeros_out  device uint8 [N, K/128] (W4A16).
 * Outputs a format does not have must be NULL or are ignored.
 */
int wqd_unpack(int fmt, const void* w_packed, const void* scales, const void* zeros,
               int64_t N, int64_t K, void* codes_out, void* scales_out, void* zeros_out,
               void* stream);

/*
 * Parity: decode n E4M3 codes (device uint8) to float32 (device) with the same
 * device conversion the FP8 weight path uses (the exhaustive 256-code check).
 */
int wqd_decode_e4m3(const uint8_t* codes, float* out, int64_t n, void* stream);

/*
 * Speculative-sampling accept / reject, the step after the verify pass (CS336
 * lecture 10 notes, section 6.1, the four steps; section 6.2, why the output
 * is an exact sample of the target).  For each of B sequences, with
 *   target       device float32 [B, k+1, V]: the target's distributions at the
 *                k + 1 verified positions (probabilities in [0, 1]);
 *   draft        device float32 [B, k, V]: the draft's distributions;
 *   draft_tokens device int32 [B, k]: the drafted tokens;
 *   u_accept     device float32 [B, k], u_draw device float32 [B]: the
 *                uniform numbers in [0, 1) the method draws, supplied by the
 *                caller;
 * draft token x_i is kept, left to right, while u_accept * draft_i(x_i) <
 * target_i(x_i) in float32 (u < min(1, target / draft); an out-of-range token
 * is rejected).  At the first rejection, position i, one token is drawn from
 * max(target_i - draft_i, 0) normalised; if every draft is kept, from
 * target_k.  A draw counts each weight in units of 2^-32 (floor(w * 2^32),
 * exact integers), takes U = floor(u_draw * T) with T the sum (the product
 * in double), and returns the smallest token whose prefix sum exceeds U.
 * U is kept below T: a u_draw of 1 or more (a generator whose range is
 * (0, 1]) draws the last token of positive weight, a NaN or negative u_draw
 * counts as 0.  A weight outside [0, 1] counts as the nearest end of that
 * range and a NaN weight as 0.
 * An empty residual draws from target_i; an all-zero row draws -1.
 * Outputs (device, caller-owned): n_kept int32 [B] (0 .. k) and out_tokens
 * int32 [B, k+1]: the kept drafts, the drawn token, then -1.  draft,
 * draft_tokens and u_accept may be NULL when k = 0.  workspace: device,
 * >= wqd_spec_workspace_bytes(B, V) (per sequence, two 64-bit unit sums per
 * 256 tokens), 8-byte aligned, contents on entry do not matter.
 * Deterministic; all arrays contiguous row-major, 4-byte aligned.
 * Errors: WQD_E_ARG (NULL pointer, B < 1, k < 0, V < 1), WQD_E_SHAPE (k > 64,
 * V > 2^20), WQD_E_ALIGN, WQD_E_WORKSPACE.
 */
int wqd_spec_workspace_bytes(int64_t B, int64_t V, size_t* bytes);
int wqd_spec_accept(const float* target, const float* draft, const int32_t* draft_tokens,
                    const float* u_accept, const float* u_draw, int64_t B, int64_t k, int64_t V,
                    int32_t* n_kept, int32_t* out_tokens, void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * Measurement: read `bytes` (multiple of 16) from device `src` with 16-byte
 * loads and write one 32-bit checksum per workgroup to `sink` (device,
 * >= wqd_stream_sink_words(bytes) words).  The HBM read ceiling.
 */
int wqd_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream);
size_t wqd_stream_sink_words(size_t bytes);

/* Measurement: device copy of `bytes` (multiple of 16) with 16-byte loads/stores. */
int wqd_stream_copy(void* dst, const void* src, size_t bytes, void* stream);

/*
 * Measurement: the matrix-core ceiling.  Every SIMD runs four wavefronts, each
 * issuing `iters` x 16 independent v_mfma_f32_16x16x32_bf16 on operands held
 * in registers, and one float per workgroup goes to `sink` (device, >=
 * wqd_mfma_peak_sink_words() floats).  wqd_mfma_peak_flops(iters) is the FLOP
 * count of one launch (host only); divided by the launch's time it gives the
 * throughput the wide verify batches are compared against.  iters >= 1, else
 * WQD_E_ARG.
 */
int wqd_mfma_peak(int64_t iters, float* sink, void* stream);
size_t wqd_mfma_peak_sink_words(void);
double wqd_mfma_peak_flops(int64_t iters);

#ifdef __cplusplus
}
#endif

#endif /* WQD_H */
