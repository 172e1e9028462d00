// Launchers shared between the kernel files and the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wqd_plan.h"

namespace wqd {

// F > 0: W holds F gate rows then F up rows (N = 2F), packed interleaved for
// the SwiGLU epilogue (src_row in wqd_device.h).
hipError_t launch_pack(int fmt, const float* W, int64_t N, int64_t K, const PackedSizes& ps, void* wp, void* scales,
                       void* zeros, int64_t F, hipStream_t st);
hipError_t launch_dequant(int fmt, const void* wp, const void* scales, const void* zeros, int64_t N, int64_t K,
                          const PackedSizes& ps, float* out, hipStream_t st);
hipError_t launch_unpack(int fmt, const void* wp, const void* scales, const void* zeros, int64_t N, int64_t K,
                         const PackedSizes& ps, void* codes, void* scales_out, void* zeros_out, hipStream_t st);
hipError_t launch_decode_e4m3(const uint8_t* codes, float* out, int64_t n, hipStream_t st);
// swiglu: the packed rows are gate/up pairs and y receives silu(gate) * up,
// [M][N / 2] (store_out in wqd_device.h).
hipError_t launch_gemv(int fmt, const GemvPlan& p, const void* x, int64_t M, int64_t N, int64_t K, const void* wp,
                       const void* scales, const void* zeros, void* y, bool swiglu, hipStream_t st);
hipError_t launch_gemv_bcast(int fmt, const BcastPlan& p, const void* x, int64_t M, int64_t N, int64_t K,
                             const void* wp, const void* scales, const void* zeros, void* y, bool swiglu,
                             hipStream_t st);
hipError_t launch_gemv_mc(int fmt, const McPlan& p, const void* x, int64_t M, int64_t N, int64_t K,
                          const void* wp, const void* scales, const void* zeros, void* y, bool swiglu, hipStream_t st);
hipError_t launch_gemv_sk(int fmt, const SkPlan& p, const void* x, int64_t M, int64_t N, int64_t K, const void* wp,
                          const void* scales, const void* zeros, void* y, void* ws, bool swiglu, hipStream_t st);
// The tiled kernel with the weights staged in LDS as well (GmPlan::wm == 3,
// BF16); launch_gemm calls it.
hipError_t launch_gemm_lds(int fmt, const GmPlan& p, const void* x, int64_t M, int64_t N, int64_t K, const void* wp,
                           const void* scales, void* y, void* part, bool swiglu, hipStream_t st);
hipError_t launch_gemm(int fmt, const GmPlan& p, const void* x, int64_t M, int64_t N, int64_t K, const void* wp,
                       const void* scales, const void* zeros, void* y, void* ws, bool swiglu, hipStream_t st);
// y = sum over s < S of part[s] (float32 [S][M][N], added in split order), FP8
// scaled per column, rounded to bfloat16.
hipError_t launch_splitk_reduce(int fmt, const float* part, int S, int64_t M, int64_t N, const void* scales, void* y,
                                bool swiglu, hipStream_t st);
hipError_t launch_mfma(int fmt, const MfmaPlan& p, int64_t M, int64_t N, int64_t K, const void* x, const void* wp,
                       const void* scales, const void* zeros, void* y, void* ws, bool swiglu, hipStream_t st);
// W8A8-FP8: activation codes and scale (workspace: the G partial maxima),
// then the product on the FP8 matrix cores.
hipError_t launch_act_quant(const void* x, int64_t M, int64_t K, int parts, void* codes, float* scale,
                            float* ws_part, hipStream_t st);
hipError_t launch_w8a8(const W8Plan& p, const void* xc, const float* xscale, int64_t M, int64_t N, int64_t K,
                       const void* wp, const void* scales, void* y, void* ws, hipStream_t st);
// Decode attention (split along the context, then the fixed-order merge).
hipError_t launch_attn(const AttnPlan& p, const void* q, const void* k, const void* v, const int32_t* lens,
                       int64_t B, float scale, float k_scale, float v_scale, void* out, void* ws, hipStream_t st);
// KV cache tiles: pack / unpack [BH][L][128] logical rows, append one position per sequence.
hipError_t launch_kv_copy(bool pack, const void* src_k, const void* src_v, void* dst_k, void* dst_v, int64_t BH,
                          int64_t L, int64_t Lmax, hipStream_t st);
hipError_t launch_kv_append(const void* k_new, const void* v_new, const int32_t* positions, int64_t B, int64_t Hkv,
                            int64_t Lmax, void* k, void* v, hipStream_t st);
// The FP8 cache: pack quantises logical bf16 rows into the tiles, unpack
// returns the tiles' codes as logical uint8 rows; append quantises one
// position per sequence.
hipError_t launch_kv8_copy(bool pack, const void* src_k, const void* src_v, void* dst_k, void* dst_v, float k_scale,
                           float v_scale, int64_t BH, int64_t L, int64_t Lmax, hipStream_t st);
hipError_t launch_kv8_append(const void* k_new, const void* v_new, float k_scale, float v_scale,
                             const int32_t* positions, int64_t B, int64_t Hkv, int64_t Lmax, void* k, void* v,
                             hipStream_t st);
// A chain of decode layers in one persistent launch (clear, then the chain);
// the workspace holds the table written by wqd_chain_prepare.
hipError_t launch_chain(int fmt, int M, int ncalls, int total_items, int grid, long long ticks, void* ws,
                        hipStream_t st);
hipError_t chain_resident_workgroups(int fmt, int M, int* out);
hipError_t chain_compute_units(int* out);
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t st);
hipError_t launch_stream_copy(void* dst, const void* src, size_t bytes, hipStream_t st);
size_t stream_sink_words(size_t bytes);
hipError_t launch_mfma_peak(int64_t iters, float* sink, hipStream_t st);
size_t mfma_peak_sink_words();
double mfma_peak_flops(int64_t iters);
// wqd_qgemm after its argument checks (shared by the entry points that call it).
int qgemm_checked(int fmt, const void* x, int64_t M, int64_t N, int64_t K, const void* w_packed, const void* scales,
                  const void* zeros, void* y, void* workspace, size_t workspace_bytes, void* stream,
                  bool swiglu = false);
// Maps a HIP error to a wqd status, keeping it for wqd_last_hip_error().
int record_hip_error(hipError_t e);
hipError_t launch_spec_accept(const float* target, const float* draft, const int32_t* tokens, const float* u_accept,
                              const float* u_draw, int64_t B, int64_t k, int64_t V, int32_t* n_kept, int32_t* out,
                              void* ws, hipStream_t st);
// Workspace of the accept / reject step: two 64-bit tile sums per 256 tokens and sequence.
size_t spec_workspace_bytes(int64_t B, int64_t V);

}  // namespace wqd
