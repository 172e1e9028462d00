// extern "C" entry points declared in include/wqd.h: validate on the host,
// plan, then enqueue on the caller's stream.  No allocation, no host sync.
#include <hip/hip_runtime.h>

#include <cmath>
#include <vector>

#include "../../include/wqd.h"
#include "wqd_internal.h"
#include "wqd_plan.h"

namespace {

thread_local int g_last_hip_error = 0;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return WQD_OK;
  g_last_hip_error = int(e);
  return WQD_E_HIP;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

bool need_scales(int fmt) { return fmt != wqd::kFmtBF16; }
bool need_zeros(int fmt) { return fmt == wqd::kFmtW4; }

int check_packed_ptrs(int fmt, const void* wp, const void* scales, const void* zeros) {
  if (!wp) return WQD_E_ARG;
  if (need_scales(fmt) && !scales) return WQD_E_ARG;
  if (need_zeros(fmt) && !zeros) return WQD_E_ARG;
  if (!wqd::aligned16(wp)) return WQD_E_ALIGN;
  if (need_scales(fmt) && !wqd::aligned16(scales)) return WQD_E_ALIGN;
  if (need_zeros(fmt) && !wqd::aligned16(zeros)) return WQD_E_ALIGN;
  return WQD_OK;
}

}  // namespace

namespace wqd {

int qgemm_checked(int fmt, const void* x, int64_t M, int64_t N, int64_t K, const void* w_packed, const void* scales,
                  const void* zeros, void* y, void* workspace, size_t workspace_bytes, void* stream, bool swiglu) {
  if (M < 1) return WQD_E_ARG;
  Choice c;
  int st = choose_path(fmt, M, N, K, &c);
  if (st != kOK) return st;
  if (!x || !y) return WQD_E_ARG;
  if (!aligned16(x) || !aligned16(y)) return WQD_E_ALIGN;
  st = check_packed_ptrs(fmt, w_packed, scales, zeros);
  if (st != WQD_OK) return st;
  size_t need = 0;
  st = wqd::workspace_bytes(fmt, M, N, K, &need);
  if (st != kOK) return st;
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return WQD_E_WORKSPACE;
    if (!aligned16(workspace)) return WQD_E_ALIGN;
  }
  if (swiglu && N % 16 != 0) return WQD_E_SHAPE;
  hipStream_t s = as_stream(stream);
  switch (c.path) {
    case kPathBcast:
      return hip_status(launch_gemv_bcast(fmt, c.bcast, x, M, N, K, w_packed, scales, zeros, y, swiglu, s));
    case kPathMc:
      return hip_status(launch_gemv_mc(fmt, c.mc, x, M, N, K, w_packed, scales, zeros, y, swiglu, s));
    case kPathStaged:
      return hip_status(launch_gemv(fmt, c.gemv, x, M, N, K, w_packed, scales, zeros, y, swiglu, s));
    case kPathGemm:
    case kPathGemmLds:
      return hip_status(launch_gemm(fmt, c.gm, x, M, N, K, w_packed, scales, zeros, y, workspace, swiglu, s));
    case kPathSkinny:
      return hip_status(launch_gemv_sk(fmt, c.sk, x, M, N, K, w_packed, scales, zeros, y, workspace, swiglu, s));
    default:
      return hip_status(launch_mfma(fmt, c.mfma, M, N, K, x, w_packed, scales, zeros, y, workspace, swiglu, s));
  }
}

int record_hip_error(hipError_t e) { return hip_status(e); }

}  // namespace wqd

extern "C" {

int wqd_version(void) { return 100; }

const char* wqd_status_str(int status) {
  switch (status) {
    case WQD_OK: return "ok";
    case WQD_E_ARG: return "invalid argument (null pointer, unknown format or bad size)";
    case WQD_E_SHAPE: return "shape not supported by this format";
    case WQD_E_ALIGN: return "pointer not 16-byte aligned";
    case WQD_E_WORKSPACE: return "workspace missing or too small";
    case WQD_E_HIP: return "HIP runtime error";
    case WQD_E_UNSUPPORTED: return "unsupported request";
    case WQD_E_TIMEOUT: return "chain run abandoned a wait";
    default: return "unknown status";
  }
}

int wqd_last_hip_error(void) { return g_last_hip_error; }

int wqd_packed_sizes(int fmt, int64_t N, int64_t K, size_t* w_bytes, size_t* scale_bytes, size_t* zero_bytes) {
  wqd::PackedSizes ps;
  const int st = wqd::packed_sizes(fmt, N, K, &ps);
  if (st != wqd::kOK) return st;
  if (w_bytes) *w_bytes = ps.w_bytes;
  if (scale_bytes) *scale_bytes = ps.s_bytes;
  if (zero_bytes) *zero_bytes = ps.z_bytes;
  return WQD_OK;
}

int wqd_workspace_bytes(int fmt, int64_t M, int64_t N, int64_t K, size_t* bytes) {
  if (!bytes) return WQD_E_ARG;
  return wqd::workspace_bytes(fmt, M, N, K, bytes);
}

int wqd_kernel_path(int fmt, int64_t M, int64_t N, int64_t K, int* path, int* waves) {
  if (!path) return WQD_E_ARG;
  wqd::Choice c;
  int st = wqd::choose_path(fmt, M, N, K, &c);
  if (st != wqd::kOK) return st;
  *path = c.path;  // enum wqd_path and wqd::Path share their values
  if (waves) {
    *waves = c.path == wqd::kPathBcast ? c.bcast.waves
           : c.path == wqd::kPathMc    ? c.mc.waves
           : c.path == wqd::kPathStaged ? c.gemv.waves
           : c.path == wqd::kPathSkinny ? c.sk.waves + 1
           : c.path == wqd::kPathGemm   ? (fmt == wqd::kFmtW4 ? 8 : 4 * c.gm.wm)
           : c.path == wqd::kPathGemmLds ? 8
                                        : 4;
  }
  return WQD_OK;
}

int wqd_gemm_tile(int fmt, int64_t M, int64_t N, int64_t K, int* rows, int* cols, int* splits, int* tail_cols,
                  int* tail_splits) {
  wqd::Choice c;
  int st = wqd::choose_path(fmt, M, N, K, &c);
  if (st != wqd::kOK) return st;
  if (c.path != wqd::kPathGemm && c.path != wqd::kPathGemmLds) return WQD_E_UNSUPPORTED;
  const wqd::GmPlan& p = c.gm;
  if (rows) *rows = p.wm == 3 ? 64 * p.lwr : p.wm == 2 ? (fmt == wqd::kFmtW4 ? 128 : 256) : 64;
  if (cols) *cols = p.wm == 3 ? 16 * (8 / p.lwr) * p.rbw : 256;
  if (splits) *splits = p.S;
  if (tail_cols) *tail_cols = p.S2 > 0 ? int(N - p.nbn1 * 256) : 0;
  if (tail_splits) *tail_splits = p.S2;
  return WQD_OK;
}

int wqd_w8a8_tile(int64_t M, int64_t N, int64_t K, int* rows, int* cols, int* splits) {
  wqd::W8Plan p;
  const int st = wqd::plan_w8a8(M, N, K, &p);
  if (st != wqd::kOK) return st;
  if (rows) *rows = p.lds ? 64 * p.lwr : 16 * p.mf * p.wr;
  if (cols) *cols = p.lds ? 16 * (8 / p.lwr) * p.rbw : 256;
  if (splits) *splits = p.S;
  return WQD_OK;
}

int wqd_pack_weights(int fmt, const float* W, int64_t N, int64_t K, void* w_packed, void* scales, void* zeros,
                     void* stream) {
  wqd::PackedSizes ps;
  int st = wqd::packed_sizes(fmt, N, K, &ps);
  if (st != wqd::kOK) return st;
  if (!W) return WQD_E_ARG;
  if (!wqd::aligned16(W)) return WQD_E_ALIGN;
  st = check_packed_ptrs(fmt, w_packed, scales, zeros);
  if (st != WQD_OK) return st;
  return hip_status(wqd::launch_pack(fmt, W, N, K, ps, w_packed, scales, zeros, 0, as_stream(stream)));
}

int wqd_pack_gate_up(int fmt, const float* W, int64_t F, int64_t K, void* w_packed, void* scales, void* zeros,
                     void* stream) {
  if (F < 1) return WQD_E_ARG;
  if (F % 8 != 0) return WQD_E_SHAPE;
  wqd::PackedSizes ps;
  int st = wqd::packed_sizes(fmt, 2 * F, K, &ps);
  if (st != wqd::kOK) return st;
  if (!W) return WQD_E_ARG;
  if (!wqd::aligned16(W)) return WQD_E_ALIGN;
  st = check_packed_ptrs(fmt, w_packed, scales, zeros);
  if (st != WQD_OK) return st;
  return hip_status(wqd::launch_pack(fmt, W, 2 * F, K, ps, w_packed, scales, zeros, F, as_stream(stream)));
}

int wqd_qgemm_swiglu(int fmt, const void* x, int64_t M, int64_t F, int64_t K, const void* w_packed,
                     const void* scales, const void* zeros, void* h, void* workspace, size_t workspace_bytes,
                     void* stream) {
  if (F < 1) return WQD_E_ARG;
  if (F % 8 != 0) return WQD_E_SHAPE;
  return wqd::qgemm_checked(fmt, x, M, 2 * F, K, w_packed, scales, zeros, h, workspace, workspace_bytes, stream,
                            true);
}

int wqd_qgemm(int fmt, const void* x, int64_t M, int64_t N, int64_t K, const void* w_packed, const void* scales,
              const void* zeros, void* y, void* workspace, size_t workspace_bytes, void* stream) {
  return wqd::qgemm_checked(fmt, x, M, N, K, w_packed, scales, zeros, y, workspace, workspace_bytes, stream);
}

static_assert(WQD_ACT_QUANT_WORKSPACE_BYTES >= wqd::kActQuantParts * sizeof(float),
              "the activation quantisation workspace holds every partial maximum");

int wqd_act_quant_fp8(const void* x, int64_t M, int64_t K, void* x_codes, float* x_scale, void* workspace,
                      size_t workspace_bytes, void* stream) {
  int parts = 0;
  const int st = wqd::plan_act_quant(M, K, &parts);
  if (st != wqd::kOK) return st;
  if (!x || !x_codes || !x_scale || !workspace) return WQD_E_ARG;
  if (workspace_bytes < WQD_ACT_QUANT_WORKSPACE_BYTES) return WQD_E_WORKSPACE;
  if (!wqd::aligned16(x) || !wqd::aligned16(x_codes) || !wqd::aligned16(workspace) ||
      reinterpret_cast<uintptr_t>(x_scale) % 4)
    return WQD_E_ALIGN;
  return hip_status(wqd::launch_act_quant(x, M, K, parts, x_codes, x_scale, reinterpret_cast<float*>(workspace),
                                          as_stream(stream)));
}

int wqd_w8a8_workspace_bytes(int64_t M, int64_t N, int64_t K, size_t* bytes) {
  if (!bytes) return WQD_E_ARG;
  wqd::W8Plan p;
  const int st = wqd::plan_w8a8(M, N, K, &p);
  if (st != wqd::kOK) return st;
  *bytes = p.ws_bytes;
  return WQD_OK;
}

int wqd_qgemm_w8a8(const void* x_codes, const float* x_scale, int64_t M, int64_t N, int64_t K, const void* w_packed,
                   const void* w_scales, void* y, void* workspace, size_t workspace_bytes, void* stream) {
  wqd::W8Plan p;
  int st = wqd::plan_w8a8(M, N, K, &p);
  if (st != wqd::kOK) return st;
  if (!x_codes || !x_scale || !y) return WQD_E_ARG;
  if (!wqd::aligned16(x_codes) || !wqd::aligned16(y) || reinterpret_cast<uintptr_t>(x_scale) % 4) return WQD_E_ALIGN;
  st = check_packed_ptrs(wqd::kFmtFP8, w_packed, w_scales, nullptr);
  if (st != WQD_OK) return st;
  if (p.ws_bytes > 0) {
    if (!workspace || workspace_bytes < p.ws_bytes) return WQD_E_WORKSPACE;
    if (!wqd::aligned16(workspace)) return WQD_E_ALIGN;
  }
  return hip_status(wqd::launch_w8a8(p, x_codes, x_scale, M, N, K, w_packed, w_scales, y, workspace,
                                     as_stream(stream)));
}

int wqd_attn_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lmax, int64_t D, size_t* bytes) {
  if (!bytes) return WQD_E_ARG;
  wqd::AttnPlan p;
  const int st = wqd::plan_attn(B, Hq, Hkv, Lmax, D, &p);
  if (st != wqd::kOK) return st;
  *bytes = p.ws_bytes;
  return WQD_OK;
}

int wqd_chain_workspace_bytes(int64_t ncalls, size_t* bytes) {
  if (!bytes || ncalls < 1 || ncalls > wqd::kChainMaxCalls) return WQD_E_ARG;
  *bytes = wqd::chain_workspace_bytes(ncalls);
  return WQD_OK;
}

int wqd_chain_prepare(int fmt, int64_t M, int64_t ncalls, const wqd_chain_call* calls, int workgroups,
                      void* workspace, size_t workspace_bytes, wqd_chain_plan* plan) {
  if (!calls || !plan || ncalls < 1 || ncalls > wqd::kChainMaxCalls || M < 1 || workgroups < 0) return WQD_E_ARG;
  if (fmt != wqd::kFmtBF16 && fmt != wqd::kFmtFP8 && fmt != wqd::kFmtW4) return WQD_E_ARG;
  if (M > wqd::kChainMaxM) return WQD_E_UNSUPPORTED;
  const size_t need = wqd::chain_workspace_bytes(ncalls);
  if (!workspace || workspace_bytes < need) return WQD_E_WORKSPACE;
  if (!wqd::aligned16(workspace)) return WQD_E_ALIGN;
  const size_t table_bytes = wqd::chain_table_offset() + size_t(ncalls) * sizeof(wqd::ChainCall);
  std::vector<char> host(table_bytes, 0);
  auto* tab = reinterpret_cast<wqd::ChainCall*>(host.data() + wqd::chain_table_offset());
  int64_t items = 0;
  for (int64_t i = 0; i < ncalls; ++i) {
    const wqd_chain_call& c = calls[i];
    int st = wqd::plan_chain_call(fmt, M, c.N, c.K, c.swiglu != 0, &tab[i]);
    if (st != wqd::kOK) return st;
    if (!c.x || !c.y) return WQD_E_ARG;
    if (!wqd::aligned16(c.x) || !wqd::aligned16(c.y)) return WQD_E_ALIGN;
    st = check_packed_ptrs(fmt, c.w_packed, c.scales, c.zeros);
    if (st != WQD_OK) return st;
    if (c.swiglu != 0 && c.swiglu != 1) return WQD_E_ARG;
    if (c.wait_for < -1 || c.wait_for >= i) return WQD_E_ARG;
    tab[i].w = c.w_packed;
    tab[i].scales = c.scales;
    tab[i].zeros = c.zeros;
    tab[i].x = c.x;
    tab[i].y = c.y;
    tab[i].wait_for = c.wait_for;
    tab[i].item0 = int32_t(items);
    items += tab[i].ni;
    if (items >= (int64_t(1) << 31)) return WQD_E_UNSUPPORTED;
  }
  int resident = 0, cus = 0;
  int st = hip_status(wqd::chain_resident_workgroups(fmt, int(M), &resident));
  if (st != WQD_OK) return st;
  st = hip_status(wqd::chain_compute_units(&cus));
  if (st != WQD_OK) return st;
  const int grid = workgroups > 0 ? workgroups : (cus < resident ? cus : resident);
  if (grid < 1 || grid > resident) return WQD_E_UNSUPPORTED;
  auto* hdr = reinterpret_cast<wqd::ChainHeader*>(host.data());
  hdr->magic = wqd::kChainMagic;
  hdr->fmt = fmt;
  hdr->M = int32_t(M);
  hdr->ncalls = int32_t(ncalls);
  hdr->total_items = int32_t(items);
  hdr->grid = grid;
  st = hip_status(hipMemcpy(workspace, host.data(), table_bytes, hipMemcpyHostToDevice));
  if (st != WQD_OK) return st;
  plan->fmt = fmt;
  plan->M = int32_t(M);
  plan->ncalls = int32_t(ncalls);
  plan->total_items = int32_t(items);
  plan->workgroups = grid;
  plan->reserved = 0;
  plan->wait_ticks = 10000000;  // 0.1 s of the 100 MHz clock
  return WQD_OK;
}

int wqd_chain_run(const wqd_chain_plan* plan, void* workspace, void* stream) {
  if (!plan || !workspace) return WQD_E_ARG;
  if (plan->M < 1 || plan->M > wqd::kChainMaxM || plan->ncalls < 1 || plan->ncalls > wqd::kChainMaxCalls ||
      plan->workgroups < 1 || plan->total_items < 1 || plan->wait_ticks < 0)
    return WQD_E_ARG;
  if (plan->fmt != wqd::kFmtBF16 && plan->fmt != wqd::kFmtFP8 && plan->fmt != wqd::kFmtW4) return WQD_E_ARG;
  if (!wqd::aligned16(workspace)) return WQD_E_ALIGN;
  return hip_status(wqd::launch_chain(plan->fmt, plan->M, plan->ncalls, plan->total_items, plan->workgroups,
                                      plan->wait_ticks, workspace, as_stream(stream)));
}

int wqd_chain_status(const void* workspace, void* stream) {
  if (!workspace) return WQD_E_ARG;
  int st = hip_status(hipStreamSynchronize(as_stream(stream)));
  if (st != WQD_OK) return st;
  int flag = 0;
  st = hip_status(hipMemcpy(&flag, static_cast<const char*>(workspace) + 128, sizeof(int), hipMemcpyDeviceToHost));
  if (st != WQD_OK) return st;
  return flag == 0 ? WQD_OK : flag == 1 ? WQD_E_TIMEOUT : WQD_E_ARG;
}

int wqd_attn_splits(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lmax, int64_t D, int* splits) {
  if (!splits) return WQD_E_ARG;
  wqd::AttnPlan p;
  const int st = wqd::plan_attn(B, Hq, Hkv, Lmax, D, &p);
  if (st != wqd::kOK) return st;
  *splits = p.S;
  return WQD_OK;
}

int wqd_decode_attention(const void* q, const void* k_cache, const void* v_cache, const int32_t* lengths,
                         int64_t B, int64_t Hq, int64_t Hkv, int64_t Lmax, int64_t D, float scale, void* out,
                         void* workspace, size_t workspace_bytes, void* stream) {
  wqd::AttnPlan p;
  const int st = wqd::plan_attn(B, Hq, Hkv, Lmax, D, &p);
  if (st != wqd::kOK) return st;
  if (!q || !k_cache || !v_cache || !lengths || !out) return WQD_E_ARG;
  if (p.ws_bytes > 0 && (!workspace || workspace_bytes < p.ws_bytes)) return WQD_E_WORKSPACE;
  if (!wqd::aligned16(q) || !wqd::aligned16(k_cache) || !wqd::aligned16(v_cache) || !wqd::aligned16(out) ||
      (p.ws_bytes > 0 && !wqd::aligned16(workspace)) || reinterpret_cast<uintptr_t>(lengths) % 4)
    return WQD_E_ALIGN;
  return hip_status(wqd::launch_attn(p, q, k_cache, v_cache, lengths, B, scale, 1.0f, 1.0f, out, workspace,
                                     as_stream(stream)));
}

namespace {
bool kv_scale_ok(float s) { return std::isfinite(s) && s > 0.0f; }
}  // namespace

int wqd_attn_fp8kv_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lmax, int64_t D, size_t* bytes) {
  if (!bytes) return WQD_E_ARG;
  wqd::AttnPlan p;
  const int st = wqd::plan_attn(B, Hq, Hkv, Lmax, D, &p, true);
  if (st != wqd::kOK) return st;
  *bytes = p.ws_bytes;
  return WQD_OK;
}

int wqd_attn_fp8kv_splits(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lmax, int64_t D, int* splits) {
  if (!splits) return WQD_E_ARG;
  wqd::AttnPlan p;
  const int st = wqd::plan_attn(B, Hq, Hkv, Lmax, D, &p, true);
  if (st != wqd::kOK) return st;
  *splits = p.S;
  return WQD_OK;
}

int wqd_decode_attention_fp8kv(const void* q, const void* k_cache, const void* v_cache, float k_scale, float v_scale,
                               const int32_t* lengths, int64_t B, int64_t Hq, int64_t Hkv, int64_t Lmax, int64_t D,
                               float scale, void* out, void* workspace, size_t workspace_bytes, void* stream) {
  wqd::AttnPlan p;
  const int st = wqd::plan_attn(B, Hq, Hkv, Lmax, D, &p, true);
  if (st != wqd::kOK) return st;
  if (!q || !k_cache || !v_cache || !lengths || !out || !kv_scale_ok(k_scale) || !kv_scale_ok(v_scale))
    return WQD_E_ARG;
  if (p.ws_bytes > 0 && (!workspace || workspace_bytes < p.ws_bytes)) return WQD_E_WORKSPACE;
  if (!wqd::aligned16(q) || !wqd::aligned16(k_cache) || !wqd::aligned16(v_cache) || !wqd::aligned16(out) ||
      (p.ws_bytes > 0 && !wqd::aligned16(workspace)) || reinterpret_cast<uintptr_t>(lengths) % 4)
    return WQD_E_ALIGN;
  return hip_status(wqd::launch_attn(p, q, k_cache, v_cache, lengths, B, scale, k_scale, v_scale, out, workspace,
                                     as_stream(stream)));
}

namespace {
int check_kv(int64_t B, int64_t Hkv, int64_t Lmax, int64_t D) {
  wqd::AttnPlan p;
  return wqd::plan_attn(B, Hkv, Hkv, Lmax, D, &p);
}
}  // namespace

int wqd_kv_pack(const void* k, const void* v, int64_t B, int64_t Hkv, int64_t L, int64_t Lmax, int64_t D,
                void* k_cache, void* v_cache, void* stream) {
  const int st = check_kv(B, Hkv, Lmax, D);
  if (st != WQD_OK) return st;
  if (L < 0 || L > Lmax) return WQD_E_ARG;
  if (!k || !v || !k_cache || !v_cache) return WQD_E_ARG;
  if (!wqd::aligned16(k) || !wqd::aligned16(v) || !wqd::aligned16(k_cache) || !wqd::aligned16(v_cache))
    return WQD_E_ALIGN;
  return hip_status(wqd::launch_kv_copy(true, k, v, k_cache, v_cache, B * Hkv, L, Lmax, as_stream(stream)));
}

int wqd_kv_unpack(const void* k_cache, const void* v_cache, int64_t B, int64_t Hkv, int64_t Lmax, int64_t D,
                  void* k_out, void* v_out, void* stream) {
  const int st = check_kv(B, Hkv, Lmax, D);
  if (st != WQD_OK) return st;
  if (!k_out || !v_out || !k_cache || !v_cache) return WQD_E_ARG;
  if (!wqd::aligned16(k_out) || !wqd::aligned16(v_out) || !wqd::aligned16(k_cache) || !wqd::aligned16(v_cache))
    return WQD_E_ALIGN;
  return hip_status(wqd::launch_kv_copy(false, k_cache, v_cache, k_out, v_out, B * Hkv, Lmax, Lmax,
                                        as_stream(stream)));
}

int wqd_kv_append(const void* k_new, const void* v_new, const int32_t* positions, int64_t B, int64_t Hkv,
                  int64_t Lmax, int64_t D, void* k_cache, void* v_cache, void* stream) {
  const int st = check_kv(B, Hkv, Lmax, D);
  if (st != WQD_OK) return st;
  if (!k_new || !v_new || !positions || !k_cache || !v_cache) return WQD_E_ARG;
  if (!wqd::aligned16(k_new) || !wqd::aligned16(v_new) || !wqd::aligned16(k_cache) || !wqd::aligned16(v_cache) ||
      reinterpret_cast<uintptr_t>(positions) % 4)
    return WQD_E_ALIGN;
  return hip_status(wqd::launch_kv_append(k_new, v_new, positions, B, Hkv, Lmax, k_cache, v_cache,
                                          as_stream(stream)));
}

int wqd_kv_pack_fp8(const void* k, const void* v, float k_scale, float v_scale, int64_t B, int64_t Hkv, int64_t L,
                    int64_t Lmax, int64_t D, void* k_cache, void* v_cache, void* stream) {
  const int st = check_kv(B, Hkv, Lmax, D);
  if (st != WQD_OK) return st;
  if (L < 0 || L > Lmax) return WQD_E_ARG;
  if (!k || !v || !k_cache || !v_cache || !kv_scale_ok(k_scale) || !kv_scale_ok(v_scale)) return WQD_E_ARG;
  if (!wqd::aligned16(k) || !wqd::aligned16(v) || !wqd::aligned16(k_cache) || !wqd::aligned16(v_cache))
    return WQD_E_ALIGN;
  return hip_status(wqd::launch_kv8_copy(true, k, v, k_cache, v_cache, k_scale, v_scale, B * Hkv, L, Lmax,
                                         as_stream(stream)));
}

int wqd_kv_unpack_fp8(const void* k_cache, const void* v_cache, int64_t B, int64_t Hkv, int64_t Lmax, int64_t D,
                      void* k_codes, void* v_codes, void* stream) {
  const int st = check_kv(B, Hkv, Lmax, D);
  if (st != WQD_OK) return st;
  if (!k_codes || !v_codes || !k_cache || !v_cache) return WQD_E_ARG;
  if (!wqd::aligned16(k_codes) || !wqd::aligned16(v_codes) || !wqd::aligned16(k_cache) || !wqd::aligned16(v_cache))
    return WQD_E_ALIGN;
  return hip_status(wqd::launch_kv8_copy(false, k_cache, v_cache, k_codes, v_codes, 1.0f, 1.0f, B * Hkv, Lmax, Lmax,
                                         as_stream(stream)));
}

int wqd_kv_append_fp8(const void* k_new, const void* v_new, float k_scale, float v_scale, const int32_t* positions,
                      int64_t B, int64_t Hkv, int64_t Lmax, int64_t D, void* k_cache, void* v_cache, void* stream) {
  const int st = check_kv(B, Hkv, Lmax, D);
  if (st != WQD_OK) return st;
  if (!k_new || !v_new || !positions || !k_cache || !v_cache || !kv_scale_ok(k_scale) || !kv_scale_ok(v_scale))
    return WQD_E_ARG;
  if (!wqd::aligned16(k_new) || !wqd::aligned16(v_new) || !wqd::aligned16(k_cache) || !wqd::aligned16(v_cache) ||
      reinterpret_cast<uintptr_t>(positions) % 4)
    return WQD_E_ALIGN;
  return hip_status(wqd::launch_kv8_append(k_new, v_new, k_scale, v_scale, positions, B, Hkv, Lmax, k_cache, v_cache,
                                           as_stream(stream)));
}

int wqd_dequant(int fmt, const void* w_packed, const void* scales, const void* zeros, int64_t N, int64_t K,
                float* W_out, void* stream) {
  wqd::PackedSizes ps;
  int st = wqd::packed_sizes(fmt, N, K, &ps);
  if (st != wqd::kOK) return st;
  if (!W_out) return WQD_E_ARG;
  st = check_packed_ptrs(fmt, w_packed, scales, zeros);
  if (st != WQD_OK) return st;
  return hip_status(wqd::launch_dequant(fmt, w_packed, scales, zeros, N, K, ps, W_out, as_stream(stream)));
}

int wqd_unpack(int fmt, const void* w_packed, const void* scales, const void* zeros, int64_t N, int64_t K,
               void* codes_out, void* scales_out, void* zeros_out, void* stream) {
  wqd::PackedSizes ps;
  int st = wqd::packed_sizes(fmt, N, K, &ps);
  if (st != wqd::kOK) return st;
  if (!codes_out) return WQD_E_ARG;
  st = check_packed_ptrs(fmt, w_packed, scales, zeros);
  if (st != WQD_OK) return st;
  if (fmt == wqd::kFmtBF16) scales_out = zeros_out = nullptr;
  if (fmt == wqd::kFmtFP8) zeros_out = nullptr;
  return hip_status(wqd::launch_unpack(fmt, w_packed, scales, zeros, N, K, ps, codes_out, scales_out, zeros_out,
                                       as_stream(stream)));
}

int wqd_decode_e4m3(const uint8_t* codes, float* out, int64_t n, void* stream) {
  if (n < 0 || (n > 0 && (!codes || !out))) return WQD_E_ARG;
  if (n == 0) return WQD_OK;
  return hip_status(wqd::launch_decode_e4m3(codes, out, n, as_stream(stream)));
}

int wqd_spec_workspace_bytes(int64_t B, int64_t V, size_t* bytes) {
  if (!bytes || B < 1 || V < 1) return WQD_E_ARG;
  if (V > (int64_t(1) << 20) || B > 0x7fffffff) return WQD_E_SHAPE;
  *bytes = wqd::spec_workspace_bytes(B, V);
  return WQD_OK;
}

int wqd_spec_accept(const float* target, const float* draft, const int32_t* draft_tokens, const float* u_accept,
                    const float* u_draw, int64_t B, int64_t k, int64_t V, int32_t* n_kept, int32_t* out_tokens,
                    void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 1 || k < 0 || V < 1 || !target || !u_draw || !n_kept || !out_tokens) return WQD_E_ARG;
  if (k > 0 && (!draft || !draft_tokens || !u_accept)) return WQD_E_ARG;
  if (k > 64 || V > (int64_t(1) << 20) || B > 0x7fffffff) return WQD_E_SHAPE;
  const void* ptrs[] = {target, draft, draft_tokens, u_accept, u_draw, n_kept, out_tokens};
  for (const void* q : ptrs)
    if (reinterpret_cast<uintptr_t>(q) % 4) return WQD_E_ALIGN;
  if (!workspace || workspace_bytes < wqd::spec_workspace_bytes(B, V)) return WQD_E_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) % 8) return WQD_E_ALIGN;
  return hip_status(wqd::launch_spec_accept(target, k > 0 ? draft : nullptr, draft_tokens, u_accept, u_draw, B, k,
                                            V, n_kept, out_tokens, workspace, as_stream(stream)));
}

size_t wqd_stream_sink_words(size_t bytes) { return wqd::stream_sink_words(bytes); }

int wqd_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink || bytes == 0 || bytes % 16) return WQD_E_ARG;
  if (!wqd::aligned16(src)) return WQD_E_ALIGN;
  return hip_status(wqd::launch_stream_read(src, bytes, sink, as_stream(stream)));
}

int wqd_stream_copy(void* dst, const void* src, size_t bytes, void* stream) {
  if (!src || !dst || bytes == 0 || bytes % 16) return WQD_E_ARG;
  if (!wqd::aligned16(src) || !wqd::aligned16(dst)) return WQD_E_ALIGN;
  return hip_status(wqd::launch_stream_copy(dst, src, bytes, as_stream(stream)));
}

size_t wqd_mfma_peak_sink_words(void) { return wqd::mfma_peak_sink_words(); }

double wqd_mfma_peak_flops(int64_t iters) { return iters < 1 ? 0.0 : wqd::mfma_peak_flops(iters); }

int wqd_mfma_peak(int64_t iters, float* sink, void* stream) {
  if (!sink || iters < 1) return WQD_E_ARG;
  return hip_status(wqd::launch_mfma_peak(iters, sink, as_stream(stream)));
}

}  // extern "C"
