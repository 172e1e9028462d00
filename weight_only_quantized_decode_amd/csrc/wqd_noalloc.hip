// wqd_qgemm_noalloc: the decode product for callers that cannot allocate
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  It runs the same kernels as wqd_qgemm; the split-K partials and
// W4A16 group x sums that wqd_qgemm keeps in a caller workspace go to a
// file-scope device array instead, one copy per GPU, held until the process
// ends.  Host code never passes the array's name to a kernel (in host code it
// is a stand-in, not a device address): the device address comes from
// hipGetSymbolAddress, taken once per device with that device current, and
// only that address is used.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/wqd.h"
#include "wqd_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(WQD_NOALLOC_SCRATCH_BYTES);
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch address on the current device (nullptr and a HIP error on failure).
void* device_scratch(hipError_t* err) {
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" int wqd_qgemm_noalloc(int fmt, const void* x, int64_t M, int64_t N, int64_t K, const void* w_packed,
                                 const void* scales, const void* zeros, void* y, void* stream) {
  size_t need = 0;
  const int st = wqd_workspace_bytes(fmt, M, N, K, &need);
  if (st != WQD_OK) return st;
  if (need > kScratchBytes) return WQD_E_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    hipError_t err = hipSuccess;
    ws = device_scratch(&err);
    if (!ws) return wqd::record_hip_error(err == hipSuccess ? hipErrorUnknown : err);
  }
  return wqd::qgemm_checked(fmt, x, M, N, K, w_packed, scales, zeros, y, ws, need, stream);
}
