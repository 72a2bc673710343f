// hq_quant_linear_noalloc: hq_quant_linear for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, hosts
// that forbid allocation). Its workspace is a file-scope device array of
// HQ_NOALLOC_SCRATCH_BYTES, one copy per GPU, held until the process ends.
//
// The array's name is a host-side stand-in in host code: its device address
// is looked up once per device (hipGetSymbolAddress, with that device
// current, on the first call there) and only that address is passed on. The
// kernels are those of hq_quant_linear, which write every workspace byte they
// later read, so nothing needs clearing between calls. Every call on a GPU
// shares that GPU's array: calls that overlap on one GPU (concurrent streams
// or host threads) race and must be serialised by the caller.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "../../include/hq.h"
#include "hq_internal.h"

namespace {

__device__ __align__(256) uint8_t scratch[HQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up once per
// device), or NULL with the error set.
void* scratch_of_current_device(int* status) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *status = hq::set_error(HQ_ERR_HIP, hipGetErrorString(e));
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *status = hq::set_error(HQ_ERR_UNSUPPORTED, "device index beyond the supported 64 devices");
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      char msg[256];
      std::snprintf(msg, sizeof(msg), "hipGetSymbolAddress of the scratch array: %s",
                    hipGetErrorString(e));
      *status = hq::set_error(HQ_ERR_HIP, msg);
      return nullptr;
    }
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" int hq_quant_linear_noalloc(const hq_desc* desc, const void* prepared, const void* X,
                                       int64_t T, void* Y, void* stream) {
  const int st = hq_validate(desc);
  if (st != HQ_OK) return st;
  if (T < 0) return hq::set_error(HQ_ERR_INVALID_ARG, "T must be >= 0");
  if (T == 0) return HQ_OK;
  const size_t need = hq_workspace_bytes(desc, T);
  if (need > size_t(HQ_NOALLOC_SCRATCH_BYTES)) {
    char msg[256];
    std::snprintf(msg, sizeof(msg),
                  "this call needs %zu workspace bytes, more than the %zu of the static "
                  "scratch array; use hq_quant_linear with a caller-owned workspace",
                  need, size_t(HQ_NOALLOC_SCRATCH_BYTES));
    return hq::set_error(HQ_ERR_WORKSPACE, msg);
  }
  int status = HQ_OK;
  void* ws = scratch_of_current_device(&status);
  if (!ws) return status;
  return hq_quant_linear(desc, prepared, X, T, Y, ws, size_t(HQ_NOALLOC_SCRATCH_BYTES), stream);
}
