// Library-held scratch of td_denoise_step_noalloc: one file-scope device
// array per GPU, in place of a caller workspace, for callers that cannot
// allocate device memory during a run (code under stream capture, tight
// serving loops, harnesses that forbid hipMalloc).
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is looked up once per device with hipGetSymbolAddress,
// with that device current, and only that address is ever handed to
// kernels.  Every call on one GPU shares that GPU's array; the kernels of
// the step write every scratch byte they later read within the same call,
// so nothing in it has to start at zero.
#include <hip/hip_runtime.h>

#include <mutex>

#include "td_internal.h"

namespace td {
namespace {

static __device__ __align__(256) unsigned char scratch[TD_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void *g_ptr[kMaxDevices];
int g_err[kMaxDevices];

void lookup(int dev) {
  void *p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  g_err[dev] = (e == hipSuccess && p != nullptr) ? TD_OK : TD_ERR_HIP;
  g_ptr[dev] = g_err[dev] == TD_OK ? p : nullptr;
}

}  // namespace

int noalloc_scratch(void **ptr) {
  *ptr = nullptr;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return TD_ERR_HIP;
  if (dev >= kMaxDevices) return TD_ERR_UNSUPPORTED;
  // the current device is the one the symbol is looked up on
  std::call_once(g_once[dev], lookup, dev);
  if (g_err[dev] != TD_OK) return g_err[dev];
  *ptr = g_ptr[dev];
  return TD_OK;
}

}  // namespace td
