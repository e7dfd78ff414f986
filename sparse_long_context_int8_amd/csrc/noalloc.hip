// Device-resident scratch of spmla_prefill_noalloc: a fixed array in the
// library's device image, so that callers which cannot allocate (code under
// stream capture, tight serving loops) can still run the whole layer.
//
// Each GPU that loads the library holds its own copy of the array, at its own
// address, until the process ends. In host code the array's name is only a
// host-side stand-in: its device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and that pointer is what
// every launch receives.
#include <mutex>

#include "spmla_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[spmla::kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

}  // namespace

namespace spmla {

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_ptr[dev] = g_err[dev] == hipSuccess ? p : nullptr;
  });
  if (g_err[dev] != hipSuccess) return g_err[dev];
  if (!g_ptr[dev]) return hipErrorInvalidSymbol;
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace spmla
