// noalloc.hip -- the workspace of rtl_linear_fused_noalloc: a file-scope device array,
// one copy per GPU (each device that loads the library holds it until the process ends),
// so that the call needs no hipMalloc.  Host code never uses the array's name as an
// address (in host code it is only a stand-in for the symbol): each device's address is
// resolved once, with that device current, by hipGetSymbolAddress and kept per device.
#include <mutex>

#include "rtl_launch.h"

namespace rtl {

constexpr size_t kNoallocBytes = (size_t)192 << 20;
static __device__ __align__(256) uint8_t scratch[kNoallocBytes];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];
}  // namespace

size_t noalloc_scratch_bytes() { return kNoallocBytes; }

hipError_t noalloc_scratch(hipStream_t stream, void** out, int* mismatch) {
  *out = nullptr;
  *mismatch = 0;
  int dev = 0, sdev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipStreamGetDevice(stream, &sdev);
  if (e != hipSuccess) return e;
  if (sdev != dev) {  // the address must be resolved with the stream's device current
    *mismatch = 1;
    return hipSuccess;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_ptr[dev] = p;
  });
  if (g_err[dev] != hipSuccess) return g_err[dev];
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace rtl
