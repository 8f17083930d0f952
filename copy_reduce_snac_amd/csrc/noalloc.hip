// noalloc.hip -- the device memory of snac_all_reduce_atomic_static: a
// file-scope device array that holds the binary32 accumulator of the
// non-deterministic AllReduce for callers that cannot allocate (code under
// HIP graph capture, serving loops, harnesses that forbid hipMalloc).
//
// The array is sized once, here; every GPU the library runs on holds its own
// copy until the process ends, at its own address.  Host code never passes
// the array's name to a kernel (on the host it is only a stand-in for the
// symbol): the device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and kept.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.hpp"

namespace snac {

namespace {

constexpr int kScratchDevices = 64;

__device__ __align__(256) float scratch[kStaticScratchBytes / sizeof(float)];

std::once_flag g_once[kScratchDevices];
float* g_ptr[kScratchDevices];
hipError_t g_err[kScratchDevices];

}  // namespace

hipError_t static_scratch(float** out) {
  *out = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_ptr[dev] = static_cast<float*>(p);
  });
  if (g_err[dev] != hipSuccess) return g_err[dev];
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace snac
