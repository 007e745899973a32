// Library-owned scratch for kvs_decode_step_noalloc: a file-scope device array
// that every call on a GPU shares, and the per-device lookup of its address.
//
// The array's name is a host-side stand-in in host code, not a device address:
// kernels and copies only ever receive the address hipGetSymbolAddress returns
// for the current device.  Each GPU the library runs on holds its own copy of
// the array, at its own address, until the process ends.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kvs.h"
#include "kvs_internal.h"

namespace kvs {

static_assert(KVS_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size keeps 256-byte alignment");

static __device__ __align__(256) uint8_t scratch[KVS_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch`, per device ordinal
}  // namespace

void* noalloc_scratch(hipError_t* err) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *err = e;
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // with `dev` current
    if (e != hipSuccess || !p) {
      *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  *err = hipSuccess;
  return g_scratch_ptr[dev];
}

}  // namespace kvs
