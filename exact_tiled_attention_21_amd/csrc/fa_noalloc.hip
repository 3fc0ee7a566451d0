// Fixed device scratch for the decode entry point that allocates nothing
// (fa_decode_splitkv_noalloc): the split kernel's per-part partial results live
// in a file-scope device array instead of a caller's workspace. Each GPU the
// library runs on holds its own copy of the array, at its own address, until the
// process ends; every call on a GPU shares that GPU's copy, so calls that
// overlap on one GPU race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/fa.h"

static __device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace fa {
namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];   // device address of `scratch` per device, looked up once
}  // namespace

// The current device's address of the scratch array (looked up with
// hipGetSymbolAddress on the first call on that device; host code uses this
// address, never the array's name, which on the host is only a stand-in).
fa_status noalloc_scratch(void** ptr, size_t* bytes) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return FA_ERR_LAUNCH;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  *bytes = FA_NOALLOC_SCRATCH_BYTES;
  return FA_OK;
}

}  // namespace fa
