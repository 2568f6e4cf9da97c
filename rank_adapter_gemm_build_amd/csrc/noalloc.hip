// Scratch memory for the allocation-free entry point (lora_linear_noalloc): a fixed
// array in the library's device image, so a call needs no device allocation at all.
// Each GPU the library runs on holds its own copy until the process ends.
//
// In host code the array's name is only a host-side handle of the symbol, not a
// device address: the device address is taken once per device with
// hipGetSymbolAddress (with that device current) and kept; only that address is
// ever handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "common.h"

namespace rax {

static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(int device, void** ptr) {
  if (!ptr || device < 0 || device >= kMaxDevices) return hipErrorInvalidValue;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != device) return hipErrorInvalidDevice;   // the caller makes `device` current first
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[device] = p;
  }
  *ptr = g_scratch_ptr[device];
  return hipSuccess;
}

}  // namespace rax
