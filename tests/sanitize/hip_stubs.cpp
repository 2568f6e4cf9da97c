// Host stand-ins for the HIP runtime and the library's kernel launchers, for a build of
// the C ABI's host code (api.cpp) under AddressSanitizer and UndefinedBehaviorSanitizer
// on a machine without a GPU.  "Device" memory is host memory, copies are memcpy,
// launches only record that they were asked for.  Test infrastructure only.
#include <hip/hip_runtime_api.h>

#include <cstdlib>
#include <cstring>

#include "common.h"

extern "C" {
hipError_t hipGetDeviceCount(int* n) { *n = 1; return hipSuccess; }
hipError_t hipGetDevice(int* d) { *d = 0; return hipSuccess; }
hipError_t hipSetDevice(int d) { return d == 0 ? hipSuccess : hipErrorInvalidDevice; }
const char* hipGetErrorString(hipError_t) { return "stub"; }
hipError_t hipMalloc(void** p, size_t n) {
  *p = std::malloc(n ? n : 1);
  return *p ? hipSuccess : hipErrorOutOfMemory;
}
hipError_t hipFree(void* p) { std::free(p); return hipSuccess; }
hipError_t hipMemset(void* p, int v, size_t n) { std::memset(p, v, n); return hipSuccess; }
hipError_t hipMemcpy(void* d, const void* s, size_t n, hipMemcpyKind) { std::memcpy(d, s, n); return hipSuccess; }
hipError_t hipMemcpy2D(void* d, size_t dp, const void* s, size_t sp, size_t w, size_t h, hipMemcpyKind) {
  for (size_t r = 0; r < h; ++r) std::memcpy(static_cast<char*>(d) + r * dp, static_cast<const char*>(s) + r * sp, w);
  return hipSuccess;
}
hipError_t hipDeviceSynchronize(void) { return hipSuccess; }
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
hipError_t hipStreamWaitEvent(hipStream_t, hipEvent_t, unsigned int) { return hipSuccess; }
hipError_t hipEventCreate(hipEvent_t* e) {
  static char store[4096][8];
  static int next = 0;
  if (next == 4096) return hipErrorOutOfMemory;
  *e = reinterpret_cast<hipEvent_t>(store[next++]);
  return hipSuccess;
}
hipError_t hipEventSynchronize(hipEvent_t) { return hipSuccess; }
hipError_t hipEventElapsedTime(float* ms, hipEvent_t, hipEvent_t) { *ms = 0.f; return hipSuccess; }
}

int g_launches = 0;   // launches the host code asked for

namespace rax {
hipError_t launch_routing(const int32_t*, int, int, int, int, int, int, int*, int*, int*, int*, int4*, int4*, int*,
                          int*, hipStream_t, const KTimer&) { ++g_launches; return hipSuccess; }
hipError_t launch_pack_slice(int, const void*, const void*, void*, void*, void*, int, int, int, int, int, int, float,
                             int, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_set_slot(SlotEntry* table, int slot, SlotEntry e, hipStream_t) {
  table[slot] = e;   // the stub table is host memory: keep it like the device would
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_shrink(int, const PoolView&, const RouteView&, const void*, int, const UView&, const Plan&,
                         const SelfRoute*, hipStream_t, const KTimer&) { ++g_launches; return hipSuccess; }
hipError_t launch_expand(int, int, const PoolView&, const SlotOrder&, const RouteView&, const UView&, void*, int,
                         const Plan&, hipStream_t, const KTimer&) { ++g_launches; return hipSuccess; }
hipError_t launch_embed_gather(int, const PoolView&, const RouteView&, const int32_t*, int, const UView&, hipStream_t,
                               const KTimer&) { ++g_launches; return hipSuccess; }
hipError_t launch_embed_gather_tok(int, const PoolView&, const RouteView&, const int32_t*, const int32_t*, int,
                                   const UView&, const SelfRoute*, hipStream_t, const KTimer&) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_finish_u(const PoolView&, const RouteView&, const UView&, const UView&, const Plan&, hipStream_t,
                           const KTimer&) { ++g_launches; return hipSuccess; }
hipError_t launch_shrink_group(int, const GroupView& G, const RouteView&, const SelfRoute*, hipStream_t, const KTimer&) {
  if (G.n < 1 || G.n > kMaxGroup) return hipErrorInvalidValue;
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_expand_group(int, int, const GroupView& G, const RouteView&, hipStream_t, const KTimer&) {
  if (G.n < 1 || G.n > kMaxGroup) return hipErrorInvalidValue;
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_bandwidth_probe(const void*, size_t, void*, size_t, int, hipStream_t) { ++g_launches; return hipSuccess; }
static float g_scratch[kNoAllocScratchBytes / sizeof(float)];
hipError_t noalloc_scratch(int, void** ptr) {
  *ptr = g_scratch;
  return hipSuccess;
}
}  // namespace rax
