// Matrix-core (MFMA) kernels for long same-slot segments: not compiled in yet
// (kHaveMfmaPath is false, so the dispatcher never calls these launchers).
#include <hip/hip_runtime.h>

#include "device_util.h"

namespace rax {

hipError_t launch_shrink_mfma(const PoolView&, const RouteView&, const void*, int, const UView&, int,
                              hipStream_t, const KTimer&) {
  return hipErrorNotSupported;
}

hipError_t launch_expand_mfma(int, const PoolView&, const RouteView&, const UView&, void*, int,
                              hipStream_t, const KTimer&) {
  return hipErrorNotSupported;
}

}  // namespace rax
