// Expand kernels of one weight / output type pair (see expand_kernels.h).
#include "expand_kernels.h"

namespace rax {
RAX_EXPAND_PAIR(w16_y32, uint16_t, float)
}  // namespace rax
