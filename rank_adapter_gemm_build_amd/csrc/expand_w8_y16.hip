// Expand kernels of one weight / output type pair (see expand_kernels.h).
#include "expand_kernels.h"

namespace rax {
RAX_EXPAND_PAIR(w8_y16, uint8_t, uint16_t)
}  // namespace rax
