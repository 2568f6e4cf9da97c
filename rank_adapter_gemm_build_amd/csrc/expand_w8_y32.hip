// Expand kernels of one weight / output type pair (see expand_kernels.h).
#include "expand_kernels.h"

namespace rax {
RAX_EXPAND_PAIR(w8_y32, uint8_t, float)
}  // namespace rax
