// Instantiations of the 16-bit forward kernel for head_dim 64.
#include "fwd16.hpp"

namespace attn {
ATTN_INSTANTIATE_FWD16(64)
}  // namespace attn
