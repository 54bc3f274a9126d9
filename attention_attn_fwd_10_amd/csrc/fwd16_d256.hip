// Instantiations of the 16-bit forward kernel for head_dim 256.
#include "fwd16.hpp"

namespace attn {
ATTN_INSTANTIATE_FWD16(256)
}  // namespace attn
