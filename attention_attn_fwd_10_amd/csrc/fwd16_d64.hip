// Instantiations of the 16-bit forward kernels for head_dim 64.
#include "fwd16.hpp"

namespace attn {
ATTN_INSTANTIATE_FWD16(64)
ATTN_INSTANTIATE_FWD16_BIAS(64)
}  // namespace attn
