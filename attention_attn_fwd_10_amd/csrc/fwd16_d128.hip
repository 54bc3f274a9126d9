// Instantiations of the 16-bit forward kernels for head_dim 128.
#include "fwd16.hpp"

namespace attn {
ATTN_INSTANTIATE_FWD16(128)
ATTN_INSTANTIATE_FWD16_BIAS(128)
ATTN_INSTANTIATE_FWD16_WIDE(128)
}  // namespace attn
