// Instantiations of the 16-bit forward kernels for head_dim 64.
#include "fwd16_pp.hpp"

namespace attn {
ATTN_INSTANTIATE_FWD16(64)
ATTN_INSTANTIATE_FWD16_BIAS(64)
ATTN_INSTANTIATE_FWD16PP(64)
}  // namespace attn
