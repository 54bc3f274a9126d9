// 8-bit fused forward (placeholder until the e4m3 kernel lands).
#include "common.hpp"

namespace attn {
hipError_t launch_fwd_fp8(const Fp8Args&, int, bool, hipStream_t) { return hipErrorNotSupported; }
}  // namespace attn
