// vc_attn_bf16.hip -- in-house BF16 flash-attention baseline (placeholder
// until the BF16 kernel lands; reports "not supported").
#include "vc_common.hpp"
#include "vc_launch.hpp"

namespace vc {

hipError_t launch_attn_bf16(const vc_shape&, float, int, uint32_t, Bshd, Bshd, const uint16_t*, BshdOut,
                            hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace vc
