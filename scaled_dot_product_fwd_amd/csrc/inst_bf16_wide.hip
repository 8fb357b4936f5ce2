// bf16 attention kernels, wide family (256-row tiles, head dims up to 128).
#include "attn_launch.h"

namespace sdpa {
int launch_attn_bf16_wide(const Plan& p, const AttnArgs& a, void* stream, std::string* err) {
  SDPA_PAIRS16_UPTO128(BF16, KIND_WIDE, MA_NONE)
  SDPA_NO_INSTANCE()
}
}  // namespace sdpa
