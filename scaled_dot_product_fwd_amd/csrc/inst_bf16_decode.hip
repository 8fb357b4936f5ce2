// bf16 attention kernels, decode family.
#include "attn_launch.h"

namespace sdpa {
int launch_attn_bf16_decode(const Plan& p, const AttnArgs& a, void* stream, std::string* err) {
  SDPA_PAIRS16(BF16, KIND_DECODE, MA_NONE)
  SDPA_NO_INSTANCE()
}
}  // namespace sdpa
