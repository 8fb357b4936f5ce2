// bf16 attention kernels, prefill family.
#include "attn_launch.h"

namespace sdpa {
int launch_attn_bf16_prefill(const Plan& p, const AttnArgs& a, void* stream, std::string* err) {
  SDPA_PAIRS16(BF16, KIND_PREFILL)
  SDPA_NO_INSTANCE()
}
}  // namespace sdpa
