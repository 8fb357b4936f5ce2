// bf16 attention kernels, prefill family.
#include "attn_launch.h"

namespace sdpa {
int launch_attn_bf16_prefill_large(const Plan& p, const AttnArgs& a, void* stream, std::string* err);

int launch_attn_bf16_prefill(const Plan& p, const AttnArgs& a, void* stream, std::string* err) {
  SDPA_PAIRS16_SMALL(BF16, KIND_PREFILL, MA_NONE)
  return launch_attn_bf16_prefill_large(p, a, stream, err);
}
}  // namespace sdpa
