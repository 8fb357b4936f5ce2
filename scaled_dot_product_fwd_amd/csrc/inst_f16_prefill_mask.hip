// f16 attention kernels with an explicit mask array, prefill family.
#include "attn_launch.h"

namespace sdpa {
int launch_attn_f16_prefill_large_mask(const Plan& p, const AttnArgs& a, void* stream, std::string* err);

int launch_attn_f16_prefill_mask(const Plan& p, const AttnArgs& a, void* stream, std::string* err) {
  SDPA_BY_MASK_ARRAY(SDPA_PAIRS16_SMALL, F16, KIND_PREFILL)
  return launch_attn_f16_prefill_large_mask(p, a, stream, err);
}
}  // namespace sdpa
