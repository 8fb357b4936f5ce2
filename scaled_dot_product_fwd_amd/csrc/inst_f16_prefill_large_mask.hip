// f16 attention kernels with an explicit mask array, prefill family, head
// dims of 192 and more (iterative ILP scheduler, as for the unmasked ones).
#include "attn_launch.h"

namespace sdpa {
int launch_attn_f16_prefill_xl_mask(const Plan& p, const AttnArgs& a, void* stream, std::string* err);

int launch_attn_f16_prefill_large_mask(const Plan& p, const AttnArgs& a, void* stream, std::string* err) {
  SDPA_BY_MASK_ARRAY(SDPA_PAIRS16_LARGE, F16, KIND_PREFILL)
  return launch_attn_f16_prefill_xl_mask(p, a, stream, err);
}
}  // namespace sdpa
