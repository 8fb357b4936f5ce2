// bf16 attention kernels with an explicit mask array, head dim 512.
#include "attn_launch.h"

namespace sdpa {
int launch_attn_bf16_prefill_xl_mask(const Plan& p, const AttnArgs& a, void* stream, std::string* err) {
  SDPA_BY_MASK_ARRAY(SDPA_PAIRS16_XL, BF16, KIND_PREFILL)
  SDPA_NO_INSTANCE()
}
}  // namespace sdpa
