// f16 attention kernels with an explicit mask array, short family.
#include "attn_launch.h"

namespace sdpa {
int launch_attn_f16_short_mask(const Plan& p, const AttnArgs& a, void* stream, std::string* err) {
  SDPA_BY_MASK_ARRAY(SDPA_PAIRS16, F16, KIND_SHORT)
  SDPA_NO_INSTANCE()
}
}  // namespace sdpa
