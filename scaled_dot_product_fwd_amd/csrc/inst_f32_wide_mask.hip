// f32 attention kernels with an explicit mask array, wide family.
#include "attn_launch.h"

namespace sdpa {
int launch_attn_f32_wide_mask(const Plan& p, const AttnArgs& a, void* stream, std::string* err) {
  SDPA_BY_MASK_ARRAY(SDPA_PAIRS32_UPTO96, F32, KIND_WIDE)
  SDPA_NO_INSTANCE()
}
}  // namespace sdpa
