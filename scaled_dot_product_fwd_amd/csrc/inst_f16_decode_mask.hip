// f16 attention kernels with an explicit mask array, decode family.
#include "attn_launch.h"

namespace sdpa {
int launch_attn_f16_decode_mask(const Plan& p, const AttnArgs& a, void* stream, std::string* err) {
  SDPA_BY_MASK_ARRAY(SDPA_PAIRS16, F16, KIND_DECODE)
  SDPA_NO_INSTANCE()
}
}  // namespace sdpa
