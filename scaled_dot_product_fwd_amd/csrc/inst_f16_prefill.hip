// f16 attention kernels, prefill family.
#include "attn_launch.h"

namespace sdpa {
int launch_attn_f16_prefill(const Plan& p, const AttnArgs& a, void* stream, std::string* err) {
  SDPA_PAIRS16(F16, KIND_PREFILL)
  SDPA_NO_INSTANCE()
}
}  // namespace sdpa
