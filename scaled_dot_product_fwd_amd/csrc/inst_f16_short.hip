// f16 attention kernels, short family.
#include "attn_launch.h"

namespace sdpa {
int launch_attn_f16_short(const Plan& p, const AttnArgs& a, void* stream, std::string* err) {
  SDPA_PAIRS16(F16, KIND_SHORT, MA_NONE)
  SDPA_NO_INSTANCE()
}
}  // namespace sdpa
