// f16 attention kernels, decode family.
#include "attn_launch.h"

namespace sdpa {
int launch_attn_f16_decode(const Plan& p, const AttnArgs& a, void* stream, std::string* err) {
  SDPA_PAIRS16(F16, KIND_DECODE, MA_NONE)
  SDPA_NO_INSTANCE()
}
}  // namespace sdpa
