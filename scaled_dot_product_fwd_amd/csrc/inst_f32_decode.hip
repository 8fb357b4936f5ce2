// f32 attention kernels, decode family.
#include "attn_launch.h"

namespace sdpa {
int launch_attn_f32_decode(const Plan& p, const AttnArgs& a, void* stream, std::string* err) {
  SDPA_PAIRS32(F32, KIND_DECODE, MA_NONE)
  SDPA_NO_INSTANCE()
}
}  // namespace sdpa
