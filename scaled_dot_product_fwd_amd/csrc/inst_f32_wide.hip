// f32 attention kernels, wide family (256-row tiles, head dims up to 96).
#include "attn_launch.h"

namespace sdpa {
int launch_attn_f32_wide(const Plan& p, const AttnArgs& a, void* stream, std::string* err) {
  SDPA_PAIRS32_UPTO96(F32, KIND_WIDE, MA_NONE)
  SDPA_NO_INSTANCE()
}
}  // namespace sdpa
