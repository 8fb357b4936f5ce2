// f32 attention kernels, prefill family.
#include "attn_launch.h"

namespace sdpa {
int launch_attn_f32_prefill(const Plan& p, const AttnArgs& a, void* stream, std::string* err) {
  SDPA_PAIRS32(F32, KIND_PREFILL, MA_NONE)
  SDPA_NO_INSTANCE()
}
}  // namespace sdpa
