// f16 attention kernels, head dim 512 (every query length): two waves per
// 32 rows split the dv tiles.
#include "attn_launch.h"

namespace sdpa {
int launch_attn_f16_prefill_xl(const Plan& p, const AttnArgs& a, void* stream, std::string* err) {
  SDPA_PAIRS16_XL(F16, KIND_PREFILL, MA_NONE)
  SDPA_NO_INSTANCE()
}
}  // namespace sdpa
