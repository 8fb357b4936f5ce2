// f16 attention kernels, prefill family, head dims of 192 and more.  This
// unit is compiled with the iterative ILP scheduler: with one wave per SIMD
// the schedule alone decides how much of the LDS latency the MFMAs hide.
#include "attn_launch.h"

namespace sdpa {
int launch_attn_f16_prefill_xl(const Plan& p, const AttnArgs& a, void* stream, std::string* err);

int launch_attn_f16_prefill_large(const Plan& p, const AttnArgs& a, void* stream, std::string* err) {
  SDPA_PAIRS16_LARGE(F16, KIND_PREFILL, MA_NONE)
  return launch_attn_f16_prefill_xl(p, a, stream, err);
}
}  // namespace sdpa
