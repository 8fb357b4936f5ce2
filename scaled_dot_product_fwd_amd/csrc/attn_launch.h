// Launch glue shared by the per-(element type, family) instantiation units.
#pragma once

#include <hip/hip_runtime.h>

#include <string>

#include "attn_kernel.h"

namespace sdpa {

template <class E, int DQK, int DV, int NWQ, int NWK, int BKW, int WPE, int MA, int NWD>
int launch_one(const Plan& p, const AttnArgs& a, void* stream, std::string* err) {
  using S = dev::Shape<E, DQK, DV, NWQ, NWK, BKW, MA, NWD>;
  auto kern = dev::attn_fwd_kernel<E, DQK, DV, NWQ, NWK, BKW, WPE, MA, NWD>;
  // Check the compiled kernel can run the workgroup size it is launched with,
  // once per instance: an oversized launch must fail loudly, never return
  // silently unwritten output (mlx PR #4185 "Add force_fused option to
  // scaled_dot_product_attention", Kernel support: pipeline size check).
  static int checked = 0;  // 0 unknown, 1 ok, -1 unusable
  if (checked == 0) {
    hipFuncAttributes attr;
    if (hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(kern)) != hipSuccess) {
      *err = "hipFuncGetAttributes failed for the attention kernel";
      return SDPA_E_HIP;
    }
    checked = (attr.maxThreadsPerBlock >= S::NT && attr.sharedSizeBytes <= 160 * 1024) ? 1 : -1;
    if (checked < 0) {
      *err = "attention kernel cannot run " + std::to_string(S::NT) + " threads per workgroup (max " +
             std::to_string(attr.maxThreadsPerBlock) + ", lds " + std::to_string(attr.sharedSizeBytes) + ")";
      return SDPA_E_HIP;
    }
  } else if (checked < 0) {
    *err = "attention kernel cannot run its workgroup size on this device";
    return SDPA_E_HIP;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)p.grid), dim3(S::NT), 0, (hipStream_t)stream, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    *err = std::string("attention kernel launch failed: ") + hipGetErrorString(e);
    return SDPA_E_HIP;
  }
  return SDPA_OK;
}

}  // namespace sdpa

// One dispatch case: the plan's padded dims (and mask array kind MA) select
// the instance; the wave arrangement follows from the kind exactly as in the
// planner.
#define SDPA_CASE(E, KIND, DQK, DV, MA)                                                        \
  if (p.dqk_pad == DQK && p.dv_pad == DV) {                                                    \
    constexpr Family f_ = family_for(KIND, dev::E::ES, DQK, DV, mask_elem_bytes(MA, dev::E::ES)); \
    if (p.fam.nwq != f_.nwq || p.fam.nwk != f_.nwk || p.fam.bkw != f_.bkw || p.fam.nwd != f_.nwd || \
        p.mask_array != MA) {                                                                  \
      *err = "plan and kernel instance disagree on the wave arrangement";                      \
      return SDPA_E_PLAN;                                                                      \
    }                                                                                          \
    return launch_one<dev::E, DQK, DV, f_.nwq, f_.nwk, f_.bkw,                                 \
                      wpe_for(KIND, dev::E::ES, DQK, DV), MA, f_.nwd>(p, a, stream, err);      \
  }

// Head-dim pairs of the 16-bit types: equal padded dims plus (80, 96) and
// (192, 128), split at 192 so that the large ones can live in units of
// their own.
#define SDPA_PAIRS16_SMALL(E, KIND, MA) \
  SDPA_CASE(E, KIND, 32, 32, MA)         \
  SDPA_CASE(E, KIND, 64, 64, MA)         \
  SDPA_CASE(E, KIND, 80, 96, MA)         \
  SDPA_CASE(E, KIND, 96, 96, MA)         \
  SDPA_CASE(E, KIND, 128, 128, MA)       \
  SDPA_CASE(E, KIND, 160, 160, MA)
#define SDPA_PAIRS16_LARGE(E, KIND, MA) \
  SDPA_CASE(E, KIND, 192, 192, MA)       \
  SDPA_CASE(E, KIND, 224, 224, MA)       \
  SDPA_CASE(E, KIND, 256, 256, MA)       \
  SDPA_CASE(E, KIND, 192, 128, MA)
#define SDPA_PAIRS16(E, KIND, MA) SDPA_PAIRS16_SMALL(E, KIND, MA) SDPA_PAIRS16_LARGE(E, KIND, MA)
// head dim 512 (16-bit types, prefill family only: the planner sends every
// query length there)
#define SDPA_PAIRS16_XL(E, KIND, MA) SDPA_CASE(E, KIND, 512, 512, MA)

// head dims up to 128 (the wide family), 16-bit types
#define SDPA_PAIRS16_UPTO128(E, KIND, MA) \
  SDPA_CASE(E, KIND, 32, 32, MA)         \
  SDPA_CASE(E, KIND, 64, 64, MA)         \
  SDPA_CASE(E, KIND, 80, 96, MA)         \
  SDPA_CASE(E, KIND, 96, 96, MA)         \
  SDPA_CASE(E, KIND, 128, 128, MA)
// float32 wide: head dims up to 96 (two waves per SIMD)
#define SDPA_PAIRS32_UPTO96(E, KIND, MA) \
  SDPA_CASE(E, KIND, 32, 32, MA)         \
  SDPA_CASE(E, KIND, 64, 64, MA)         \
  SDPA_CASE(E, KIND, 96, 96, MA)

// float32 stops at 128.
#define SDPA_PAIRS32(E, KIND, MA)  \
  SDPA_CASE(E, KIND, 32, 32, MA)   \
  SDPA_CASE(E, KIND, 64, 64, MA)   \
  SDPA_CASE(E, KIND, 96, 96, MA)   \
  SDPA_CASE(E, KIND, 128, 128, MA)

// Mask-array units: the plan's array kind picks the boolean or additive set.
#define SDPA_BY_MASK_ARRAY(PAIRS, E, KIND) \
  if (p.mask_array == MA_BOOL) {           \
    PAIRS(E, KIND, MA_BOOL)                \
  } else {                                 \
    PAIRS(E, KIND, MA_ADD)                 \
  }

#define SDPA_NO_INSTANCE()                                                               \
  *err = "no kernel instance for dqk_pad=" + std::to_string(p.dqk_pad) +                 \
         " dv_pad=" + std::to_string(p.dv_pad);                                          \
  return SDPA_E_HEAD_DIM;
