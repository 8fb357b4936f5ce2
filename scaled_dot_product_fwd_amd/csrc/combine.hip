// Split combine: merges the per-split partial results of one packed row by
// log-sum-exp (mlx issue #3826 "2.3-2.8x latency jump from L=8 to L=12
// queries", third comment: the two-pass kernel there merges the partial
// results of its key splits by log-sum-exp).
//
// For splits s with running max m_s (log2 units), sum l_s and unnormalised
// output O_s:  M = max_s m_s,  w_s = 2^(m_s - M),  L = sum_s w_s l_s,
// o = sum_s w_s O_s / L,  lse = ln2 * (M + log2 L).  A split that saw no
// visible key has m_s = -inf and contributes w_s = 0; a row with no visible
// key in any split (possible only through a mask array) writes o = 0 and
// lse = -inf.
#include <hip/hip_runtime.h>

#include <string>

#include "attn_kernel.h"

namespace sdpa {
namespace dev {

constexpr int kCombineThreads = 256;
constexpr int kCombineMaxSplits = kMaxSplitsPerRow;
constexpr int kCombineRegs = 8;  // partial outputs a thread holds in registers

// One workgroup per packed row.  Thread (g, c) owns 4 head-dim columns c of
// the splits s = g, g + NG, g + 2 NG, ... (NG = threads / (dv / 4)); every
// load it needs -- its (m, l) pair and up to kCombineRegs partial outputs --
// is issued before the first wait, so a row costs one memory round trip.
// The weights follow once the row max is known; the NG group sums are added
// in LDS.
template <class E>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(CombineArgs a) {
  __shared__ float msh[kCombineMaxSplits];
  __shared__ f32x4 part[kCombineThreads];
  __shared__ float red[kCombineThreads / 64], red_l[kCombineThreads / 64];
  // row = z * R + r; with xcd_rows the workgroups of XCD w % 8 take the
  // rows of the KV heads z = w % 8 (mod 8), whose splits ran on that XCD
  const int w = blockIdx.x;
  const int z = a.xcd_rows ? 8 * (w / (8 * a.R)) + w % 8 : w / a.R;
  const int r = a.xcd_rows ? (w / 8) % a.R : w % a.R;
  const int row = z * a.R + r;
  const int b = z / a.Hkv, kvh = z % a.Hkv;
  const int g = r % a.G, i = r / a.G, h = kvh * a.G + g;
  if (a.q_lens && i >= min(max(a.q_lens[b], 0), a.Lq)) return;  // past the entry's queries: not written
  // this row's partials: [row][split], or with balanced lengths [r][split]
  // inside its entry's segment of the KV head (see kv_balance_count)
  int ns = a.splits;
  int64_t prow = (int64_t)row * a.splits;  // first partial of the row
  if (a.kv_balance > 0) {
    const int W = a.B * a.splits;
    const int T = kv_balance_total(a.kv_lens, a.B, a.Lk, a.kv_balance);
    int P = 0;
    for (int e = 0; e < b; ++e)
      P += kv_balance_count(kv_balance_blocks(a.kv_lens, e, a.Lk, a.kv_balance), W, a.B, T);
    ns = kv_balance_count(kv_balance_blocks(a.kv_lens, b, a.Lk, a.kv_balance), W, a.B, T);
    prow = ((int64_t)kvh * W + P) * a.R + (int64_t)r * ns;
  }
  const float* ml = a.ws_ml + prow * 2;
  const int tid = threadIdx.x;
  const int nc = a.dv / 4;              // 4-column groups: dv % 8 == 0, dv <= 4 * threads
  const int ng = kCombineThreads / nc;  // split groups
  const int gi = tid / nc, c = tid % nc;
  const float* wo = a.ws_o + prow * a.dv + 4 * c;

  f32x4 v[kCombineRegs];
#pragma unroll
  for (int u = 0; u < kCombineRegs; ++u) {
    const int sp = gi + u * ng;
    v[u] = (gi < ng && sp < ns) ? *(const f32x4*)(wo + (int64_t)sp * a.dv) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float mx = kNegInf, lp_m = kNegInf, lp_l = 0.f;
  for (int sp = tid; sp < ns; sp += kCombineThreads) {
    const float2 q = *(const float2*)(ml + 2 * sp);
    msh[sp] = q.x;
    if (sp == tid) { lp_m = q.x; lp_l = q.y; }  // first pair of this thread, kept for the sum
    mx = fmaxf(mx, q.x);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();  // also publishes msh
  float M = red[0];
#pragma unroll
  for (int w = 1; w < kCombineThreads / 64; ++w) M = fmaxf(M, red[w]);
  const float Mu = (M == kNegInf) ? 0.f : M;

  // L = sum_s 2^(m_s - M) l_s
  float lp = tid < ns ? __builtin_amdgcn_exp2f(lp_m - Mu) * lp_l : 0.f;
  for (int sp = tid + kCombineThreads; sp < ns; sp += kCombineThreads)
    lp += __builtin_amdgcn_exp2f(msh[sp] - Mu) * ml[2 * sp + 1];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) lp += __shfl_xor(lp, o);
  if ((tid & 63) == 0) red_l[tid >> 6] = lp;

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (gi < ng) {
#pragma unroll
    for (int u = 0; u < kCombineRegs; ++u) {
      const int sp = gi + u * ng;
      if (sp < ns) acc += __builtin_amdgcn_exp2f(msh[sp] - Mu) * v[u];
    }
    for (int sp = gi + kCombineRegs * ng; sp < ns; sp += ng)
      acc += __builtin_amdgcn_exp2f(msh[sp] - Mu) * *(const f32x4*)(wo + (int64_t)sp * a.dv);
  }
  part[tid] = acc;
  __syncthreads();  // publishes part and red_l
  if (tid < nc) {
    f32x4 sum = part[tid];
    for (int q = 1; q < ng; ++q) sum += part[q * nc + tid];
    float L = red_l[0];
#pragma unroll
    for (int w = 1; w < kCombineThreads / 64; ++w) L += red_l[w];
    const float inv = L > 0.f ? 1.0f / L : 0.f;  // L = 0: a mask array left the row no key
    char* orow = (char*)a.o + ((int64_t)b * a.os[0] + (int64_t)h * a.os[1] + (int64_t)i * a.os[2]) * E::ES;
    const int d = 4 * tid;
    if constexpr (E::ES == 2) {
      u32x2 w;
      w[0] = E::pack2(sum[0] * inv, sum[1] * inv);
      w[1] = E::pack2(sum[2] * inv, sum[3] * inv);
      *(u32x2*)(orow + d * 2) = w;
    } else {
      *(f32x4*)(orow + d * 4) = sum * inv;
    }
    if (tid == 0 && a.lse) a.lse[((int64_t)b * a.Hq + h) * a.Lq + i] = (Mu + log2f(L)) * kLn2;
  }
}

}  // namespace dev

int launch_combine(const Plan& p, const CombineArgs& a, void* stream, std::string* err) {
  if (a.dv > 4 * dev::kCombineThreads || a.dv % 4 != 0) {
    *err = "combine supports head dims up to " + std::to_string(4 * dev::kCombineThreads);
    return SDPA_E_PLAN;
  }
  if (a.splits > dev::kCombineMaxSplits) {
    *err = "combine supports at most " + std::to_string(dev::kCombineMaxSplits) + " splits";
    return SDPA_E_PLAN;
  }
  const dim3 grid((unsigned)p.combine_grid), block(dev::kCombineThreads);
  switch (p.dtype) {
    case SDPA_BF16: hipLaunchKernelGGL(dev::combine_kernel<dev::BF16>, grid, block, 0, (hipStream_t)stream, a); break;
    case SDPA_F16: hipLaunchKernelGGL(dev::combine_kernel<dev::F16>, grid, block, 0, (hipStream_t)stream, a); break;
    default: hipLaunchKernelGGL(dev::combine_kernel<dev::F32>, grid, block, 0, (hipStream_t)stream, a); break;
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    *err = std::string("combine kernel launch failed: ") + hipGetErrorString(e);
    return SDPA_E_HIP;
  }
  return SDPA_OK;
}

}  // namespace sdpa
