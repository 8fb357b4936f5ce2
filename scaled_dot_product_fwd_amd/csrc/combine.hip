// Split combine: merges the per-split partial results of one packed row by
// log-sum-exp (mlx issue #3826 "2.3-2.8x latency jump from L=8 to L=12
// queries", third comment: the split-S + logsumexp merge of the 2-pass path).
//
// For splits s with running max m_s (log2 units), sum l_s and unnormalised
// output O_s:  M = max_s m_s,  w_s = 2^(m_s - M),  L = sum_s w_s l_s,
// o = sum_s w_s O_s / L,  lse = ln2 * (M + log2 L).  A split that saw no
// visible key has m_s = -inf and contributes w_s = 0.
#include <hip/hip_runtime.h>

#include <string>

#include "attn_kernel.h"

namespace sdpa {
namespace dev {

constexpr int kCombineThreads = 128;
constexpr int kCombineMaxSplits = 1024;

__device__ __forceinline__ float block_max(float x, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  x = fmaxf(red[0], red[1]);
  __syncthreads();
  return x;
}

__device__ __forceinline__ float block_sum(float x, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  x = red[0] + red[1];
  __syncthreads();
  return x;
}

template <class E>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(CombineArgs a) {
  __shared__ float wsh[kCombineMaxSplits];
  __shared__ float red[2];
  const int row = blockIdx.x;  // z * R + r
  const int z = row / a.R, r = row % a.R;
  const int b = z / a.Hkv, kvh = z % a.Hkv;
  const int g = r % a.G, i = r / a.G, h = kvh * a.G + g;
  const float* ml = a.ws_ml + (int64_t)row * a.splits * 2;
  const int tid = threadIdx.x;

  float mx = kNegInf;
  for (int s = tid; s < a.splits; s += kCombineThreads) mx = fmaxf(mx, ml[2 * s]);
  const float M = block_max(mx, red);
  const float Mu = (M == kNegInf) ? 0.f : M;
  float part = 0.f;
  for (int s = tid; s < a.splits; s += kCombineThreads) {
    const float w = __builtin_amdgcn_exp2f(ml[2 * s] - Mu);
    wsh[s] = w;
    part += w * ml[2 * s + 1];
  }
  const float L = block_sum(part, red);  // its barriers also publish wsh
  const float inv = 1.0f / L;

  const float* wo = a.ws_o + (int64_t)row * a.splits * a.dv;
  char* orow = (char*)a.o + ((int64_t)b * a.os[0] + (int64_t)h * a.os[1] + (int64_t)i * a.os[2]) * E::ES;
  for (int d = tid; d < a.dv; d += kCombineThreads) {
    float acc = 0.f;
    for (int s = 0; s < a.splits; ++s) acc += wsh[s] * wo[(int64_t)s * a.dv + d];
    const float val = acc * inv;
    if constexpr (E::ES == 2) *(unsigned short*)(orow + d * 2) = E::to_store(val);
    else *(float*)(orow + d * 4) = val;
  }
  if (tid == 0 && a.lse) a.lse[((int64_t)b * a.Hq + h) * a.Lq + i] = (Mu + log2f(L)) * kLn2;
}

}  // namespace dev

int launch_combine(const Plan& p, const CombineArgs& a, void* stream, std::string* err) {
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
