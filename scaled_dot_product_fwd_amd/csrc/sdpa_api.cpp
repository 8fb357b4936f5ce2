// C entry points of libsdpa_fwd (declared in include/sdpa.h).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>

#include "sdpa_internal.h"

namespace {

thread_local std::string g_last_error;
thread_local hipEvent_t g_prof_start = nullptr;
thread_local hipEvent_t g_prof_stop = nullptr;

int set_error(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

int ok() {
  g_last_error.clear();
  return SDPA_OK;
}

// gfx950 check of the current device, cached per device ordinal.
int check_device(std::string* err) {
  static std::mutex mu;
  static signed char state[64] = {0};  // 0 unknown, 1 gfx950, -1 other
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    *err = "no HIP device is available";
    return SDPA_E_DEVICE;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (dev < 64 && state[dev] != 0) {
    if (state[dev] > 0) return SDPA_OK;
    *err = "the current HIP device is not a gfx950 (MI355X-class) GPU";
    return SDPA_E_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    *err = "hipGetDeviceProperties failed";
    return SDPA_E_DEVICE;
  }
  const bool is950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) state[dev] = is950 ? 1 : -1;
  if (!is950) {
    *err = std::string("the current HIP device is ") + prop.gcnArchName + ", not gfx950";
    return SDPA_E_DEVICE;
  }
  return SDPA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" {

int sdpa_desc_init(sdpa_desc_t* d, int64_t batch, int64_t heads_q, int64_t heads_kv, int64_t len_q,
                   int64_t len_k, int64_t dim_qk, int64_t dim_v, int32_t dtype) {
  if (!d) return set_error(SDPA_E_NULL, "desc is NULL");
  std::memset(d, 0, sizeof(*d));
  d->batch = batch;
  d->heads_q = heads_q;
  d->heads_kv = heads_kv;
  d->len_q = len_q;
  d->len_k = len_k;
  d->dim_qk = dim_qk;
  d->dim_v = dim_v;
  d->q_stride[2] = dim_qk;
  d->q_stride[1] = len_q * dim_qk;
  d->q_stride[0] = heads_q * len_q * dim_qk;
  d->k_stride[2] = dim_qk;
  d->k_stride[1] = len_k * dim_qk;
  d->k_stride[0] = heads_kv * len_k * dim_qk;
  d->v_stride[2] = dim_v;
  d->v_stride[1] = len_k * dim_v;
  d->v_stride[0] = heads_kv * len_k * dim_v;
  d->o_stride[2] = dim_v;
  d->o_stride[1] = len_q * dim_v;
  d->o_stride[0] = heads_q * len_q * dim_v;
  d->dtype = dtype;
  d->mask = SDPA_MASK_NONE;
  d->window = 0;
  d->scale = dim_qk > 0 ? (float)(1.0 / std::sqrt((double)dim_qk)) : 1.0f;
  return ok();
}

int sdpa_workspace_bytes(const sdpa_desc_t* d, size_t* bytes) {
  if (!bytes) return set_error(SDPA_E_NULL, "bytes is NULL");
  sdpa::Plan p;
  std::string err;
  const int rc = sdpa::make_plan(d, &p, &err);
  if (rc != SDPA_OK) return set_error(rc, err);
  *bytes = p.workspace;
  return ok();
}

int sdpa_describe_plan(const sdpa_desc_t* d, char* buf, size_t len) {
  if (!buf || len == 0) return set_error(SDPA_E_NULL, "buf is NULL or empty");
  sdpa::Plan p;
  std::string err;
  const int rc = sdpa::make_plan(d, &p, &err);
  if (rc != SDPA_OK) return set_error(rc, err);
  const std::string s = sdpa::describe(d, p);
  const size_t n = s.size() < len - 1 ? s.size() : len - 1;
  std::memcpy(buf, s.data(), n);
  buf[n] = '\0';
  return ok();
}

}  // extern "C"

namespace {

// The forward call behind sdpa_forward_varlen and sdpa_forward_noalloc, on a
// plan already made: argument checks, then the attention kernel and, for a
// split plan, the combine.
int forward_planned(const sdpa_desc_t* d, const sdpa::Plan& p, const void* q, const void* k, const void* v,
                    const void* mask, const int32_t* q_lens, const int32_t* kv_lens, void* o, float* lse,
                    void* workspace, size_t workspace_bytes, sdpa_stream_t stream) {
  hipEvent_t ev_start = g_prof_start, ev_stop = g_prof_stop;  // consumed by this call
  g_prof_start = g_prof_stop = nullptr;
  if (!q || !k || !v || !o) return set_error(SDPA_E_NULL, "q, k, v and o must be non-NULL device pointers");
  std::string err;
  int rc = SDPA_OK;
  if ((p.mask_array != sdpa::MA_NONE) != (mask != nullptr))
    return set_error(SDPA_E_NULL, p.mask_array != sdpa::MA_NONE
                                      ? "desc names a mask array but mask is NULL"
                                      : "mask is given but desc->mask_array is SDPA_MASK_ARRAY_NONE");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (mask && !aligned16(mask)))
    return set_error(SDPA_E_STRIDE, "q, k, v, o and mask must be 16-byte aligned");
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u))
    return set_error(SDPA_E_STRIDE, "lse must be 4-byte aligned");
  if ((q_lens && (reinterpret_cast<uintptr_t>(q_lens) & 3u)) ||
      (kv_lens && (reinterpret_cast<uintptr_t>(kv_lens) & 3u)))
    return set_error(SDPA_E_STRIDE, "q_lens and kv_lens must be 4-byte aligned");
  if (p.workspace > 0) {
    if (!workspace || workspace_bytes < p.workspace)
      return set_error(SDPA_E_WORKSPACE, "the plan needs a workspace of " + std::to_string(p.workspace) +
                                             " bytes (got " + std::to_string(workspace_bytes) + ")");
    if (reinterpret_cast<uintptr_t>(workspace) & 255u)
      return set_error(SDPA_E_WORKSPACE, "workspace must be 256-byte aligned");
  }
  rc = check_device(&err);
  if (rc != SDPA_OK) return set_error(rc, err);

  sdpa::AttnArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.mask_arr = mask;
  a.q_lens = q_lens;
  a.kv_lens = kv_lens;
  for (int j = 0; j < 3; ++j) {
    a.qs[j] = d->q_stride[j];
    a.ks[j] = d->k_stride[j];
    a.vs[j] = d->v_stride[j];
    a.os[j] = d->o_stride[j];
    a.ms[j] = mask ? d->mask_stride[j] : 0;
  }
  a.B = (int)d->batch;
  a.Hq = (int)d->heads_q;
  a.Hkv = (int)d->heads_kv;
  a.Lq = (int)d->len_q;
  a.Lk = (int)d->len_k;
  a.dqk = (int)d->dim_qk;
  a.dv = (int)d->dim_v;
  a.G = (int)(d->heads_q / d->heads_kv);
  a.R = a.G * a.Lq;
  a.mask = p.mask;
  a.window = p.window;
  a.c = (float)((double)d->scale * 1.4426950408889634074);  // log2(e)
  a.scale = d->scale;
  a.splits = p.splits;
  a.row_tiles = p.row_tiles;
  // Masked prefill visits its longest row tiles first: tile-major across
  // heads when nothing else orders the grid, else within each head.
  a.heavy_first = p.mask != sdpa::MASK_NONE && p.row_tiles > 1 ? (p.splits == 1 && p.xcd_group == 0 ? 2 : 1) : 0;
  a.xcd_group = p.xcd_group;
  // Per-batch key lengths on a split plan: deal the workgroups by the
  // entries' key blocks (a window's tiles see about W keys whatever the
  // length, so it keeps the even deal).
  a.kv_balance = (kv_lens && p.splits > 1 && p.mask != sdpa::MASK_WINDOW) ? p.fam.nwk * p.fam.bkw : 0;
  if (p.splits > 1) {
    const size_t rows_total = (size_t)d->batch * d->heads_kv * a.R * p.splits;
    const size_t o_bytes = (rows_total * (size_t)d->dim_v * 4 + 255) / 256 * 256;
    a.ws_o = static_cast<float*>(workspace);
    a.ws_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + o_bytes);
  }

  using L = int (*)(const sdpa::Plan&, const sdpa::AttnArgs&, void*, std::string*);
  // [with a mask array][dtype][kind]
  static const L table[2][3][sdpa::kNumKinds] = {
      {{sdpa::launch_attn_f32_prefill, sdpa::launch_attn_f32_short, sdpa::launch_attn_f32_decode,
        sdpa::launch_attn_f32_wide},
       {sdpa::launch_attn_f16_prefill, sdpa::launch_attn_f16_short, sdpa::launch_attn_f16_decode,
        sdpa::launch_attn_f16_wide},
       {sdpa::launch_attn_bf16_prefill, sdpa::launch_attn_bf16_short, sdpa::launch_attn_bf16_decode,
        sdpa::launch_attn_bf16_wide}},
      {{sdpa::launch_attn_f32_prefill_mask, sdpa::launch_attn_f32_short_mask, sdpa::launch_attn_f32_decode_mask,
        sdpa::launch_attn_f32_wide_mask},
       {sdpa::launch_attn_f16_prefill_mask, sdpa::launch_attn_f16_short_mask, sdpa::launch_attn_f16_decode_mask,
        sdpa::launch_attn_f16_wide_mask},
       {sdpa::launch_attn_bf16_prefill_mask, sdpa::launch_attn_bf16_short_mask,
        sdpa::launch_attn_bf16_decode_mask, sdpa::launch_attn_bf16_wide_mask}},
  };
  const L launch = table[p.mask_array != sdpa::MA_NONE][p.dtype][p.kind];
  if (ev_start && hipEventRecord(ev_start, (hipStream_t)stream) != hipSuccess)
    return set_error(SDPA_E_HIP, "hipEventRecord(start) failed");
  rc = launch(p, a, stream, &err);
  if (rc != SDPA_OK) return set_error(rc, err);
  if (p.splits > 1) {
    sdpa::CombineArgs c;
    c.ws_o = a.ws_o;
    c.ws_ml = a.ws_ml;
    c.o = o;
    c.lse = lse;
    c.q_lens = q_lens;
    c.kv_lens = kv_lens;
    c.kv_balance = a.kv_balance;
    c.xcd_rows = p.combine_xcd ? 1 : 0;
    c.Lk = a.Lk;
    for (int j = 0; j < 3; ++j) c.os[j] = d->o_stride[j];
    c.B = a.B;
    c.Hq = a.Hq;
    c.Hkv = a.Hkv;
    c.Lq = a.Lq;
    c.dv = a.dv;
    c.G = a.G;
    c.R = a.R;
    c.splits = p.splits;
    rc = sdpa::launch_combine(p, c, stream, &err);
    if (rc != SDPA_OK) return set_error(rc, err);
  }
  if (ev_stop && hipEventRecord(ev_stop, (hipStream_t)stream) != hipSuccess)
    return set_error(SDPA_E_HIP, "hipEventRecord(stop) failed");
  return ok();
}

// Scratch of sdpa_forward_noalloc: the split partials (O, m, l) live here
// instead of in a caller workspace.  Each device that loads the library holds
// its own copy until the process ends.  Host code never passes the name
// `scratch` to a kernel (on the host it is only a stand-in for the symbol):
// it passes the device address hipGetSymbolAddress returns, taken once per
// device with that device current.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

int scratch_ptr(void** out, std::string* err) {
  static std::mutex mu;
  static void* ptrs[64] = {nullptr};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    *err = "no HIP device is available";
    return SDPA_E_DEVICE;
  }
  if (dev >= 64) {
    *err = "sdpa_forward_noalloc supports device ordinals below 64";
    return SDPA_E_DEVICE;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      *err = std::string("hipGetSymbolAddress(scratch) failed: ") + hipGetErrorString(e);
      return SDPA_E_HIP;
    }
    ptrs[dev] = ptr;
  }
  *out = ptrs[dev];
  return SDPA_OK;
}

}  // namespace

extern "C" {

int sdpa_forward_varlen(const sdpa_desc_t* d, const void* q, const void* k, const void* v, const void* mask,
                        const int32_t* q_lens, const int32_t* kv_lens, void* o, float* lse, void* workspace,
                        size_t workspace_bytes, sdpa_stream_t stream) {
  sdpa::Plan p;
  std::string err;
  const int rc = sdpa::make_plan(d, &p, &err);
  if (rc != SDPA_OK) {
    g_prof_start = g_prof_stop = nullptr;
    return set_error(rc, err);
  }
  return forward_planned(d, p, q, k, v, mask, q_lens, kv_lens, o, lse, workspace, workspace_bytes, stream);
}

int sdpa_forward_noalloc(const sdpa_desc_t* d, const void* q, const void* k, const void* v, const void* mask,
                         const int32_t* q_lens, const int32_t* kv_lens, void* o, float* lse,
                         sdpa_stream_t stream) {
  sdpa::Plan p;
  std::string err;
  int rc = sdpa::make_plan(d, &p, &err);
  if (rc != SDPA_OK) {
    g_prof_start = g_prof_stop = nullptr;
    return set_error(rc, err);
  }
  if (p.workspace > kScratchBytes) {
    g_prof_start = g_prof_stop = nullptr;
    return set_error(SDPA_E_WORKSPACE, "sdpa_forward_noalloc: the plan needs " + std::to_string(p.workspace) +
                                           " bytes of split scratch, above its fixed " +
                                           std::to_string(kScratchBytes) +
                                           " bytes (force fewer splits with num_splits, or pass a workspace "
                                           "to sdpa_forward_varlen)");
  }
  void* ws = nullptr;
  if (p.workspace > 0) {
    rc = scratch_ptr(&ws, &err);
    if (rc != SDPA_OK) {
      g_prof_start = g_prof_stop = nullptr;
      return set_error(rc, err);
    }
  }
  return forward_planned(d, p, q, k, v, mask, q_lens, kv_lens, o, lse, ws, p.workspace ? kScratchBytes : 0,
                         stream);
}

int sdpa_forward_masked(const sdpa_desc_t* d, const void* q, const void* k, const void* v, const void* mask,
                        void* o, float* lse, void* workspace, size_t workspace_bytes, sdpa_stream_t stream) {
  return sdpa_forward_varlen(d, q, k, v, mask, nullptr, nullptr, o, lse, workspace, workspace_bytes, stream);
}

int sdpa_forward(const sdpa_desc_t* d, const void* q, const void* k, const void* v, void* o, float* lse,
                 void* workspace, size_t workspace_bytes, sdpa_stream_t stream) {
  if (d && d->mask_array != SDPA_MASK_ARRAY_NONE) {
    g_prof_start = g_prof_stop = nullptr;
    return set_error(SDPA_E_MASK, "desc names a mask array: call sdpa_forward_masked with the array");
  }
  return sdpa_forward_varlen(d, q, k, v, nullptr, nullptr, nullptr, o, lse, workspace, workspace_bytes, stream);
}

int sdpa_backward_workspace_bytes(const sdpa_desc_t* d, size_t* bytes) {
  if (!bytes) return set_error(SDPA_E_NULL, "bytes is NULL");
  sdpa::BwdPlan p;
  std::string err;
  const int rc = sdpa::make_bwd_plan(d, &p, &err);
  if (rc != SDPA_OK) return set_error(rc, err);
  *bytes = p.workspace;
  return ok();
}

int sdpa_backward_varlen(const sdpa_desc_t* d, const void* q, const void* k, const void* v, const void* mask,
                         const int32_t* q_lens, const int32_t* kv_lens, const void* o, const void* dout,
                         const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                         sdpa_stream_t stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv)
    return set_error(SDPA_E_NULL, "q, k, v, o, dout, lse, dq, dk and dv must be non-NULL device pointers");
  sdpa::BwdPlan p;
  std::string err;
  int rc = sdpa::make_bwd_plan(d, &p, &err);
  if (rc != SDPA_OK) return set_error(rc, err);
  const bool has_arr = d->mask_array != SDPA_MASK_ARRAY_NONE;
  if (has_arr != (mask != nullptr))
    return set_error(SDPA_E_NULL, has_arr ? "desc names a mask array but mask is NULL"
                                          : "mask is given but desc->mask_array is SDPA_MASK_ARRAY_NONE");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv) || (mask && !aligned16(mask)))
    return set_error(SDPA_E_STRIDE, "q, k, v, o, dout, dq, dk, dv and mask must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(lse) & 3u) return set_error(SDPA_E_STRIDE, "lse must be 4-byte aligned");
  if (!workspace || workspace_bytes < p.workspace)
    return set_error(SDPA_E_WORKSPACE, "the backward pass needs a workspace of " + std::to_string(p.workspace) +
                                           " bytes (got " + std::to_string(workspace_bytes) + ")");
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return set_error(SDPA_E_WORKSPACE, "workspace must be 256-byte aligned");
  rc = check_device(&err);
  if (rc != SDPA_OK) return set_error(rc, err);

  sdpa::BwdArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.grad_q = dq;
  a.grad_k = dk;
  a.grad_v = dv;
  a.q_lens = q_lens;
  a.kv_lens = kv_lens;
  a.mask_arr = mask;
  a.ma = d->mask_array == SDPA_MASK_ARRAY_BOOL ? sdpa::MA_BOOL
                                                : (d->mask_array == SDPA_MASK_ARRAY_ADD ? sdpa::MA_ADD : sdpa::MA_NONE);
  a.mes = sdpa::mask_elem_bytes(a.ma, 2);
  for (int j = 0; j < 3; ++j) {
    a.ms[j] = mask ? d->mask_stride[j] : 0;
    a.qs[j] = d->q_stride[j];
    a.ks[j] = d->k_stride[j];
    a.vs[j] = d->v_stride[j];
    a.os[j] = d->o_stride[j];
  }
  a.B = (int)d->batch;
  a.Hq = (int)d->heads_q;
  a.Hkv = (int)d->heads_kv;
  a.Lq = (int)d->len_q;
  a.Lk = (int)d->len_k;
  a.dqk = (int)d->dim_qk;
  a.dv = (int)d->dim_v;
  a.G = (int)(d->heads_q / d->heads_kv);
  a.R = a.G * a.Lq;
  a.Rp = p.Rp;
  a.off = a.Lk - a.Lq;
  a.mask = p.mask;
  a.window = p.window;
  a.c = (float)((double)d->scale * 1.4426950408889634074);
  a.scale = d->scale;
  const size_t zrp = (size_t)d->batch * d->heads_kv * p.Rp;
  a.ws_lse2 = static_cast<float*>(workspace);
  a.ws_d = a.ws_lse2 + zrp;
  a.ws_qi = reinterpret_cast<int*>(a.ws_d + zrp);
  a.kv_parts = p.kv_parts;
  a.ws_part = p.kv_parts > 1 ? reinterpret_cast<float*>(static_cast<char*>(workspace) + p.part_offset) : nullptr;
  rc = sdpa::launch_backward(p, a, stream, &err);
  if (rc != SDPA_OK) return set_error(rc, err);
  return ok();
}

int sdpa_backward(const sdpa_desc_t* d, const void* q, const void* k, const void* v, const void* o,
                  const void* dout, const float* lse, void* dq, void* dk, void* dv, void* workspace,
                  size_t workspace_bytes, sdpa_stream_t stream) {
  if (d && d->mask_array != SDPA_MASK_ARRAY_NONE)
    return set_error(SDPA_E_MASK, "desc names a mask array: call sdpa_backward_varlen with the array");
  return sdpa_backward_varlen(d, q, k, v, nullptr, nullptr, nullptr, o, dout, lse, dq, dk, dv, workspace,
                              workspace_bytes, stream);
}

int sdpa_set_profile_events(void* start, void* stop) {
  if ((start == nullptr) != (stop == nullptr))
    return set_error(SDPA_E_NULL, "start and stop must both be set or both be NULL");
  g_prof_start = static_cast<hipEvent_t>(start);
  g_prof_stop = static_cast<hipEvent_t>(stop);
  return ok();
}

const char* sdpa_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
