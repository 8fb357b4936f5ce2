// Internal host/device interface of libsdpa_fwd: kernel arguments, the plan
// the host builds for a call, and the launchers the instantiation units export.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>

#include "../../include/sdpa.h"

namespace sdpa {

// Mask kinds after canonicalisation (see plan.cpp).
enum : int { MASK_NONE = 0, MASK_CAUSAL = 1, MASK_WINDOW = 2 };

// Arguments of the split / unsplit attention kernel.  Passed by value.
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;          // nullable
  float* ws_o;         // split partial outputs [z][r][split][dv] (unnormalised)
  float* ws_ml;        // split partial (m, l) pairs [z][r][split][2], m in log2 units
  const void* mask_arr; // explicit mask array (kernels instantiated for one)
  const int* q_lens;   // nullable [B]: valid queries per batch entry
  const int* kv_lens;  // nullable [B]: valid keys per batch entry
  int64_t qs[3], ks[3], vs[3], os[3];  // element strides of (batch, head, position)
  int64_t ms[3];       // mask array element strides of (batch, query head, query)
  int B, Hq, Hkv, Lq, Lk, dqk, dv, G;
  int R;               // packed rows per KV head = G * Lq; row r -> (g = r % G, i = r / G)
  int mask;            // canonical mask kind
  int window;          // window size when mask == MASK_WINDOW
  float c;             // scale * log2(e): scores live in log2 units on the device
  float scale;         // scale itself (an additive mask is added in natural-log units)
  int splits;          // key splits per row tile (1: normalise in place)
  int row_tiles;       // ceil(R / rows per workgroup)
  int heavy_first;     // causal/window prefill: longest row tiles first (1: within each head, 2: across heads)
  int xcd_group;       // > 0: consecutive work items run in groups of this many on one XCD
  int kv_balance;      // > 0 (split plans with kv_lens): deal each KV head's B * splits
                       // workgroups to the batch entries by their blocks of this many keys
};

// Largest number of split partials one packed row may have (the combine
// holds their maxima in LDS).
constexpr int kMaxSplitsPerRow = 1024;

// Balanced per-batch key lengths: the W = B * splits workgroups of a KV head
// are dealt to the batch entries in proportion to their key blocks (blocks
// of `bk` keys): entry e with nb_e > 0 blocks gets
//   s_e = min(nb_e, 1 + nb_e (W - B) / T, kMaxSplitsPerRow)
// workgroups, the consecutive ones from P_e = s_0 + ... + s_(e-1); an empty
// entry gets none.  T is all entries' blocks, so the s_e add up to at most W
// (the rest of the workgroups have nothing to do).  The attention kernel and
// the combine both use these, so they agree on where each entry's partials
// sit.
#if defined(__HIPCC__)
#define SDPA_HD __host__ __device__
#else
#define SDPA_HD
#endif
SDPA_HD inline int kv_balance_blocks(const int* kv_lens, int e, int Lk, int bk) {
  const int len = kv_lens[e] < 0 ? 0 : (kv_lens[e] > Lk ? Lk : kv_lens[e]);
  return (len + bk - 1) / bk;
}
SDPA_HD inline int kv_balance_total(const int* kv_lens, int B, int Lk, int bk) {
  int T = 0;
  for (int e = 0; e < B; ++e) T += kv_balance_blocks(kv_lens, e, Lk, bk);
  return T;
}
SDPA_HD inline int kv_balance_count(int nb, int W, int B, int T) {
  if (nb <= 0) return 0;
  int s = 1 + (int)((int64_t)nb * (W - B) / T);
  if (s > nb) s = nb;
  if (s > kMaxSplitsPerRow) s = kMaxSplitsPerRow;
  return s;
}
#undef SDPA_HD

// Arguments of the split combine kernel.
struct CombineArgs {
  const float* ws_o;
  const float* ws_ml;
  void* o;
  float* lse;
  const int* q_lens;  // nullable [B]: rows past an entry's queries are skipped
  const int* kv_lens; // nullable [B]: with kv_balance, where each entry's partials sit
  int64_t os[3];
  int B, Hq, Hkv, Lq, Lk, dv, G, R, splits;
  int kv_balance;     // see AttnArgs::kv_balance
  int xcd_rows;       // 1: workgroup w takes KV head row group z with z % 8 == w % 8 (B Hkv % 8 == 0)
};

// Kernel family = how the waves of a workgroup divide the work.
struct Family {
  int nwq;   // waves stacked along query rows (32 rows each)
  int nwk;   // waves splitting each key block between them
  int bkw;   // keys per wave per iteration (multiple of 32)
  int nwd = 1;  // waves splitting the dv tiles of the same rows
};

enum : int { KIND_PREFILL = 0, KIND_SHORT = 1, KIND_DECODE = 2, KIND_WIDE = 3 };
constexpr int kNumKinds = 4;

// Explicit mask array kinds as the kernels see them (0: none).  Bytes per
// mask element: 1 for a boolean array, the element size for an additive one.
enum : int { MA_NONE = 0, MA_BOOL = 1, MA_ADD = 2 };
constexpr int mask_elem_bytes(int ma, int elem_bytes) {
  return ma == MA_NONE ? 0 : (ma == MA_BOOL ? 1 : elem_bytes);
}

// The wave arrangement of each kind, sized so that the two LDS buffers of K
// and V tiles (and of the mask tile, mes bytes per element, when a mask
// array is given) fit: prefill keeps two workgroups per CU (<= 80 KB), decode
// takes the largest key block that fits one workgroup's 160 KB.  Shared by
// the planner and the kernel instantiation units.
// Largest K / V row (position) stride in bytes: a key block spans at most 128
// rows, addressed with 32-bit offsets from its first row.
constexpr int64_t kMaxRowStrideBytes = (int64_t)16 << 20;

constexpr Family family_for(int kind, int elem_bytes, int dqk_pad, int dv_pad, int mes = 0) {
  const int key_bytes = (dqk_pad + dv_pad) * elem_bytes;  // one key of K plus V
  // Head dims above 256 (512): a 32-row wave cannot hold Q and the whole O
  // row in registers, so two waves share each 32 rows and split the dv
  // tiles; 32-key blocks keep the two buffers at 128 KB.  Every query
  // length uses this one arrangement.
  if ((dqk_pad > dv_pad ? dqk_pad : dv_pad) > 256) return Family{2, 1, 32, 2};
  if (kind == KIND_DECODE)
    return (key_bytes + 32 * mes) * 128 * 2 <= 160 * 1024 ? Family{1, 4, 32} : Family{1, 2, 32};
  if (kind == KIND_SHORT) return Family{2, 2, 32};
  // Wide: eight 32-row waves share each 64-key block, so up to 256 packed
  // rows read K/V once (head dims up to 128, two waves per SIMD).
  if (kind == KIND_WIDE)
    return (key_bytes + 256 * mes) * 64 * 2 <= 160 * 1024 ? Family{8, 1, 64} : Family{8, 1, 32};
  // Prefill: 64-key blocks when two workgroups still fit per CU.  Both head
  // dims 192 or more and no mask array: 32-key blocks, which leave room for
  // the software-pipelined loop (two blocks of scores beside Q and O); with
  // an array the plain loop measures faster (it skips removed blocks whole).
  // Otherwise 64-key blocks when the head dims are so large that one
  // workgroup per CU is all the registers allow anyway (then the longer block
  // halves the per-block overheads).
  const int per_key = key_bytes + 128 * mes;  // K, V and a 128-row mask column
  if (per_key * 64 * 2 <= 80 * 1024) return Family{4, 1, 64};
  if (dqk_pad >= 192 && dv_pad >= 192 && mes == 0) return Family{4, 1, 32};
  const int dmax = dqk_pad > dv_pad ? dqk_pad : dv_pad;
  return dmax >= 192 && per_key * 64 * 2 <= 160 * 1024 ? Family{4, 1, 64} : Family{4, 1, 32};
}

// Waves per SIMD each kernel instance is compiled for: two (so one wave's
// softmax overlaps the other's MFMA) where the registers of a 32-row tile fit
// 256 per wave without spilling, else one.
constexpr int wpe_for(int kind, int elem_bytes, int dqk_pad, int dv_pad) {
  const int dmax = dqk_pad > dv_pad ? dqk_pad : dv_pad;
  if (kind == KIND_DECODE) return 1;
  if (kind == KIND_WIDE) return 2;
  if (elem_bytes == 4) return dmax <= 96 ? 2 : 1;
  if (dqk_pad == 192 && dv_pad == 128) return 2;
  return dmax <= (kind == KIND_PREFILL ? 160 : 128) ? 2 : 1;
}

struct Plan {
  int dtype;
  int kind;              // KIND_PREFILL / KIND_SHORT / KIND_DECODE / KIND_WIDE
  int dqk_pad, dv_pad;   // head dims rounded up to the instantiated tile dims
  Family fam;
  int rows_per_wg;       // 32 * nwq
  int row_tiles;
  int splits;
  int mask, window;      // canonical mask
  int mask_array;        // MA_NONE / MA_BOOL / MA_ADD
  int mes;               // bytes per mask array element (0 without one)
  int64_t grid;          // workgroups of the attention kernel
  int xcd_group;         // see AttnArgs::xcd_group
  bool combine_xcd;      // see CombineArgs::xcd_rows
  int64_t combine_grid;  // workgroups of the combine kernel (0 when unsplit)
  size_t workspace;      // bytes
  size_t lds_bytes;      // static LDS of the chosen attention kernel
};

// Validation + planning (plan.cpp).  Returns SDPA_OK or an error status and
// fills *err with the violated constraint.
int make_plan(const sdpa_desc_t* d, Plan* plan, std::string* err);
std::string describe(const sdpa_desc_t* d, const Plan& p);

// Launchers, one per (element type, kernel family) instantiation unit.
// Return SDPA_OK, SDPA_E_HEAD_DIM when no kernel is instantiated for the plan,
// or SDPA_E_HIP with *err set when the launch fails.
#define SDPA_DECLARE_LAUNCH(NAME) \
  int NAME(const Plan& p, const AttnArgs& a, void* stream, std::string* err);
SDPA_DECLARE_LAUNCH(launch_attn_bf16_prefill)
SDPA_DECLARE_LAUNCH(launch_attn_bf16_short)
SDPA_DECLARE_LAUNCH(launch_attn_bf16_decode)
SDPA_DECLARE_LAUNCH(launch_attn_f16_prefill)
SDPA_DECLARE_LAUNCH(launch_attn_f16_short)
SDPA_DECLARE_LAUNCH(launch_attn_f16_decode)
SDPA_DECLARE_LAUNCH(launch_attn_f32_prefill)
SDPA_DECLARE_LAUNCH(launch_attn_f32_short)
SDPA_DECLARE_LAUNCH(launch_attn_f32_decode)
// the same with an explicit mask array (boolean or additive, from the plan)
SDPA_DECLARE_LAUNCH(launch_attn_bf16_prefill_mask)
SDPA_DECLARE_LAUNCH(launch_attn_bf16_short_mask)
SDPA_DECLARE_LAUNCH(launch_attn_bf16_decode_mask)
SDPA_DECLARE_LAUNCH(launch_attn_f16_prefill_mask)
SDPA_DECLARE_LAUNCH(launch_attn_f16_short_mask)
SDPA_DECLARE_LAUNCH(launch_attn_f16_decode_mask)
SDPA_DECLARE_LAUNCH(launch_attn_f32_prefill_mask)
SDPA_DECLARE_LAUNCH(launch_attn_f32_short_mask)
SDPA_DECLARE_LAUNCH(launch_attn_f32_decode_mask)
// 256-row tiles (head dims up to 128), without and with a mask array
SDPA_DECLARE_LAUNCH(launch_attn_bf16_wide)
SDPA_DECLARE_LAUNCH(launch_attn_f16_wide)
SDPA_DECLARE_LAUNCH(launch_attn_f32_wide)
SDPA_DECLARE_LAUNCH(launch_attn_bf16_wide_mask)
SDPA_DECLARE_LAUNCH(launch_attn_f16_wide_mask)
SDPA_DECLARE_LAUNCH(launch_attn_f32_wide_mask)
#undef SDPA_DECLARE_LAUNCH
int launch_combine(const Plan& p, const CombineArgs& a, void* stream, std::string* err);

// ---------------------------------------------------------------------------
// Backward pass (dQ, dK, dV).
// ---------------------------------------------------------------------------
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;   // strides of o
  const float* lse;   // forward log-sum-exp [B, Hq, Lq], natural log
  void* grad_q;       // dQ, strides of q
  void* grad_k;       // dK, strides of k
  void* grad_v;       // dV, strides of v
  float* ws_lse2;     // [B*Hkv][Rp] lse in log2 units per packed row (+inf: row has no gradient)
  float* ws_d;        // [B*Hkv][Rp] D = dO . O per packed row
  int* ws_qi;         // [Rp] query index of packed row r (r / G)
  float* ws_part;     // kv_parts > 1: [kv_parts][B*Hkv][Lk][dqk + dv] float32 partial dK (unscaled), dV
  int kv_parts;       // row parts of each dK/dV key tile (1: the kernel writes dK, dV itself)
  const int* q_lens;  // nullable [B]: valid queries per batch entry
  const int* kv_lens; // nullable [B]: valid keys per batch entry
  const void* mask_arr;  // explicit mask array of the forward (ma != MA_NONE)
  int64_t ms[3];         // its element strides of (batch, query head, query)
  int ma, mes;           // MA_NONE / MA_BOOL / MA_ADD, bytes per element
  int64_t qs[3], ks[3], vs[3], os[3];
  int B, Hq, Hkv, Lq, Lk, dqk, dv, G, R, Rp;
  int off;            // Lk - Lq (an entry with lengths uses its own)
  int mask, window;
  float c;            // scale * log2(e), any sign
  float scale;
};

struct BwdPlan {
  int dtype;
  int d_pad;          // both head dims padded to this (32, 64, 96 or 128)
  int mask, window;   // canonical
  int Rp;             // packed rows rounded up to 32
  int64_t prep_grid, dq_grid, dkdv_grid;
  int kv_parts;       // row parts per dK/dV key tile; > 1 adds the partial sums' kernel
  int64_t sum_grid;   // workgroups of that kernel (0 when kv_parts == 1)
  size_t part_offset; // byte offset of the partial dK/dV in the workspace
  size_t workspace;
};

int make_bwd_plan(const sdpa_desc_t* d, BwdPlan* p, std::string* err);
int launch_backward(const BwdPlan& p, const BwdArgs& a, void* stream, std::string* err);

// LDS bytes of an attention kernel instance (host mirror of the kernel's
// static layout, used by the planner's capacity check).
size_t attn_lds_bytes(int dtype, int dqk_pad, int dv_pad, const Family& f, int mes = 0);

}  // namespace sdpa
