/*
 * sdpa.h - C ABI of the MI355X (gfx950) fused scaled-dot-product attention
 * forward library (libsdpa_fwd.so).
 *
 * Operation (mlx PR #4185 "Add force_fused option to
 * scaled_dot_product_attention", API and Background; mlx PR #3552
 * "feat(fast): add sliding-window SDPA kernel path", Summary and Public API):
 *
 *     O[b,h] = softmax(scale * Q[b,h] K[b,kv]^T + mask) V[b,kv],
 *     kv = h / (Hq / Hkv)                      (grouped-query attention)
 *
 * computed tile by tile with an online softmax, so the Lq x Lk score matrix
 * never exists in memory.  Masks:
 *   SDPA_MASK_NONE    every key is visible;
 *   SDPA_MASK_CAUSAL  query row i sits at key position p = i + Lk - Lq (rows
 *                     aligned to the last Lq keys) and sees keys j <= p;
 *   SDPA_MASK_WINDOW  causal and additionally p - window < j, i.e. the last
 *                     `window` key positions up to and including p.
 * An explicit mask array (mlx PR #3552, Public API: the `mask_arr` argument
 * beside the mask mode; its boolean and floating-point kinds are the two
 * mask specialisations that mlx PR #4185's validation tells apart) may be
 * given on top of the mask mode, through sdpa_forward_masked():
 *   SDPA_MASK_ARRAY_BOOL  one byte per element: 1 keeps the key, 0 removes
 *                         it (a C/C++ bool; no other byte values);
 *   SDPA_MASK_ARRAY_ADD   the q/k/v element type, added to the scaled score
 *                         (natural-log units; -inf removes the key; +inf and
 *                         NaN are not allowed).
 * A key counts only if the mask mode keeps it and the array does too.  A row
 * that keeps no key (possible only through an array) gets o = 0 and
 * lse = -inf.
 * The optional log-sum-exp output is lse[b,h,i] = ln sum_j exp(s_ij) over the
 * kept keys, s_ij = scale*q_i.k_j (+ the additive mask), natural log, float32.
 *
 * Tensors (element strides; the head-dim stride is always 1):
 *   q [B, Hq,  Lq, Dqk]   k [B, Hkv, Lk, Dqk]   v [B, Hkv, Lk, Dv]
 *   o [B, Hq,  Lq, Dv]    lse [B, Hq, Lq] contiguous float32 (optional)
 *   mask [B, Hq, Lq, Lk]  element strides mask_stride[] for (batch, query
 *                         head, query); 0 broadcasts a dim; key stride 1
 * Every row stride is a multiple of 16 bytes; the k and v position strides
 * (k_stride[2], v_stride[2]) are at most 16 MiB.
 * q, k, v and o share one element type (float32, float16 or bfloat16).
 * Accumulation is float32; o is rounded once, to nearest even.
 *
 * Ownership: the caller owns every buffer.  The library keeps no pointer
 * after a call returns and allocates no device memory: a split plan needs a
 * caller workspace of sdpa_workspace_bytes() bytes (0 for an unsplit plan).
 * All pointers are device pointers of the current HIP device.
 *
 * Errors: every entry point returns SDPA_OK (0) or a negative sdpa_status_t.
 * Validation runs on the host before anything is launched; on any error
 * nothing is launched and o / lse are left untouched.  sdpa_last_error()
 * returns a thread-local message naming the violated constraint.  Calls are
 * asynchronous on `stream` and reentrant.
 */
#ifndef SDPA_FWD_H
#define SDPA_FWD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SDPA_F32 = 0,
  SDPA_F16 = 1,
  SDPA_BF16 = 2
} sdpa_dtype_t;

typedef enum {
  SDPA_MASK_NONE = 0,
  SDPA_MASK_CAUSAL = 1,
  SDPA_MASK_WINDOW = 2
} sdpa_mask_t;

typedef enum {
  SDPA_MASK_ARRAY_NONE = 0,
  SDPA_MASK_ARRAY_BOOL = 1,  /* bool bytes: 1 = keep, 0 = remove */
  SDPA_MASK_ARRAY_ADD = 2    /* q's element type, added to the scaled score */
} sdpa_mask_array_t;

typedef enum {
  SDPA_OK = 0,
  SDPA_E_NULL = -1,      /* a required pointer is NULL */
  SDPA_E_SHAPE = -2,     /* a size < 1, Hq not a multiple of Hkv, size overflow */
  SDPA_E_HEAD_DIM = -3,  /* head dim not a multiple of 8, above 512, or above 128 in float32 */
  SDPA_E_DTYPE = -4,     /* unknown element type */
  SDPA_E_MASK = -5,      /* unknown mask or mask array kind, causal/window with Lq > Lk, bad window */
  SDPA_E_STRIDE = -6,    /* stride or pointer alignment (16-byte rows) violated */
  SDPA_E_WORKSPACE = -7, /* workspace missing or smaller than required */
  SDPA_E_SCALE = -8,     /* scale is not finite */
  SDPA_E_DEVICE = -9,    /* no usable gfx950 device */
  SDPA_E_HIP = -10,      /* a HIP runtime call or kernel launch failed */
  SDPA_E_PLAN = -11      /* a plan override cannot be honoured */
} sdpa_status_t;

/* A HIP stream (hipStream_t); NULL selects the null stream. */
typedef void* sdpa_stream_t;

typedef struct {
  int64_t batch, heads_q, heads_kv, len_q, len_k, dim_qk, dim_v;
  /* element strides of the (batch, head, position) dims of each tensor */
  int64_t q_stride[3], k_stride[3], v_stride[3], o_stride[3];
  int32_t dtype;   /* sdpa_dtype_t */
  int32_t mask;    /* sdpa_mask_t */
  int32_t window;  /* >= 1 iff mask == SDPA_MASK_WINDOW, else 0 */
  float scale;     /* finite; any sign; 0 allowed */
  /* Plan overrides (0 = let the planner choose).  They select among the same
   * kernels, never a different code path.  num_splits forces the number of
   * key splits (>= 1); for the backward it forces the number of row parts
   * each dK/dV key tile is cut into (1..64).  row_tile forces the query rows
   * per workgroup (32, 64 or 128). */
  int32_t num_splits;
  int32_t row_tile;
  /* Explicit mask array (sdpa_forward_masked only).  mask_array is a
   * sdpa_mask_array_t; mask_stride[] are element strides of its (batch, query
   * head, query) dims, each >= 0 and a multiple of 16 bytes (0 broadcasts
   * that dim).  The array is read in 16-byte pieces, so every row's storage
   * must extend to Lk rounded up to a multiple of 16 bytes (pad the key
   * dimension: the padding is never used). */
  int32_t mask_array;
  int64_t mask_stride[3];
} sdpa_desc_t;

/* Fills *desc with contiguous [B,H,L,D] strides for the given sizes, no mask,
 * scale = 1/sqrt(dim_qk), no overrides.  Returns SDPA_OK or SDPA_E_NULL.
 * The descriptor carries the operation's arguments (mlx PR #4185, API: q, k,
 * v, scale and the mask; mlx PR #3552, Public API: the mask mode and
 * window_size); 1/sqrt(D) is the scale the workloads on the pages use. */
int sdpa_desc_init(sdpa_desc_t* desc, int64_t batch, int64_t heads_q, int64_t heads_kv,
                   int64_t len_q, int64_t len_k, int64_t dim_qk, int64_t dim_v,
                   int32_t dtype);

/* Workspace bytes the plan for *desc needs (0 when the plan does not split
 * the key range).  Validates *desc; host only, launches nothing.  A split
 * plan keeps one partial output with its running max and sum per key split
 * until the log-sum-exp merge combines them (mlx issue #3826, second and
 * third comments: the key range is split and the splits are merged by
 * log-sum-exp); this is their size: [B*Hkv][G*Lq][splits] x (Dv + 2) float32,
 * 256-byte aligned. */
int sdpa_workspace_bytes(const sdpa_desc_t* desc, size_t* bytes);

/* Forward pass (mlx PR #4185, API: the fused forward, which always runs a
 * fused kernel and raises with the violated constraint when none covers the
 * shape; mlx PR #3552, Public API and Implementation: the mask mode, the
 * window and the bottom-right query alignment).  q, k, v, o: device
 * pointers, 16-byte aligned, laid out as described above.  lse: NULL or a contiguous [B,Hq,Lq] float32 buffer.
 * workspace: at least sdpa_workspace_bytes() bytes (may be NULL when that is
 * 0).  Enqueues one kernel (unsplit) or a split kernel plus a combine kernel
 * on `stream` and returns without synchronising. */
int sdpa_forward(const sdpa_desc_t* desc, const void* q, const void* k, const void* v,
                 void* o, float* lse, void* workspace, size_t workspace_bytes,
                 sdpa_stream_t stream);

/* Forward pass with an explicit mask array (see above): as sdpa_forward,
 * plus `mask`, a 16-byte aligned device pointer to the array of kind
 * desc->mask_array, laid out by desc->mask_stride.  mask must be NULL exactly
 * when desc->mask_array is SDPA_MASK_ARRAY_NONE (then this is sdpa_forward).
 * sdpa_forward itself rejects a desc that names a mask array. */
int sdpa_forward_masked(const sdpa_desc_t* desc, const void* q, const void* k, const void* v,
                        const void* mask, void* o, float* lse, void* workspace,
                        size_t workspace_bytes, sdpa_stream_t stream);

/* Forward pass with per-batch lengths: as sdpa_forward_masked (mask may be
 * NULL, see there), plus two optional device arrays of desc->batch int32
 * lengths (4-byte aligned, NULL = the full length for every entry):
 *   q_lens[b]  in [0, Lq]  queries of entry b (rows i < q_lens[b]);
 *   kv_lens[b] in [0, Lk]  keys of entry b (keys j < kv_lens[b]).
 * Entry b's query i sits at key position i + kv_lens[b] - q_lens[b]: the
 * K-relative coordinates of mlx PR #3552 "feat(fast): add sliding-window SDPA
 * kernel path" (Implementation) applied to the valid part, which covers
 * varlen decode and a chunk of queries appended to a cache that holds its own
 * keys first (kv_lens = cached + chunk).  Keys j >= kv_lens[b] are never
 * read.  Rows i >= q_lens[b] of o and lse are not written.  A row with no
 * visible key (kv_lens[b] = 0, or a causal row placed before key 0 when
 * q_lens[b] > kv_lens[b]) gets o = 0 and lse = -inf.  The arrays are read on
 * the device only; values outside the stated ranges are clamped into them.
 * The plan (splits, tiles, workspace) follows desc's padded Lq and Lk. */
int sdpa_forward_varlen(const sdpa_desc_t* desc, const void* q, const void* k, const void* v,
                        const void* mask, const int32_t* q_lens, const int32_t* kv_lens, void* o,
                        float* lse, void* workspace, size_t workspace_bytes, sdpa_stream_t stream);

/* Forward pass that allocates nothing, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments and results as
 * sdpa_forward_varlen without the workspace: a split plan keeps its partial
 * outputs in a fixed scratch array of 64 MiB that the library holds on each
 * device it runs on until the process ends.  A plan whose workspace
 * (sdpa_workspace_bytes) exceeds 64 MiB is rejected with SDPA_E_WORKSPACE
 * before anything is launched (force fewer splits with desc->num_splits, or
 * pass a workspace to sdpa_forward_varlen).  No part of the scratch needs to
 * start at zero: every partial a call's combine reads is written earlier in
 * the same call.  All calls on one device share its scratch and each leaves
 * its partials there: calls on one stream are ordered, but calls that
 * overlap on one device (different streams or threads) race and must not be
 * issued.  The call makes no hipMalloc or hipFree. */
int sdpa_forward_noalloc(const sdpa_desc_t* desc, const void* q, const void* k, const void* v,
                         const void* mask, const int32_t* q_lens, const int32_t* kv_lens, void* o,
                         float* lse, sdpa_stream_t stream);

/* Backward pass (mlx PR #4185, Background and API: training needs the
 * log-sum-exp; mlx PR #3552, Outstanding: the VJP).  Given the forward's
 * inputs, its output o and log-sum-exp lse (contiguous float32 [B,Hq,Lq], as
 * sdpa_forward writes it) and the upstream gradient dout, writes
 *   dq = scale dS K,  dk = scale dS^T Q,  dv = P^T dout,
 *   P = softmax(scale Q K^T + mask),  dS = P (dout V^T - rowsum(dout o)),
 * with grouped-query sums over each KV head's query heads.  dout uses
 * desc's o strides, dq the q strides, dk / dv the k / v strides; all in the
 * input type (float16 or bfloat16), head dims up to 128, the causal and
 * window modes (a mask array goes through sdpa_backward_varlen).
 * Deterministic (no atomics).  Needs a
 * workspace of sdpa_backward_workspace_bytes() bytes (256-byte aligned):
 * per-row terms, plus float32 partial dK/dV when the plan cuts the dK/dV key
 * tiles into row parts (grouped queries that leave too few tiles to fill the
 * chip or balance a causal mask).  Enqueues three kernels, four with row
 * parts: the prep and dK/dV kernels on `stream`, the dQ kernel on a stream
 * the library keeps per device (made on the first backward call on that
 * device outside a graph capture), forked from `stream` after the prep and
 * joined back into it before the call returns, so work enqueued on `stream`
 * afterwards sees all three gradients.  `stream` must belong to the current
 * device.  Concurrent calls serialize their enqueue on a lock; the dQ
 * kernels of calls on different streams of one device run in turn. */
int sdpa_backward_workspace_bytes(const sdpa_desc_t* desc, size_t* bytes);
int sdpa_backward(const sdpa_desc_t* desc, const void* q, const void* k, const void* v, const void* o,
                  const void* dout, const float* lse, void* dq, void* dk, void* dv, void* workspace,
                  size_t workspace_bytes, sdpa_stream_t stream);

/* Backward with an explicit mask array and / or per-batch lengths (the
 * counterpart of sdpa_forward_varlen, same arguments and meaning: `mask` as
 * in sdpa_forward_masked, required iff desc->mask_array is not NONE;
 * q_lens / kv_lens nullable int32 device arrays [B], entry b using its first
 * q_lens[b] queries and kv_lens[b] keys, query i at key position
 * i + kv_lens[b] - q_lens[b]).  The mask array is a constant of the forward:
 * no gradient is produced for it.  Every gradient position past an entry's
 * lengths is written as 0, as is dq of a row left without keys: those
 * outputs depend on no input.  The padded rows and keys are never read (a
 * row or key past the lengths reads the entry's last valid one), so they
 * may hold anything. */
int sdpa_backward_varlen(const sdpa_desc_t* desc, const void* q, const void* k, const void* v, const void* mask,
                         const int32_t* q_lens, const int32_t* kv_lens, const void* o, const void* dout,
                         const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                         sdpa_stream_t stream);

/* Writes a one-line, NUL-terminated description of the plan (kernel family,
 * tile, splits, grid, workspace) into buf.  Host only.  The kernel choice is
 * shown to the caller rather than hidden behind a heuristic (mlx PR #4185,
 * Proposed changes and Background: the caller, not a fixed dispatch
 * threshold, decides, and the follow-up hardening adds capability
 * diagnostics).  Validates as sdpa_forward does;
 * on error buf is left untouched. */
int sdpa_describe_plan(const sdpa_desc_t* desc, char* buf, size_t len);

/* Measurement hook (per-call timing as in mlx issue #3826, report: ten
 * warm-up calls, then forty timed ones): the next
 * forward call on this thread records the two
 * hipEvent_t `start` and `stop` on its stream immediately before the launch
 * of its attention kernel and after its last kernel (the split combine, when
 * the plan splits), then forgets them, so the pair brackets the device time
 * of the whole call.  Passing NULL for both cancels a pending pair.  The
 * events stay owned by the caller. */
int sdpa_set_profile_events(void* start, void* stop);

/* Message of the last failed call on this thread ("" if none): it names the
 * violated constraint, e.g. the unsupported head dim or causal with Lq > Lk
 * (mlx PR #4185, API and Validation: an unsupported shape raises with the
 * specific constraint named).  A successful call clears it. */
const char* sdpa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SDPA_FWD_H */
