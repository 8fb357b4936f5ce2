// Host-side validation and planning for libsdpa_fwd.  Pure C++: no HIP calls,
// nothing launched, so every error path can be exercised without a GPU.
//
// Validation follows the force-fused contract of mlx PR #4185 "Add
// force_fused option to scaled_dot_product_attention" (API, Validation): a
// shape no fused kernel covers raises with the violated constraint named
// (unsupported head dims such as 512, causal with qL > kL), instead of
// silently falling back.
//
// Planning picks the kernel family from the packed row count R = G * Lq and
// the number of key splits from the occupancy the row tiles alone would give,
// so that short query tiles still spread the key range over the whole chip
// (mlx issue #3826 "2.3-2.8x latency jump from L=8 to L=12 queries": a launch
// of one workgroup per head that streams all keys serially is the cliff).
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <sstream>
#include <string>

#include "sdpa_internal.h"

namespace sdpa {

namespace {

constexpr int kTargetCUs = 256;        // gfx950 compute units (MI355X)
constexpr int64_t kMaxLen = 1 << 30;   // keeps every in-kernel index in int32
constexpr int kMaxSplits = 1024;
constexpr int kMaxDim = 512;    // 16-bit types; float32 stops at 128

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int fail(std::string* err, int code, const std::string& msg) {
  if (err) *err = msg;
  return code;
}

const char* dtype_name(int dt) {
  switch (dt) {
    case SDPA_F32: return "float32";
    case SDPA_F16: return "float16";
    case SDPA_BF16: return "bfloat16";
    default: return "?";
  }
}

const char* mask_name(int m) {
  switch (m) {
    case MASK_NONE: return "none";
    case MASK_CAUSAL: return "causal";
    case MASK_WINDOW: return "window";
    default: return "?";
  }
}

}  // namespace

size_t attn_lds_bytes(int dtype, int dqk_pad, int dv_pad, const Family& f, int mes) {
  // Mirrors Shape<> in attn_kernel.h: two K, two V and (with a mask array)
  // two mask tile buffers, which the cross-wave merge reuses (with a little
  // more for the smallest dims); with the dv split, a 4 KB score-exchange
  // tile per wave after them.
  const int es = dtype == SDPA_F32 ? 4 : 2;
  const size_t tiles = (size_t)2 * f.nwk * f.bkw * ((dqk_pad + dv_pad) * es + 32 * f.nwq * mes) +
                       (f.nwd > 1 ? (size_t)f.nwq * f.nwk * f.nwd * 4096 : 0);
  const size_t slots = (size_t)f.nwq * (f.nwk - 1);
  const size_t merge = (slots * 32 * 8 + 15) / 16 * 16 + slots * 32 * (32 + 4) * 4;
  return std::max(tiles, merge);
}

int make_plan(const sdpa_desc_t* d, Plan* p, std::string* err) {
  if (!d) return fail(err, SDPA_E_NULL, "desc is NULL");
  if (!p) return fail(err, SDPA_E_NULL, "plan is NULL");
  const int64_t B = d->batch, Hq = d->heads_q, Hkv = d->heads_kv, Lq = d->len_q, Lk = d->len_k;
  const int64_t Dqk = d->dim_qk, Dv = d->dim_v;
  if (B < 1 || Hq < 1 || Hkv < 1 || Lq < 1 || Lk < 1 || Dqk < 1 || Dv < 1) {
    std::ostringstream s;
    s << "every size must be >= 1 (got B=" << B << " Hq=" << Hq << " Hkv=" << Hkv << " Lq=" << Lq
      << " Lk=" << Lk << " Dqk=" << Dqk << " Dv=" << Dv << ")";
    return fail(err, SDPA_E_SHAPE, s.str());
  }
  if (Hq % Hkv != 0) {
    std::ostringstream s;
    s << "grouped-query attention needs heads_q to be a multiple of heads_kv (got Hq=" << Hq
      << ", Hkv=" << Hkv << ")";
    return fail(err, SDPA_E_SHAPE, s.str());
  }
  if (Lq > kMaxLen || Lk > kMaxLen || (Hq / Hkv) * Lq > kMaxLen || B * Hkv > kMaxLen) {
    return fail(err, SDPA_E_SHAPE, "sizes exceed the supported range (Lq, Lk, G*Lq and B*Hkv must be <= 2^30)");
  }
  if (d->dtype != SDPA_F32 && d->dtype != SDPA_F16 && d->dtype != SDPA_BF16) {
    return fail(err, SDPA_E_DTYPE, "dtype must be SDPA_F32, SDPA_F16 or SDPA_BF16 (got " +
                                       std::to_string(d->dtype) + ")");
  }
  if (Dqk % 8 || Dv % 8 || Dqk > kMaxDim || Dv > kMaxDim) {
    std::ostringstream s;
    s << "no fused kernel for head dims (Dqk=" << Dqk << ", Dv=" << Dv
      << "): supported head dims are multiples of 8 from 8 to " << kMaxDim;
    return fail(err, SDPA_E_HEAD_DIM, s.str());
  }
  int dqk_pad = (int)ceil_div(Dqk, 32) * 32;
  int dv_pad = (int)ceil_div(Dv, 32) * 32;
  if (dqk_pad == 192 && dv_pad <= 128) {
    dv_pad = 128;  // the asymmetric (192, 128) instance
  } else if (dqk_pad > 256 || dv_pad > 256) {
    dqk_pad = dv_pad = 512;  // the one instance above 256
  } else {
    const int m = dqk_pad > dv_pad ? dqk_pad : dv_pad;
    dqk_pad = dv_pad = m;  // zero padding in-kernel: no host copy
    // The QK product steps 16 deep along the head dim, so a 16-bit Q and K of
    // head dim 72 or 80 pad to 80, not 96 (mlx-rs issue #339, findings: pad
    // 72 to 80 rather than to the next larger kernel); V keeps whole 32-wide
    // dv tiles.  One MFMA in six fewer per key tile, K tiles a sixth smaller.
    if (m == 96 && Dqk <= 80 && d->dtype != SDPA_F32) dqk_pad = 80;
  }
  if (d->dtype == SDPA_F32 && (dqk_pad > 128 || dv_pad > 128)) {
    std::ostringstream s;
    s << "no fused float32 kernel for head dims (Dqk=" << Dqk << ", Dv=" << Dv
      << "): float32 supports head dims up to 128";
    return fail(err, SDPA_E_HEAD_DIM, s.str());
  }
  if (d->mask != SDPA_MASK_NONE && d->mask != SDPA_MASK_CAUSAL && d->mask != SDPA_MASK_WINDOW) {
    return fail(err, SDPA_E_MASK, "mask must be SDPA_MASK_NONE, SDPA_MASK_CAUSAL or SDPA_MASK_WINDOW (got " +
                                      std::to_string(d->mask) + ")");
  }
  if (d->mask != SDPA_MASK_NONE && Lq > Lk) {
    std::ostringstream s;
    s << "causal masking requires Lq <= Lk: queries align to the last Lq keys (got Lq=" << Lq
      << ", Lk=" << Lk << ")";
    return fail(err, SDPA_E_MASK, s.str());
  }
  if (d->mask == SDPA_MASK_WINDOW && d->window < 1) {
    return fail(err, SDPA_E_MASK, "a sliding window needs window >= 1 (got " + std::to_string(d->window) + ")");
  }
  if (d->mask != SDPA_MASK_WINDOW && d->window != 0) {
    return fail(err, SDPA_E_MASK, "window must be 0 unless mask is SDPA_MASK_WINDOW (got " +
                                      std::to_string(d->window) + ")");
  }
  if (!std::isfinite(d->scale)) return fail(err, SDPA_E_SCALE, "scale must be finite");
  const int es = d->dtype == SDPA_F32 ? 4 : 2;
  const int64_t* strides[4] = {d->q_stride, d->k_stride, d->v_stride, d->o_stride};
  const char* names[4] = {"q", "k", "v", "o"};
  for (int t = 0; t < 4; ++t) {
    for (int j = 0; j < 3; ++j) {
      if (strides[t][j] < 0 || (strides[t][j] * es) % 16 != 0) {
        std::ostringstream s;
        s << names[t] << "_stride[" << j << "] = " << strides[t][j]
          << " must be >= 0 and a multiple of 16 bytes (rows are read with 16-byte loads)";
        return fail(err, SDPA_E_STRIDE, s.str());
      }
    }
  }
  // A key block's rows (at most 128) are addressed by 32-bit byte offsets
  // from the block's first row.
  for (int t = 1; t <= 2; ++t) {
    if (strides[t][2] * es > kMaxRowStrideBytes) {
      std::ostringstream s;
      s << names[t] << "_stride[2] = " << strides[t][2] << " elements is more than "
        << (kMaxRowStrideBytes >> 20) << " MiB per row (a key block's rows are addressed with 32-bit offsets)";
      return fail(err, SDPA_E_STRIDE, s.str());
    }
  }
  if (d->mask_array != SDPA_MASK_ARRAY_NONE && d->mask_array != SDPA_MASK_ARRAY_BOOL &&
      d->mask_array != SDPA_MASK_ARRAY_ADD) {
    return fail(err, SDPA_E_MASK, "mask_array must be SDPA_MASK_ARRAY_NONE, _BOOL or _ADD (got " +
                                      std::to_string(d->mask_array) + ")");
  }
  const int ma = d->mask_array == SDPA_MASK_ARRAY_BOOL ? MA_BOOL : (d->mask_array == SDPA_MASK_ARRAY_ADD ? MA_ADD : MA_NONE);
  const int mes = mask_elem_bytes(ma, es);
  if (ma != MA_NONE) {
    for (int j = 0; j < 3; ++j) {
      if (d->mask_stride[j] < 0 || (d->mask_stride[j] * mes) % 16 != 0) {
        std::ostringstream s;
        s << "mask_stride[" << j << "] = " << d->mask_stride[j]
          << " must be >= 0 and a multiple of 16 bytes (mask rows are read in 16-byte pieces; pad the key dim)";
        return fail(err, SDPA_E_STRIDE, s.str());
      }
    }
  }
  if (d->num_splits < 0 || d->num_splits > kMaxSplits) {
    return fail(err, SDPA_E_PLAN, "num_splits must be 0 (auto) or 1.." + std::to_string(kMaxSplits));
  }
  if (d->row_tile != 0 && d->row_tile != 32 && d->row_tile != 64 && d->row_tile != 128 && d->row_tile != 256) {
    return fail(err, SDPA_E_PLAN, "row_tile must be 0 (auto), 32, 64, 128 or 256 (got " +
                                      std::to_string(d->row_tile) + ")");
  }

  // ---- canonical mask ----
  int mask = d->mask, window = d->window;
  if (mask == MASK_WINDOW && window >= Lk) { mask = MASK_CAUSAL; window = 0; }  // window covers every key <= p
  if (mask == MASK_CAUSAL && Lq == 1) mask = MASK_NONE;                        // the single query sees every key

  const int64_t G = Hq / Hkv;
  const int64_t R = G * Lq;
  // Row tile: 32 rows (decode family) up to 32 packed rows and for exactly
  // 64, as two decode tiles (the decode family streams K/V best, and the two
  // tiles of a split share an L2: speculative verify Lq=16, G=4 measures
  // 4-12% faster than one 64-row tile); 64 rows (short family) for the rest
  // up to 64; 128 rows (prefill family) beyond.
  // Head dim 512 has one arrangement (two 32-row groups, each on two waves
  // that split the dv tiles): 64 rows for every query length.
  const bool xl = dqk_pad > 256;
  if (xl && d->row_tile != 0 && d->row_tile != 64) {
    return fail(err, SDPA_E_PLAN, "head dim 512 runs 64-row tiles only (row_tile must be 0 or 64, got " +
                                      std::to_string(d->row_tile) + ")");
  }
  // 256 rows (wide family: eight 32-row waves, K/V read once per 256 rows)
  // for 128 < R <= 256 where its two waves per SIMD fit (head dims up to
  // 128, float32 up to 96): two 128-row tiles would read K/V twice
  // (speculative verify Lq=48, G=4, Lk=32768: 48 -> measured below).
  const bool wide_ok = !xl && std::max(dqk_pad, dv_pad) <= (d->dtype == SDPA_F32 ? 96 : 128);
  if (d->row_tile == 256 && !wide_ok) {
    return fail(err, SDPA_E_PLAN, "row_tile 256 needs head dims up to 128 (float32: 96)");
  }
  int rows = xl ? 64
             : d->row_tile ? d->row_tile
                           : (R <= 32 || R == 64 ? 32 : (R <= 64 ? 64 : (R <= 128 || !wide_ok || R > 256 ? 128 : 256)));
  // A long prefill whose 128-row tiles would fill at most half of the CUs
  // (few heads, about a thousand queries) takes 64-row tiles instead (two
  // waves per SIMD up to head dim 128): every CU then gets a tile.  Measured:
  // H=16, L=1024, D=72 (128 -> 256 workgroups) 20.5 -> 19.1 us; with more
  // tiles than that the 128-row tile stays faster (H=20, L=1500, D=64:
  // 240 -> 480 workgroups, 26.9 -> 28.9 us).  Fewer tiles than a quarter of
  // the CUs split the keys instead (below); mask arrays keep their tiles.
  const int64_t tiles128 = B * Hkv * ceil_div(R, 128);
  if (!d->row_tile && rows == 128 && R > 128 && std::max(dqk_pad, dv_pad) <= 128 && ma == MA_NONE &&
      tiles128 >= kTargetCUs / 4 && tiles128 <= kTargetCUs / 2)
    rows = 64;
  const int64_t row_tiles = ceil_div(R, rows);
  const int64_t base = B * Hkv * row_tiles;
  const int kind = xl ? KIND_PREFILL
                      : rows == 32 ? KIND_DECODE : (rows == 64 ? KIND_SHORT : (rows == 256 ? KIND_WIDE : KIND_PREFILL));
  const Family fam = family_for(kind, es, dqk_pad, dv_pad, mes);
  const int64_t bk = (int64_t)fam.nwk * fam.bkw;

  // Key blocks a row tile visits (the longest tile; every tile for `none`).
  int64_t keys = Lk;
  if (mask == MASK_WINDOW) keys = std::min<int64_t>(Lk, window + rows);  // window plus one tile of rows
  const int64_t nblocks = ceil_div(keys, bk);

  int64_t splits = 1;
  if (d->num_splits > 0) {
    splits = d->num_splits;
  } else {
    // Split the key range when the row tiles alone leave the chip idle: aim
    // for one workgroup per CU.  A second resident workgroup does not raise a
    // CU's throughput for these kernels (measured: their waves stall on
    // their own dependency chains, and two workgroups' waves compete for the
    // same matrix cores and vector units), while every extra split adds partial-result
    // traffic and combine work: speculative verify at Lk = 16384, Lq = 32 runs
    // 39.2 us with 64 splits and 29.3 us with 32.  A full-size prefill tile
    // (128 rows) is only split when very few tiles exist: its partial outputs
    // would cost HBM traffic comparable to the K/V it reads, while an unsplit
    // wave of large tiles already keeps the MFMA units busy.
    // A range of three key blocks or fewer stays whole: its extra blocks cost
    // less than the combine launch that splitting adds (decode at Lk = 256,
    // two 128-key blocks: 12.6 us split, 10.3 us whole).
    const int64_t target = kTargetCUs;
    const bool starved = rows < 128 ? base < target : base < kTargetCUs / 4;
    if (starved && nblocks > 3) splits = std::min<int64_t>(ceil_div(target, base), nblocks);
    splits = std::max<int64_t>(1, std::min<int64_t>(splits, kMaxSplits));
  }
  if (base * splits > 0x7fffffffLL) return fail(err, SDPA_E_SHAPE, "grid too large");
  // The combine launches one workgroup per packed row.
  if (splits > 1 && B * Hkv * R > 0x7fffffffLL) {
    if (d->num_splits > 1)
      return fail(err, SDPA_E_PLAN, "a split plan needs B*Hq*Lq <= 2^31 - 1 (one combine workgroup per row)");
    splits = 1;
  }

  p->dtype = d->dtype;
  p->kind = kind;
  p->dqk_pad = dqk_pad;
  p->dv_pad = dv_pad;
  p->fam = fam;
  p->rows_per_wg = rows;
  p->row_tiles = (int)row_tiles;
  p->splits = (int)splits;
  p->mask = mask;
  p->window = window;
  p->mask_array = ma;
  p->mes = mes;
  p->grid = base * splits;
  // Work items that read the same key blocks run in groups on one XCD, whose
  // L2 then serves the re-reads: the row tiles of one split, and neighbouring
  // row tiles under a sliding window once several rounds of workgroups queue
  // up (a window tile shares most of its keys with its neighbours and none
  // with distant tiles).  Measured: split verify Lq=64 65 -> 52 us, window
  // L=8192 -7%; no gain for causal tiles (which all share the key prefix)
  // nor for a single round of window tiles.
  p->xcd_group = ((splits > 1 && row_tiles > 1) ||
                  (mask == MASK_WINDOW && base * splits >= 4 * (int64_t)kTargetCUs)) ? 8 : 0;
  // Unmasked prefill without a split: every row tile of a KV head reads the
  // whole of its K/V, so the tiles of one head go to one XCD (the largest
  // group size that divides the head's tiles and tiles the grid exactly) and
  // that head's K/V stays in one L2 instead of passing through all eight.
  // Measured, interleaved on one box: H=16, L=4096, D=72 (32 tiles per head)
  // 114-122 -> 112-114 us; H=20, L=1500, D=64 (12 tiles, groups of 6)
  // 27.2-28.2 -> 25.8-27.7 us.
  if (mask == MASK_NONE && ma == MA_NONE && splits == 1 && row_tiles > 1) {
    for (int64_t g = row_tiles; g >= 1; --g) {
      if (row_tiles % g == 0 && base % (8 * g) == 0) {
        p->xcd_group = (int)g;
        break;
      }
    }
  }
  // One row tile per KV head and a multiple of 8 heads: all splits of a head
  // run on one XCD, and the combine takes that head's rows on the same XCD,
  // so the partials it reads were written through its own L2.
  p->combine_xcd = splits > 1 && row_tiles == 1 && (B * Hkv) % 8 == 0;
  if (p->combine_xcd) p->xcd_group = splits;
  p->combine_grid = splits > 1 ? B * Hkv * R : 0;
  p->workspace = 0;
  if (splits > 1) {
    // [partial O][partial (m, l)]
    const size_t rows_total = (size_t)(B * Hkv * R * splits);
    const size_t o_bytes = (rows_total * (size_t)Dv * 4 + 255) / 256 * 256;
    p->workspace = o_bytes + rows_total * 8;
  }
  p->lds_bytes = attn_lds_bytes(d->dtype, dqk_pad, dv_pad, fam, mes);
  return SDPA_OK;
}

int make_bwd_plan(const sdpa_desc_t* d, BwdPlan* p, std::string* err) {
  // Everything the forward checks (shapes, strides, masks, scale) holds here
  // too; the backward adds its own limits.
  Plan fp;
  const int rc = make_plan(d, &fp, err);
  if (rc != SDPA_OK) return rc;
  if (d->dtype == SDPA_F32)
    return fail(err, SDPA_E_DTYPE, "the backward pass runs float16 and bfloat16 only");
  if (d->dim_qk > 128 || d->dim_v > 128) {
    std::ostringstream s;
    s << "no backward kernel for head dims (Dqk=" << d->dim_qk << ", Dv=" << d->dim_v
      << "): the backward pass supports head dims up to 128";
    return fail(err, SDPA_E_HEAD_DIM, s.str());
  }
  const int64_t m = std::max(d->dim_qk, d->dim_v);
  const int64_t G = d->heads_q / d->heads_kv;
  const int64_t R = G * d->len_q;
  const int64_t Z = d->batch * d->heads_kv;
  p->dtype = d->dtype;
  p->d_pad = (int)ceil_div(m, 32) * 32;
  p->mask = fp.mask;
  p->window = fp.window;
  p->Rp = (int)ceil_div(R, 32) * 32;
  p->prep_grid = ceil_div(Z * p->Rp, 16);  // 16 rows per 256-thread workgroup
  p->dq_grid = Z * ceil_div(R, 128);       // 128 packed rows per workgroup
  // dK/dV takes 128 keys per workgroup and walks every packed row that can
  // see them.  Under grouped queries a key tile's rows span all G query
  // heads, so there are G times fewer tiles, each G times longer; under a
  // causal mask their lengths also fall from R rows (the first tile) to one
  // tile's worth (the last), and the longest alone can outlast everything
  // else.  The row range of each tile is then cut into kv_parts parts, each
  // part a workgroup that writes float32 partial dK, dV; a last kernel adds
  // the parts in order (deterministic).  Parts are added, in powers of two,
  // while the tiles are too few to fill the chip or (causal) while the
  // longest tile is longer than the chip's share of the total, and while
  // each part keeps at least 8 blocks of 32 rows.  desc->num_splits > 0
  // forces the count (1..64).
  const int64_t key_tiles = ceil_div(d->len_k, 128);
  const int64_t items = Z * key_tiles;
  int parts = 1;
  if (d->num_splits > 0) {
    if (d->num_splits > 64)
      return fail(err, SDPA_E_PLAN, "num_splits for the backward (row parts of each dK/dV key tile) must be 1..64");
    parts = d->num_splits;
  } else {
    int64_t want = ceil_div(kTargetCUs, items);
    if (fp.mask == MASK_CAUSAL) want = std::max<int64_t>(want, ceil_div(2 * kTargetCUs, Z * (key_tiles + 1)));
    const int64_t nb_max = ceil_div(R, 32);  // 32-row blocks of the longest tile
    while (parts < want && parts < 16 && 2 * parts * 8 <= nb_max) parts *= 2;
  }
  p->kv_parts = parts;
  p->dkdv_grid = items * parts;
  const int64_t dsum = d->dim_qk + d->dim_v;
  p->sum_grid = parts > 1 ? ceil_div(Z * d->len_k * (dsum / 4), 256) : 0;
  if (p->prep_grid > 0x7fffffffLL || p->dq_grid > 0x7fffffffLL || p->dkdv_grid > 0x7fffffffLL ||
      p->sum_grid > 0x7fffffffLL)
    return fail(err, SDPA_E_SHAPE, "grid too large");
  // [lse2][D] per (batch, KV head, packed row), then the query index per
  // row, then (kv_parts > 1) the partial dK, dV
  p->part_offset = ((size_t)(2 * Z * p->Rp + p->Rp) * 4 + 255) / 256 * 256;
  const size_t part_bytes = parts > 1 ? (size_t)parts * Z * d->len_k * dsum * 4 : 0;
  p->workspace = (p->part_offset + part_bytes + 255) / 256 * 256;
  return SDPA_OK;
}

std::string describe(const sdpa_desc_t* d, const Plan& p) {
  std::ostringstream s;
  const char* fam = p.kind == KIND_DECODE  ? "decode"
                    : p.kind == KIND_SHORT ? "short"
                    : p.kind == KIND_WIDE  ? "wide"
                                           : "prefill";
  s << "family=" << fam << " dtype=" << dtype_name(p.dtype) << " dqk=" << d->dim_qk << "->" << p.dqk_pad
    << " dv=" << d->dim_v << "->" << p.dv_pad << " rows_per_wg=" << p.rows_per_wg
    << " waves=" << p.fam.nwq << "x" << p.fam.nwk << (p.fam.nwd > 1 ? "x" + std::to_string(p.fam.nwd) : "")
    << " block_keys=" << p.fam.nwk * p.fam.bkw
    << " row_tiles=" << p.row_tiles << " splits=" << p.splits << " mask=" << mask_name(p.mask);
  if (p.mask == MASK_WINDOW) s << "(" << p.window << ")";
  if (p.mask_array != MA_NONE) s << " mask_array=" << (p.mask_array == MA_BOOL ? "bool" : "add");
  s << " grid=" << p.grid << " xcd_group=" << p.xcd_group << " combine_grid=" << p.combine_grid
    << " combine_xcd=" << (p.combine_xcd ? 1 : 0)
    << " lds=" << p.lds_bytes
    << " workspace=" << p.workspace;
  return s.str();
}

}  // namespace sdpa
