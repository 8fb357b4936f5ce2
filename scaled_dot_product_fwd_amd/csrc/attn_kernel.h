// Fused attention forward kernel for gfx950 (CDNA4, wave64, MFMA).
//
// One workgroup owns a tile of packed query rows of one (batch, KV head) and a
// contiguous range of key blocks, and walks that range block by block with an
// online softmax (running row max m and row sum l, rescaled accumulator), so
// the Lq x Lk score matrix never exists (mlx PR #4185 "Add force_fused option
// to scaled_dot_product_attention", Background: tiled K/V keep the transient
// bounded regardless of kL).
//
// Data flow per key block (BK = NWK * BKW keys):
//   HBM/L2 --16-byte loads--> registers --> LDS  K tile   [key][d]   (row padded)
//                                          --> LDS V^T tile [dv][key] (transposed
//                                              on the way in, row padded)
//   S^T = K Q^T   MFMA 32x32 (keys x queries), Q kept in registers
//   mask edge blocks only, online softmax in log2 units (exp2 is native)
//   O^T += V^T P^T MFMA 32x32 (dv x queries), P rounded to the input type
// Working on S^T rather than S puts one query row in each lane (plus its
// partner lane l^32), so the row max / row sum need a single cross-lane step
// and the rescale of O is a per-lane scalar.
//
// Packed rows: row r of a KV head is query head g = r % G of the group and
// query position i = r / G.  This packs the G query heads that share a KV head
// (grouped-query attention) into one tile, so K/V are read once for all of
// them (mlx issue #3826 "2.3-2.8x latency jump from L=8 to L=12 queries",
// third comment: several query rows reuse the K/V already loaded).
//
// Key range of a tile (mlx PR #3552 "feat(fast): add sliding-window SDPA
// kernel path", Implementation): causal limits the last block to the tile's
// last query position (kb_lim); a window raises the first block to the tile's
// first query position minus the window (kb_start), so whole blocks below the
// window are never loaded.  Only blocks that straddle an edge (the diagonal,
// any row's window edge, or the Lk tail) apply a per-element mask; every block
// whose first key lies below the last row's window edge is masked, which is
// exact for unaligned windows too.
//
// Split-K (mlx issue #3826, second and third comments: the block-parallel
// reduction over S): the block range may be cut into `splits` parts handled by
// different workgroups; each writes its unnormalised O with (m, l) and a
// combine kernel merges them by log-sum-exp.
#pragma once

#include <hip/hip_runtime.h>

#include "sdpa_internal.h"

namespace sdpa {
namespace dev {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994530942f;

// ---------------------------------------------------------------------------
// Element types.  `frag` is what one lane feeds one MFMA operand.
//   16-bit types: v_mfma_f32_32x32x16_{bf16,f16}; operand = 8 elements of a
//     row (A: row = lane%32, k = 8*(lane/32)+e; B: col = lane%32, same k).
//   float32:      v_mfma_f32_32x32x2_f32; operand = 1 element (k = lane/32).
// Accumulator (both): lane l, register e holds row 8*(e/4) + 4*(l/32) + e%4,
// column l%32.
// ---------------------------------------------------------------------------
struct BF16 {
  static constexpr int ES = 2;     // bytes per element
  static constexpr int KQK = 16;   // head-dim elements per MFMA
  static constexpr int EPL = 8;    // elements per lane per operand
  static constexpr int KPV = 16;   // keys per PV MFMA
  using frag = u32x4;
  static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ unsigned pack2(float x, float y) {
    __bf16 a = (__bf16)x, b = (__bf16)y;  // round to nearest even
    return (unsigned)__builtin_bit_cast(unsigned short, a) |
           ((unsigned)__builtin_bit_cast(unsigned short, b) << 16);
  }
  static __device__ __forceinline__ unsigned short to_store(float x) {
    return __builtin_bit_cast(unsigned short, (__bf16)x);
  }
};

struct F16 {
  static constexpr int ES = 2;
  static constexpr int KQK = 16;
  static constexpr int EPL = 8;
  static constexpr int KPV = 16;
  using frag = u32x4;
  static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ unsigned pack2(float x, float y) {
    _Float16 a = (_Float16)x, b = (_Float16)y;  // round to nearest even
    return (unsigned)__builtin_bit_cast(unsigned short, a) |
           ((unsigned)__builtin_bit_cast(unsigned short, b) << 16);
  }
  static __device__ __forceinline__ unsigned short to_store(float x) {
    return __builtin_bit_cast(unsigned short, (_Float16)x);
  }
};

struct F32 {
  static constexpr int ES = 4;
  static constexpr int KQK = 2;
  static constexpr int EPL = 1;
  static constexpr int KPV = 2;
  using frag = float;
  static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// Position of key `kk` (0..BK-1) inside a V^T LDS row.  For the 16-bit types
// the 4-key groups are swizzled inside each 16-key step so that the 8 keys a
// lane feeds one PV MFMA (keys 16s + 8i' + 4h + j, i'=0..1, j=0..3, taken from
// accumulator registers 8s..8s+7) sit contiguously at 16s + 8h + 4i' + j.
template <class E>
__device__ __forceinline__ int vt_pos(int kk) {
  if constexpr (E::ES == 2) {
    return (kk & ~12) | ((kk & 4) << 1) | ((kk & 8) >> 1);
  } else {
    return kk;
  }
}

// Static shape of one kernel instance.
template <class E, int DQK, int DV, int NWQ, int NWK, int BKW>
struct Shape {
  static constexpr int NW = NWQ * NWK;
  static constexpr int NT = NW * 64;
  static constexpr int BM = NWQ * 32;          // rows per workgroup
  static constexpr int BK = NWK * BKW;         // keys per block
  static constexpr int NKT = BKW / 32;         // 32-key tiles per wave
  static constexpr int NDT = DV / 32;          // 32-wide dv tiles
  static constexpr int NQS = DQK / E::KQK;     // QK MFMAs per key tile
  static constexpr int CH = 16 / E::ES;        // elements per 16-byte chunk
  static constexpr int KROW = DQK * E::ES + 16;  // K tile row bytes (padded)
  static constexpr int VROW = BK * E::ES + 16;   // V^T tile row bytes (padded)
  static constexpr int KBYTES = BK * KROW;
  static constexpr int VBYTES = DV * VROW;
  static constexpr int BUF = KBYTES + VBYTES;
  // Double-buffer the tiles when that still leaves room for two workgroups.
  static constexpr bool DB = 2 * BUF <= 80 * 1024;
  static constexpr int TILE_BYTES = (DB ? 2 : 1) * BUF;
  // Cross-wave merge scratch (NWK > 1): O[slot][q][DV+4] and (m, l)[slot][q].
  static constexpr int MROW = DV + 4;
  static constexpr int MERGE_BYTES = NWK > 1 ? NWQ * NWK * 32 * MROW * 4 + NWQ * NWK * 32 * 8 : 0;
  static constexpr int LDS = TILE_BYTES > MERGE_BYTES ? TILE_BYTES : MERGE_BYTES;
  // Global -> LDS staging work per thread.
  static constexpr int KCHUNKS = BK * DQK / CH;
  static constexpr int KPT = (KCHUNKS + NT - 1) / NT;
  static constexpr int VUNITS = (BK / 4) * (DV / CH);  // 4 keys x one chunk of dv
  static constexpr int VPT = (VUNITS + NT - 1) / NT;
  static_assert(BKW % 32 == 0, "BKW must be a multiple of 32");
  static_assert(DQK % E::KQK == 0 && DV % 32 == 0, "bad head-dim tile");
  static_assert(DQK % CH == 0 && DV % CH == 0, "bad chunking");
};

__device__ __forceinline__ float wave_max32(float x) {  // combine lanes l and l^32
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float wave_sum32(float x) { return x + __shfl_xor(x, 32); }

template <class E, int DQK, int DV, int NWQ, int NWK, int BKW>
__global__ __launch_bounds__(NWQ * NWK * 64) void attn_fwd_kernel(AttnArgs a) {
  using S = Shape<E, DQK, DV, NWQ, NWK, BKW>;
  using frag = typename E::frag;
  __shared__ __attribute__((aligned(16))) char smem[S::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wq = wave % NWQ;
  const int wk = wave / NWQ;
  const int col = lane & 31;  // query column of this lane in S^T / O^T
  const int hl = lane >> 5;   // lane half

  // ---- workgroup -> (row tile, split, batch * KV head) ----
  int id = blockIdx.x;
  int rt = id % a.row_tiles;
  id /= a.row_tiles;
  const int split = id % a.splits;
  const int z = id / a.splits;
  if (a.heavy_first) rt = a.row_tiles - 1 - rt;
  const int b = z / a.Hkv;
  const int kvh = z % a.Hkv;

  // ---- rows of this lane / wave / workgroup ----
  const int r_wg = rt * S::BM;
  const int r_wave = r_wg + wq * 32;
  const int r = r_wave + col;
  const bool row_ok = r < a.R;
  const int gq = r % a.G;
  const int iq = r / a.G;
  const int pos = iq + a.off;  // absolute key position of this row's query
  const int hq = kvh * a.G + gq;

  const int r_last_wg = min(a.R, r_wg + S::BM) - 1;
  const int pmin_wg = r_wg / a.G + a.off;
  const int pmax_wg = r_last_wg / a.G + a.off;
  const int r_last_wave = min(a.R - 1, r_wave + 31);
  const int pmin_w = min(r_wave, a.R - 1) / a.G + a.off;
  const int pmax_w = r_last_wave / a.G + a.off;

  // ---- key block range of the tile, then of this split ----
  int k_lo = 0, k_hi = a.Lk;
  if (a.mask != MASK_NONE) k_hi = min(a.Lk, pmax_wg + 1);
  if (a.mask == MASK_WINDOW) k_lo = max(0, pmin_wg - a.window + 1);
  const int kb_first = k_lo / S::BK;
  const int kb_end = (k_hi + S::BK - 1) / S::BK;
  const int nb = kb_end - kb_first;
  const int sb0 = kb_first + (int)(((long long)nb * split) / a.splits);
  const int sb1 = kb_first + (int)(((long long)nb * (split + 1)) / a.splits);

  // ---- Q fragments (B operand of S^T = K Q^T), kept in registers ----
  frag qf[S::NQS];
  {
    const char* qrow = (const char*)a.q +
                       ((int64_t)b * a.qs[0] + (int64_t)hq * a.qs[1] + (int64_t)iq * a.qs[2]) * E::ES;
#pragma unroll
    for (int s = 0; s < S::NQS; ++s) {
      const int d = s * E::KQK + hl * E::EPL;
      if constexpr (E::ES == 2) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (row_ok && d < a.dqk) v = *(const u32x4*)(qrow + (int64_t)d * 2);
        qf[s] = v;
      } else {
        float v = 0.f;
        if (row_ok && d < a.dqk) v = *(const float*)(qrow + (int64_t)d * 4);
        qf[s] = v;
      }
    }
  }

  f32x16 oacc[S::NDT];
#pragma unroll
  for (int t = 0; t < S::NDT; ++t) oacc[t] = f32x16{};
  float m_run = kNegInf;  // running max, log2 units
  float l_run = 0.f;      // running sum

  // ---- global -> register staging of one key block ----
  const char* kbase = (const char*)a.k + ((int64_t)b * a.ks[0] + (int64_t)kvh * a.ks[1]) * E::ES;
  const char* vbase = (const char*)a.v + ((int64_t)b * a.vs[0] + (int64_t)kvh * a.vs[1]) * E::ES;
  const int64_t kstr = a.ks[2] * E::ES;
  const int64_t vstr = a.vs[2] * E::ES;
  u32x4 kreg[S::KPT];
  u32x4 vreg[S::VPT][4];

  auto load_block = [&](int blk) {
    const int k0 = blk * S::BK;
#pragma unroll
    for (int i = 0; i < S::KPT; ++i) {
      const int c = tid + i * S::NT;
      const int row = c / (DQK / S::CH);
      const int cc = c % (DQK / S::CH);
      u32x4 v = {0u, 0u, 0u, 0u};
      if (c < S::KCHUNKS && k0 + row < a.Lk && cc * S::CH < a.dqk)
        v = *(const u32x4*)(kbase + (int64_t)(k0 + row) * kstr + cc * 16);
      kreg[i] = v;
    }
#pragma unroll
    for (int i = 0; i < S::VPT; ++i) {
      const int u = tid + i * S::NT;
      const int kg = u % (S::BK / 4);
      const int dg = u / (S::BK / 4);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        u32x4 v = {0u, 0u, 0u, 0u};
        const int key = k0 + kg * 4 + kk;
        if (u < S::VUNITS && key < a.Lk && dg * S::CH < a.dv)
          v = *(const u32x4*)(vbase + (int64_t)key * vstr + dg * 16);
        vreg[i][kk] = v;
      }
    }
  };

  auto store_block = [&](int buf) {
    char* kl = smem + buf * S::BUF;
    char* vl = kl + S::KBYTES;
#pragma unroll
    for (int i = 0; i < S::KPT; ++i) {
      const int c = tid + i * S::NT;
      if (c < S::KCHUNKS) {
        const int row = c / (DQK / S::CH);
        const int cc = c % (DQK / S::CH);
        *(u32x4*)(kl + row * S::KROW + cc * 16) = kreg[i];
      }
    }
#pragma unroll
    for (int i = 0; i < S::VPT; ++i) {
      const int u = tid + i * S::NT;
      if (u < S::VUNITS) {
        const int kg = u % (S::BK / 4);
        const int dg = u / (S::BK / 4);
        const int p0 = vt_pos<E>(kg * 4);
        if constexpr (E::ES == 2) {
          // 4 keys x 8 dv  ->  8 rows of V^T, 4 keys (8 bytes) each.
#pragma unroll
          for (int w = 0; w < 4; ++w) {  // dv pair 2w, 2w+1
            const unsigned x0 = vreg[i][0][w], x1 = vreg[i][1][w];
            const unsigned x2 = vreg[i][2][w], x3 = vreg[i][3][w];
            u32x2 lo, hi;
            lo[0] = (x0 & 0xffffu) | (x1 << 16);
            lo[1] = (x2 & 0xffffu) | (x3 << 16);
            hi[0] = (x0 >> 16) | (x1 & 0xffff0000u);
            hi[1] = (x2 >> 16) | (x3 & 0xffff0000u);
            const int dvr = dg * S::CH + 2 * w;
            *(u32x2*)(vl + dvr * S::VROW + p0 * 2) = lo;
            *(u32x2*)(vl + (dvr + 1) * S::VROW + p0 * 2) = hi;
          }
        } else {
          // 4 keys x 4 dv  ->  4 rows of V^T, 4 keys (16 bytes) each.
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            u32x4 t;
            t[0] = vreg[i][0][e];
            t[1] = vreg[i][1][e];
            t[2] = vreg[i][2][e];
            t[3] = vreg[i][3][e];
            *(u32x4*)(vl + (dg * S::CH + e) * S::VROW + p0 * 4) = t;
          }
        }
      }
    }
  };

  const int nblk = sb1 - sb0;
  if (nblk > 0) {
    load_block(sb0);
    store_block(0);
  }
  __syncthreads();

  for (int j = 0; j < nblk; ++j) {
    const int blk = sb0 + j;
    const int buf = S::DB ? (j & 1) : 0;
    const bool more = j + 1 < nblk;
    if (more) load_block(blk + 1);

    const char* kl = smem + buf * S::BUF;
    const char* vl = kl + S::KBYTES;
    const int kw = blk * S::BK + wk * BKW;  // first key of this wave's slice

    // ---- S^T = K Q^T for this wave's BKW keys ----
    f32x16 sacc[S::NKT];
#pragma unroll
    for (int kt = 0; kt < S::NKT; ++kt) {
      sacc[kt] = f32x16{};
      const char* krow = kl + (wk * BKW + kt * 32 + col) * S::KROW;
#pragma unroll
      for (int s = 0; s < S::NQS; ++s) {
        const int d = s * E::KQK + hl * E::EPL;
        frag af;
        if constexpr (E::ES == 2) af = *(const u32x4*)(krow + d * 2);
        else af = *(const float*)(krow + d * 4);
        sacc[kt] = E::mma(af, qf[s], sacc[kt]);
      }
    }

    // ---- scale into log2 units, mask edge blocks ----
    // Edge test for this wave's rows: diagonal, window edge or Lk tail.
    const bool edge = (kw + BKW > a.Lk) ||
                      (a.mask != MASK_NONE && kw + BKW - 1 > pmin_w) ||
                      (a.mask == MASK_WINDOW && kw < pmax_w - a.window + 1);
    float mx = kNegInf;
#pragma unroll
    for (int kt = 0; kt < S::NKT; ++kt) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float t = sacc[kt][e] * a.c;
        if (edge) {
          const int key = kw + kt * 32 + 8 * (e >> 2) + 4 * hl + (e & 3);
          bool vis = key < a.Lk;
          if (a.mask != MASK_NONE) vis = vis && key <= pos;
          if (a.mask == MASK_WINDOW) vis = vis && key > pos - a.window;
          t = vis ? t : kNegInf;
        }
        sacc[kt][e] = t;
        mx = fmaxf(mx, t);
      }
    }

    // ---- online softmax ----
    mx = wave_max32(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;  // fully masked rows stay at 0
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float rs = 0.f;
#pragma unroll
    for (int kt = 0; kt < S::NKT; ++kt) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = __builtin_amdgcn_exp2f(sacc[kt][e] - m_use);
        sacc[kt][e] = p;
        rs += p;
      }
    }
    rs = wave_sum32(rs);
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int t = 0; t < S::NDT; ++t) oacc[t] *= alpha;

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int kt = 0; kt < S::NKT; ++kt) {
      const int kcol = wk * BKW + kt * 32;  // first key of this tile inside the block
#pragma unroll
      for (int s2 = 0; s2 < 32 / E::KPV; ++s2) {
        frag bf;
        if constexpr (E::ES == 2) {
          u32x4 pk;
#pragma unroll
          for (int w = 0; w < 4; ++w)
            pk[w] = E::pack2(sacc[kt][8 * s2 + 2 * w], sacc[kt][8 * s2 + 2 * w + 1]);
          bf = pk;
        } else {
          bf = sacc[kt][s2];
        }
#pragma unroll
        for (int t = 0; t < S::NDT; ++t) {
          const char* vrow = vl + (t * 32 + col) * S::VROW;
          frag af;
          if constexpr (E::ES == 2) {
            af = *(const u32x4*)(vrow + (kcol + 16 * s2 + 8 * hl) * 2);
          } else {
            const int kk = kcol + 8 * (s2 >> 2) + 4 * hl + (s2 & 3);
            af = *(const float*)(vrow + kk * 4);
          }
          oacc[t] = E::mma(af, bf, oacc[t]);
        }
      }
    }

    if (more) {
      if constexpr (S::DB) {
        store_block(buf ^ 1);
      } else {
        __syncthreads();
        store_block(0);
      }
    }
    __syncthreads();
  }

  // ---- epilogue ----
  const int64_t ws_row = ((int64_t)z * a.R + r) * a.splits + split;

  if constexpr (NWK == 1) {
    if (!row_ok) return;
    if (a.splits == 1) {
      const float inv = 1.0f / l_run;
      char* orow = (char*)a.o + ((int64_t)b * a.os[0] + (int64_t)hq * a.os[1] + (int64_t)iq * a.os[2]) * E::ES;
#pragma unroll
      for (int t = 0; t < S::NDT; ++t) {
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int d = t * 32 + 8 * i4 + 4 * hl;
          if (d < a.dv) {
            if constexpr (E::ES == 2) {
              u32x2 w;
              w[0] = E::pack2(oacc[t][4 * i4 + 0] * inv, oacc[t][4 * i4 + 1] * inv);
              w[1] = E::pack2(oacc[t][4 * i4 + 2] * inv, oacc[t][4 * i4 + 3] * inv);
              *(u32x2*)(orow + d * 2) = w;
            } else {
              float4 w = make_float4(oacc[t][4 * i4 + 0] * inv, oacc[t][4 * i4 + 1] * inv,
                                     oacc[t][4 * i4 + 2] * inv, oacc[t][4 * i4 + 3] * inv);
              *(float4*)(orow + d * 4) = w;
            }
          }
        }
      }
      if (a.lse && hl == 0)
        a.lse[((int64_t)b * a.Hq + hq) * a.Lq + iq] = (m_run + log2f(l_run)) * kLn2;
    } else {
      float* wo = a.ws_o + ws_row * a.dv;
#pragma unroll
      for (int t = 0; t < S::NDT; ++t) {
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int d = t * 32 + 8 * i4 + 4 * hl;
          if (d < a.dv)
            *(float4*)(wo + d) = make_float4(oacc[t][4 * i4 + 0], oacc[t][4 * i4 + 1],
                                             oacc[t][4 * i4 + 2], oacc[t][4 * i4 + 3]);
        }
      }
      if (hl == 0) *(float2*)(a.ws_ml + ws_row * 2) = make_float2(m_run, l_run);
    }
  } else {
    // Merge the NWK key slices of the same rows through LDS.  The tile
    // buffers are free: the loop ended with a barrier.
    float* mo = (float*)smem;                                    // [NWQ*NWK][32][MROW]
    float* mml = (float*)(smem + NWQ * NWK * 32 * S::MROW * 4);  // [NWQ*NWK][32][2]
    {
      const int slot = wq * NWK + wk;
      float* myo = mo + (slot * 32 + col) * S::MROW;
#pragma unroll
      for (int t = 0; t < S::NDT; ++t) {
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int d = t * 32 + 8 * i4 + 4 * hl;
          *(float4*)(myo + d) = make_float4(oacc[t][4 * i4 + 0], oacc[t][4 * i4 + 1],
                                            oacc[t][4 * i4 + 2], oacc[t][4 * i4 + 3]);
        }
      }
      if (hl == 0) {
        mml[(slot * 32 + col) * 2 + 0] = m_run;
        mml[(slot * 32 + col) * 2 + 1] = l_run;
      }
    }
    __syncthreads();
    const int rows_here = min(S::BM, a.R - r_wg);
    for (int e = tid; e < S::BM * DV; e += S::NT) {
      const int q = e / DV;  // row inside the workgroup tile
      const int d = e % DV;
      if (q >= rows_here || d >= a.dv) continue;
      const int qw = q >> 5, qc = q & 31;
      float M = kNegInf;
#pragma unroll
      for (int w = 0; w < NWK; ++w) M = fmaxf(M, mml[((qw * NWK + w) * 32 + qc) * 2]);
      const float Mu = (M == kNegInf) ? 0.f : M;
      float L = 0.f, acc = 0.f;
#pragma unroll
      for (int w = 0; w < NWK; ++w) {
        const int sl = (qw * NWK + w) * 32 + qc;
        const float sc = __builtin_amdgcn_exp2f(mml[sl * 2] - Mu);
        L += sc * mml[sl * 2 + 1];
        acc += sc * mo[sl * S::MROW + d];
      }
      const int rr = r_wg + q;
      const int g2 = rr % a.G, i2 = rr / a.G, h2 = kvh * a.G + g2;
      if (a.splits == 1) {
        const float val = acc / L;
        char* orow = (char*)a.o + ((int64_t)b * a.os[0] + (int64_t)h2 * a.os[1] + (int64_t)i2 * a.os[2]) * E::ES;
        if constexpr (E::ES == 2) *(unsigned short*)(orow + d * 2) = E::to_store(val);
        else *(float*)(orow + d * 4) = val;
        if (d == 0 && a.lse) a.lse[((int64_t)b * a.Hq + h2) * a.Lq + i2] = (Mu + log2f(L)) * kLn2;
      } else {
        const int64_t wr = ((int64_t)z * a.R + rr) * a.splits + split;
        a.ws_o[wr * a.dv + d] = acc;
        if (d == 0) *(float2*)(a.ws_ml + wr * 2) = make_float2(M, L);
      }
    }
  }
}

}  // namespace dev
}  // namespace sdpa
