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
//   HBM/L2 --LDS DMA (global_load_lds, 16 B per lane)--> LDS K tile [key][d]
//                                                    --> LDS V tile [key][dv]
//   Both tiles keep the global row-major layout; 16-byte chunks are XOR
//   swizzled per row so the MFMA operand reads below hit distinct banks.  The
//   next block's DMA is in flight while the current block is computed (two
//   LDS buffers), and no register is spent on staging.
//   S^T = K Q^T    MFMA 32x32 (keys x queries), Q kept in registers
//   mask edge blocks only; online softmax in log2 units (exp2 is native)
//   O^T += V^T P^T MFMA 32x32 (dv x queries), P rounded to the input type;
//   the V^T operand comes straight from the row-major V tile through the
//   gfx950 transposing LDS read (ds_read_b64_tr_b16).
// Working on S^T rather than S puts one query row in each lane (plus its
// partner lane l^32), so the row max needs a single cross-lane step and the
// rescale of O is a per-lane scalar.
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
// exact for unaligned windows too.  Inside a block, a wave whose rows see none
// of its keys skips the block's arithmetic.
//
// Split-K (mlx issue #3826, second and third comments: the block-parallel
// reduction over S): the block range may be cut into `splits` parts handled by
// different workgroups; each writes its unnormalised O with (m, l) and a
// combine kernel merges them by log-sum-exp.
//
// Lazy rescaling: the reference max m of a row only moves when a block's max
// exceeds it by more than kRescale (log2 units); otherwise the block is
// accumulated against the old reference, so probabilities stay <= 2^kRescale
// and the O/l rescale (Dv multiplies per row) is skipped for most blocks.  The
// result is the same softmax: O, l and m stay mutually consistent.
#pragma once

#include <hip/hip_runtime.h>

#include "sdpa_internal.h"

namespace sdpa {
namespace dev {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

#define SDPA_LDS __attribute__((address_space(3)))

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kRescale = 8.0f;  // lazy-rescale threshold, log2 units

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

constexpr int low_pow2(int x) { return x & -x; }
constexpr int cmin(int a, int b) { return a < b ? a : b; }
constexpr int cmax(int a, int b) { return a > b ? a : b; }

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
  static constexpr int KCH = DQK * E::ES / 16; // 16-byte chunks per K row
  static constexpr int VCH = DV * E::ES / 16;  // 16-byte chunks per V row
  static constexpr int KROW = DQK * E::ES;
  static constexpr int VROW = DV * E::ES;
  static constexpr int KBYTES = BK * KROW;
  static constexpr int VBYTES = BK * VROW;
  static constexpr int BUF = KBYTES + VBYTES;
  static constexpr int KDMA = KBYTES / 1024;   // 1 KB DMA instructions per tile
  static constexpr int VDMA = VBYTES / 1024;
  // Chunk swizzles.  K: chunk ^ (row % KSW) spreads the 8 rows a 16-byte
  // read serves per cycle over 8 slots.  V: chunk ^ 2*(row % VSW) spreads
  // the 4 rows of a transposing read group over 4 slots of 32 bytes.
  static constexpr int KSW = cmin(8, low_pow2(KCH));
  static constexpr int VSW = cmax(1, cmin(4, low_pow2(VCH) / 2));
  // Double-buffered tiles.
  static constexpr int TILE_BYTES = 2 * BUF;
  // Cross-wave merge scratch (NWK > 1): O[slot][q][DV+4] and (m, l)[slot][q].
  static constexpr int MROW = DV + 4;
  static constexpr int MERGE_BYTES = NWK > 1 ? NWQ * NWK * 32 * MROW * 4 + NWQ * NWK * 32 * 8 : 0;
  static constexpr int LDS = TILE_BYTES > MERGE_BYTES ? TILE_BYTES : MERGE_BYTES;
  static_assert(BKW % 32 == 0, "BKW must be a multiple of 32");
  static_assert(DQK % E::KQK == 0 && DV % 32 == 0, "bad head-dim tile");
  static_assert(KBYTES % 1024 == 0 && VBYTES % 1024 == 0, "tiles must be whole DMA instructions");
  static_assert(LDS <= 160 * 1024, "LDS budget of one workgroup exceeded");
};

__device__ __forceinline__ float wave_max32(float x) {  // combine lanes l and l^32
  return fmaxf(x, __shfl_xor(x, 32));
}

// Wait until every outstanding vector-memory operation of this wave (the
// LDS DMA of the next block, the Q loads) has completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

template <class E, int DQK, int DV, int NWQ, int NWK, int BKW>
__global__ __launch_bounds__(NWQ * NWK * 64) void attn_fwd_kernel(AttnArgs a) {
  using S = Shape<E, DQK, DV, NWQ, NWK, BKW>;
  using frag = typename E::frag;
  __shared__ __attribute__((aligned(1024))) char smem[S::LDS];

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
  const int nblk = sb1 - sb0;

  // ---- LDS DMA of one key block into buffer `buf` ----
  const char* kbase = (const char*)a.k + ((int64_t)b * a.ks[0] + (int64_t)kvh * a.ks[1]) * E::ES;
  const char* vbase = (const char*)a.v + ((int64_t)b * a.vs[0] + (int64_t)kvh * a.vs[1]) * E::ES;
  const int64_t kstr = a.ks[2] * E::ES;
  const int64_t vstr = a.vs[2] * E::ES;
  const int kch_valid = a.dqk * E::ES / 16;  // chunks of real data per row
  const int vch_valid = a.dv * E::ES / 16;

  auto dma_block = [&](int blk, int buf) {
    const int k0 = blk * S::BK;
    char* kl = smem + buf * S::BUF;
    char* vl = kl + S::KBYTES;
    // Every lane fetches one 16-byte chunk per instruction; rows past Lk and
    // chunks past the real head dim re-read valid data (masked or multiplied
    // by zero later), so no access leaves the tensors.
#pragma unroll
    for (int i = wave; i < S::KDMA; i += S::NW) {
      const int slot = i * 64 + lane;
      const int row = slot / S::KCH;
      const int c = (slot % S::KCH) ^ (row & (S::KSW - 1));
      const int grow = min(k0 + row, a.Lk - 1);
      const char* src = kbase + (int64_t)grow * kstr + min(c, kch_valid - 1) * 16;
      __builtin_amdgcn_global_load_lds((const void*)src, (SDPA_LDS void*)(kl + i * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int i = wave; i < S::VDMA; i += S::NW) {
      const int slot = i * 64 + lane;
      const int row = slot / S::VCH;
      const int c = (slot % S::VCH) ^ (2 * (row & (S::VSW - 1)));
      const int grow = min(k0 + row, a.Lk - 1);
      const char* src = vbase + (int64_t)grow * vstr + min(c, vch_valid - 1) * 16;
      __builtin_amdgcn_global_load_lds((const void*)src, (SDPA_LDS void*)(vl + i * 1024), 16, 0, 0);
    }
  };

  if (nblk > 0) dma_block(sb0, 0);

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
  float m_ref = kNegInf;  // reference max of this row, log2 units (same in both lane halves)
  float l_run = 0.f;      // this lane's share of the row sum (halves add up at the end)
  const bool pos_scale = a.c > 0.f;

  wait_vmem();
  __syncthreads();

  for (int j = 0; j < nblk; ++j) {
    const int blk = sb0 + j;
    const int buf = j & 1;
    if (j + 1 < nblk) dma_block(blk + 1, buf ^ 1);

    const char* kl = smem + buf * S::BUF;
    const char* vl = kl + S::KBYTES;
    const int kw = blk * S::BK + wk * BKW;  // first key of this wave's slice

    // A wave whose rows see none of its keys skips the arithmetic.
    const bool skip = kw >= a.Lk || (a.mask != MASK_NONE && kw > pmax_w) ||
                      (a.mask == MASK_WINDOW && kw + BKW - 1 <= pmin_w - a.window);
    if (!skip) {
      // ---- S^T = K Q^T for this wave's BKW keys ----
      f32x16 sacc[S::NKT];
#pragma unroll
      for (int kt = 0; kt < S::NKT; ++kt) {
        sacc[kt] = f32x16{};
        const int row = wk * BKW + kt * 32 + col;
        const char* krow = kl + row * S::KROW;
        const int sw = row & (S::KSW - 1);
#pragma unroll
        for (int s = 0; s < S::NQS; ++s) {
          frag af;
          if constexpr (E::ES == 2) {
            const int c = (2 * s + hl) ^ sw;  // 8 elements = one chunk
            af = *(const u32x4*)(krow + c * 16);
          } else {
            const int d = 2 * s + hl;
            af = *(const float*)(krow + (((d >> 2) ^ sw) << 4) + (d & 3) * 4);
          }
          sacc[kt] = E::mma(af, qf[s], sacc[kt]);
        }
      }

      // ---- mask edge blocks (diagonal, window edge, Lk tail) ----
      const bool edge = (kw + BKW > a.Lk) || (a.mask != MASK_NONE && kw + BKW - 1 > pmin_w) ||
                        (a.mask == MASK_WINDOW && kw <= pmax_w - a.window);
      if (edge) {
#pragma unroll
        for (int kt = 0; kt < S::NKT; ++kt) {
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = kw + kt * 32 + 8 * (e >> 2) + 4 * hl + (e & 3);
            bool vis = key < a.Lk;
            if (a.mask != MASK_NONE) vis = vis && key <= pos;
            if (a.mask == MASK_WINDOW) vis = vis && key > pos - a.window;
            // masked scores become -inf in log2 units whatever the scale's sign
            if (!vis) sacc[kt][e] = pos_scale ? kNegInf : __builtin_inff();
          }
        }
      }

      // ---- online softmax with lazy rescaling ----
      float mx;
      if (pos_scale) {
        mx = kNegInf;
#pragma unroll
        for (int kt = 0; kt < S::NKT; ++kt)
#pragma unroll
          for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[kt][e]);
      } else {  // scale <= 0: the largest scaled score is the smallest raw one
        mx = __builtin_inff();
#pragma unroll
        for (int kt = 0; kt < S::NKT; ++kt)
#pragma unroll
          for (int e = 0; e < 16; ++e) mx = fminf(mx, sacc[kt][e]);
      }
      mx = pos_scale ? wave_max32(mx) : -wave_max32(-mx);
      // block max in log2 units; an all-masked block gives -inf (or NaN for
      // a zero scale times +inf, treated as -inf by the comparison below)
      const float mxs = (mx == kNegInf || mx == __builtin_inff()) ? kNegInf : mx * a.c;
      const bool need = mxs > m_ref + kRescale;
      if (__builtin_amdgcn_ballot_w64(need)) {
        const float m_new = need ? mxs : m_ref;
        const float alpha = need ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.0f;
        l_run *= alpha;
#pragma unroll
        for (int t = 0; t < S::NDT; ++t) oacc[t] *= alpha;
        m_ref = m_new;
      }
      const float msub = (m_ref == kNegInf) ? 0.f : m_ref;
#pragma unroll
      for (int kt = 0; kt < S::NKT; ++kt) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float x = sacc[kt][e];
          const float t = pos_scale ? __builtin_fmaf(x, a.c, -msub)
                                    : ((x == __builtin_inff()) ? kNegInf : x * a.c - msub);
          const float p = __builtin_amdgcn_exp2f(t);
          sacc[kt][e] = p;
          l_run += p;
        }
      }

      // ---- O^T += V^T P^T ----
#pragma unroll
      for (int kt = 0; kt < S::NKT; ++kt) {
        const int kbase_t = wk * BKW + kt * 32;  // first key of this tile inside the block
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
            frag af;
            if constexpr (E::ES == 2) {
              // Transposing read: lane t16 of group g supplies the address of
              // 4 dv values of one key; the hardware hands lane i of the group
              // element i%4 of the chunk addressed by lane 4j + i/4, i.e. the
              // 4 keys (j = 0..3) of dv column 16*(g%2) + i.
              const int g = lane >> 4, t16 = lane & 15;
              const int dv0 = 32 * t + 16 * (g & 1) + 4 * (t16 & 3);
              u32x2 half[2];
#pragma unroll
              for (int rr = 0; rr < 2; ++rr) {
                const int row = kbase_t + 16 * s2 + 8 * rr + 4 * (g >> 1) + (t16 >> 2);
                const int c = (dv0 >> 3) ^ (2 * (row & (S::VSW - 1)));
                const char* p = vl + row * S::VROW + c * 16 + (dv0 & 7) * 2;
                const i16x4 v4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SDPA_LDS i16x4*)p);
                half[rr] = __builtin_bit_cast(u32x2, v4);
              }
              u32x4 f;
              f[0] = half[0][0];
              f[1] = half[0][1];
              f[2] = half[1][0];
              f[3] = half[1][1];
              af = f;
            } else {
              const int row = kbase_t + 8 * (s2 >> 2) + 4 * hl + (s2 & 3);
              const int dv = 32 * t + col;
              const int c = (dv >> 2) ^ (2 * (row & (S::VSW - 1)));
              af = *(const float*)(vl + row * S::VROW + c * 16 + (dv & 3) * 4);
            }
            oacc[t] = E::mma(af, bf, oacc[t]);
          }
        }
      }
    }

    wait_vmem();
    __syncthreads();
  }

  // ---- epilogue ----
  const float l_row = l_run + __shfl_xor(l_run, 32);  // both halves' keys
  const int64_t ws_row = ((int64_t)z * a.R + r) * a.splits + split;

  if constexpr (NWK == 1) {
    if (!row_ok) return;
    if (a.splits == 1) {
      const float inv = 1.0f / l_row;
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
        a.lse[((int64_t)b * a.Hq + hq) * a.Lq + iq] = (m_ref + log2f(l_row)) * kLn2;
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
      if (hl == 0) *(float2*)(a.ws_ml + ws_row * 2) = make_float2(m_ref, l_row);
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
        mml[(slot * 32 + col) * 2 + 0] = m_ref;
        mml[(slot * 32 + col) * 2 + 1] = l_row;
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
