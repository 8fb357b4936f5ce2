// Backward pass of fused attention for gfx950: dQ, dK, dV of
// O = softmax(scale Q K^T + mask) V, given dO and the forward's log-sum-exp.
//
// With P recomputed from the saved log-sum-exp (no running max: P = 2^(s c -
// lse2) is final), the gradients are dV = P^T dO, dS = P (dO V^T - D) with
// D_i = dO_i . O_i, dQ = scale dS K and dK = scale dS^T Q (mlx PR #4185
// "Add force_fused option to scaled_dot_product_attention", API: the
// log-sum-exp is the output training needs; mlx PR #3552 "feat(fast): add
// sliding-window SDPA kernel path", Outstanding: the VJP was not extended).
//
// Three kernels, none with atomics, so every result is deterministic:
//   bwd_prep   per packed row: D, the log-sum-exp in log2 units, the query
//              index; laid out in packed-row order so tiles of rows are
//              contiguous.
//   bwd_dq     a row tile (128 packed rows, one 32-row group per wave) walks
//              the key blocks: S^T = K Q^T and dP^T = V dO^T (Q, dO in
//              registers), dS^T, then dQ^T += K^T dS^T through the
//              transposing LDS read of the K tile -- the forward's layout
//              with dS^T in place of P^T and K in place of V.
//   bwd_dkdv   a key tile (128 keys, 32 per wave; K and V rows stay in LDS)
//              walks the query blocks (32 packed rows, shared by the waves):
//              S = Q K^T and dP = dO V^T with the keys on the lanes, then
//              dV^T += dO^T P and dK^T += Q^T dS through transposing reads of
//              the Q and dO tiles.  Packed rows cover all G query heads of
//              the KV head, so grouped-query sums come out of the loop.
// Tiles move by the same 16-byte LDS DMA as the forward (counted waits).
//
// bwd_dq and bwd_dkdv only read what bwd_prep wrote and write disjoint
// outputs, so dQ runs on a second stream of the library's own beside dK/dV
// (fork after the prep, join before the call returns to the caller's
// stream).  One dK/dV workgroup (99 KB of LDS) and one dQ workgroup (32 KB)
// then share a CU, two waves per SIMD where each kernel alone leaves one.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "attn_kernel.h"

namespace sdpa {
namespace dev {

// LDS tile whose rows hold D 16-bit elements: logical 16-byte chunk c of
// row r sits at chunk c ^ sw(r), a permutation inside aligned groups of KG
// chunks.  The backward reads the same tile both ways -- 16 consecutive rows
// at one logical chunk (row operands) and 4 consecutive rows at 4
// consecutive chunks (transposing reads) -- so sw must spread both over the
// 256-byte bank window: with u = r >> KSH (rows sharing a window differ in
// the low KSH bits), sw is a bijection of u's low bits whose two top bits
// change with u's lowest bits.  (The forward's K swizzle alone is 4x
// conflicted on the transposing reads at D = 128, its V swizzle 4x on row
// reads.)
template <int D>
struct Tile {
  static constexpr int ROWB = D * 2;
  static constexpr int CH = ROWB / 16;
  static constexpr int KG = (CH % 16 == 0) ? 16 : (CH % 8 == 0) ? 8 : 4;
  static constexpr int KSH = KG == 16 ? 0 : (KG == 8 ? 1 : 2);
  static __device__ __forceinline__ int sw(int row) {
    const int u = row >> KSH;
    if constexpr (KG == 16) return ((u & 3) << 2) | ((u >> 2) & 3);
    else if constexpr (KG == 8) return ((u & 1) << 2) | ((u >> 1) & 3);
    else return u & 3;
  }
  static __device__ __forceinline__ int off(int row, int chunk) { return row * ROWB + 16 * (chunk ^ sw(row)); }
};

// MFMA operand of 8 consecutive elements of tile row `row` (k-step s, lane
// half hl): the A operand with rows on the lanes, or the B operand with
// columns on the lanes.
template <int D>
__device__ __forceinline__ u32x4 row_frag(const SDPA_LDS char* t, int row, int s, int hl) {
  return *(const SDPA_LDS u32x4*)(t + Tile<D>::off(row, 2 * s + hl));
}

// A operand of tile^T: output rows are the tile columns 32 tt .. 32 tt + 31,
// the k dimension is 16 tile rows from row0, in the order pack_frag uses
// for the B operand (the forward's V^T read).
template <int D>
__device__ __forceinline__ u32x4 tr_frag(const SDPA_LDS char* t, int row0, int tt, int lane) {
  const int g = lane >> 4, t16 = lane & 15;
  const int r = row0 + 4 * (g >> 1) + (t16 >> 2);
  const int chunk = 4 * tt + 2 * (g & 1) + ((t16 & 3) >> 1);
  const int b8 = 8 * (t16 & 1);
  const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SDPA_LDS i16x4*)(t + Tile<D>::off(r, chunk) + b8));
  const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SDPA_LDS i16x4*)(t + Tile<D>::off(r + 8, chunk) + b8));
  const u32x2 h0 = __builtin_bit_cast(u32x2, v0), h1 = __builtin_bit_cast(u32x2, v1);
  u32x4 f;
  f[0] = h0[0];
  f[1] = h0[1];
  f[2] = h1[0];
  f[3] = h1[1];
  return f;
}

// B operand from an accumulator (rows = the k dimension of the next
// product): registers 8 s2 .. 8 s2 + 7, rounded to the input type.
template <class E>
__device__ __forceinline__ u32x4 pack_frag(const f32x16& x, int s2) {
  u32x4 pk;
#pragma unroll
  for (int w = 0; w < 4; ++w) pk[w] = E::pack2(x[8 * s2 + 2 * w], x[8 * s2 + 2 * w + 1]);
  return pk;
}

// LDS DMA of NR rows into `lds`: the 1 KB instructions are dealt out to the
// NW waves; rowptr(row) is the row's global base; chunks past the real width
// (vch chunks) re-read the last real one (their products are discarded or
// meet zero operands).
template <int D, int NR, int NW, class RowPtr>
__device__ __forceinline__ void dma_rows(unsigned lds, int wave_u, int lane, int vch, RowPtr rowptr) {
  using T = Tile<D>;
  constexpr int NI = NR * T::ROWB / 1024;
  static_assert(NR * T::ROWB % 1024 == 0, "tiles must be whole DMA instructions");
  constexpr int PW = (NI + NW - 1) / NW;
#pragma unroll
  for (int ii = 0; ii < PW; ++ii) {
    const int ins = ii * NW + wave_u;
    if ((ii + 1) * NW > NI && ins >= NI) continue;
    const int sl = ins * 64 + lane;
    const int row = sl / T::CH;
    const int lch = (sl % T::CH) ^ T::sw(row);
    lds_dma16<false>(rowptr(row) + min(lch, vch - 1) * 16, lds + ins * 1024);
  }
}

// s_waitcnt takes its count as an immediate: wait until at most n (a
// wave-uniform count, 0 <= n <= N) vector memory operations are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt_upto(int n) {
  if constexpr (N > 0) {
    if (n < N) {
      wait_vmcnt_upto<N - 1>(n);
      return;
    }
  }
  wait_vmcnt<N>();
}

template <class E>
__device__ __forceinline__ float lo16(unsigned w) {
  return E::to_float((unsigned short)(w & 0xffffu));
}
template <class E>
__device__ __forceinline__ float hi16(unsigned w) {
  return E::to_float((unsigned short)(w >> 16));
}

// Batch entry b's valid queries and keys (per-batch lengths, clamped to the
// padded shape; the whole padded shape without them).  Its query i sits at
// key position i + Lk_b - Lq_b.
struct EntryLens {
  int Lq, Lk, R, off;
};
__device__ __forceinline__ EntryLens entry_lens(const BwdArgs& a, int b) {
  EntryLens e;
  e.Lq = a.q_lens ? min(max(a.q_lens[b], 0), a.Lq) : a.Lq;
  e.Lk = a.kv_lens ? min(max(a.kv_lens[b], 0), a.Lk) : a.Lk;
  e.R = a.G * e.Lq;
  e.off = e.Lk - e.Lq;
  return e;
}

// ---- per packed row: D = dO . O, lse in log2 units, query index ----
// 16 lanes per row, 8 elements each (dv <= 128).
template <class E>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdArgs a) {
  const int tid = threadIdx.x;
  const int l16 = tid & 15;
  const int64_t grow = (int64_t)blockIdx.x * 16 + (tid >> 4);  // z * Rp + r
  const int64_t Z = (int64_t)a.B * a.Hkv;
  if (grow >= Z * a.Rp) return;  // no barriers below
  const int z = (int)(grow / a.Rp), r = (int)(grow % a.Rp);
  const int b = z / a.Hkv, kvh = z % a.Hkv;
  const bool ok = r < entry_lens(a, b).R;  // rows past the entry's queries: P = 0, D = 0
  float dsum = 0.f, lse2 = __builtin_inff();
  if (ok) {
    const int i = r / a.G, h = kvh * a.G + r % a.G;
    const int d0 = 8 * l16;
    if (d0 < a.dv) {
      const char* orow = (const char*)a.o + ((int64_t)b * a.os[0] + (int64_t)h * a.os[1] + (int64_t)i * a.os[2]) * 2;
      const char* drow =
          (const char*)a.dout + ((int64_t)b * a.os[0] + (int64_t)h * a.os[1] + (int64_t)i * a.os[2]) * 2;
      const u32x4 ov = *(const u32x4*)(orow + d0 * 2);
      const u32x4 dw = *(const u32x4*)(drow + d0 * 2);
#pragma unroll
      for (int w = 0; w < 4; ++w) dsum += lo16<E>(ov[w]) * lo16<E>(dw[w]) + hi16<E>(ov[w]) * hi16<E>(dw[w]);
    }
    const float l = a.lse[((int64_t)b * a.Hq + h) * a.Lq + i];
    lse2 = l == kNegInf ? __builtin_inff() : l * kLog2e;  // a row without keys gets P = 0
  }
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) dsum += __shfl_xor(dsum, o, 16);
  if (l16 == 0) {
    a.ws_lse2[grow] = lse2;
    a.ws_d[grow] = dsum;
  }
  if (z == 0 && l16 == 1) a.ws_qi[r] = min(r, a.R - 1) / a.G;
}

// ---- dQ: rows on the lanes, walking the key blocks ----
// MASKED: instantiated for an explicit mask array (a.ma != MA_NONE); the
// plain instance carries none of its code or registers.
template <class E, int D, bool MASKED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1))) void bwd_dq_kernel(BwdArgs a) {
  using T = Tile<D>;
  // keys per block: 64 while two key tiles' scores fit the registers (head
  // dims up to 96: 228 VGPRs at 96); at 128 they would spill into the
  // accumulation registers (causal L=4096 backward 422 -> 433 us, grouped
  // queries 739 -> 816 us), while at 96 the longer block saves a barrier per
  // 32 keys (L=2048 D=96 173 -> 168 us)
  constexpr int BK = D <= 96 ? 64 : 32;
  constexpr int NKT = BK / 32;
  constexpr int NQS = D / 16;
  constexpr int NDT = D / 32;
  constexpr int TB = BK * T::ROWB;  // one K or V tile
  constexpr int NI = TB / 1024;
  constexpr int DMA_MAX = 2 * ((NI + 3) / 4);
  static_assert(2 * DMA_MAX <= 63, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) char smem_[4 * TB];  // K0 K1 V0 V1
  SDPA_LDS char* const smem = (SDPA_LDS char*)smem_;
  const unsigned lds_base = (unsigned)(uintptr_t)smem;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int col = lane & 31, hl = lane >> 5;
  // Tile-major order, heaviest first: under a causal mask the last row tiles
  // see the most keys, so they go out first, every head's before any lighter
  // tile, and the short tiles fill in behind them (in-order dispatch onto
  // free CUs then balances like longest-processing-time-first).
  const int row_tiles = (a.R + 127) / 128;
  const int Z = (int)(gridDim.x / row_tiles);
  const int rt = row_tiles - 1 - (int)(blockIdx.x / Z);
  const int z = blockIdx.x % Z;
  const int b = z / a.Hkv, kvh = z % a.Hkv;
  const EntryLens en = entry_lens(a, b);
  const int r_wg = rt * 128;
  const int r = r_wg + wave * 32 + col;
  if (r_wg >= en.R) {
    // Every row of the tile lies past the entry's queries (uniform, before
    // any barrier): their gradient is 0.
    if (r < a.R) {
      const int iz = r / a.G, hz = kvh * a.G + r % a.G;
      char* zrow = (char*)a.grad_q + ((int64_t)b * a.qs[0] + (int64_t)hz * a.qs[1] + (int64_t)iz * a.qs[2]) * 2;
      for (int d = 8 * hl; d < a.dqk; d += 16)
        *(u32x4*)(zrow + d * 2) = u32x4{0u, 0u, 0u, 0u};
    }
    return;
  }
  const bool row_ok = r < en.R;
  const int rc = min(r, en.R - 1);  // rows past the entry read its last row (their P is 0)
  const int iq = rc / a.G;
  const int hq = kvh * a.G + rc % a.G;
  const int pos = iq + en.off;
  const int pmax_wg = (min(en.R, r_wg + 128) - 1) / a.G + en.off;
  const int pmin_wg = r_wg / a.G + en.off;
  const int pmin_w = min(r_wg + wave * 32, en.R - 1) / a.G + en.off;
  const int pmax_w = min(r_wg + wave * 32 + 31, en.R - 1) / a.G + en.off;

  int k_lo = 0, k_hi = en.Lk;
  if (a.mask != MASK_NONE) k_hi = min(en.Lk, pmax_wg + 1);
  if (a.mask == MASK_WINDOW) k_lo = max(0, pmin_wg - a.window + 1);
  const int kb_first = k_lo / BK;
  const int nblk = max(0, (k_hi + BK - 1) / BK - kb_first);

  const char* kbase = (const char*)a.k + ((int64_t)b * a.ks[0] + (int64_t)kvh * a.ks[1]) * 2;
  const char* vbase = (const char*)a.v + ((int64_t)b * a.vs[0] + (int64_t)kvh * a.vs[1]) * 2;
  const int64_t kstr = a.ks[2] * 2, vstr = a.vs[2] * 2;
  // Per-lane part of each DMA source (row and swizzled chunk of the tile),
  // fixed for the whole loop; a block adds its first key's row offset.  The
  // tail block (keys past Lk) clamps each row to the last key instead.
  constexpr int PW = (NI + 3) / 4;
  int krow[PW], kcb[PW], vcb[PW];
  int64_t kofs[PW], vofs[PW];
#pragma unroll
  for (int ii = 0; ii < PW; ++ii) {
    const int sl = (ii * 4 + wave_u) * 64 + lane;
    const int row = sl / T::CH;
    const int lch = (sl % T::CH) ^ T::sw(row);
    krow[ii] = row;
    kcb[ii] = min(lch, a.dqk / 8 - 1) * 16;
    vcb[ii] = min(lch, a.dv / 8 - 1) * 16;
    kofs[ii] = (int64_t)row * kstr + kcb[ii];
    vofs[ii] = (int64_t)row * vstr + vcb[ii];
  }
  auto dma = [&](int blk, int buf) __attribute__((always_inline)) {
    const int k0 = blk * BK;
    const bool full = k0 + BK <= en.Lk;
    const char* kb = kbase + (int64_t)k0 * kstr;
    const char* vb = vbase + (int64_t)k0 * vstr;
#pragma unroll
    for (int ii = 0; ii < PW; ++ii) {
      const int ins = ii * 4 + wave_u;
      if ((ii + 1) * 4 > NI && ins >= NI) continue;
      const char* ks = full ? kb + kofs[ii] : kbase + (int64_t)min(k0 + krow[ii], en.Lk - 1) * kstr + kcb[ii];
      const char* vs = full ? vb + vofs[ii] : vbase + (int64_t)min(k0 + krow[ii], en.Lk - 1) * vstr + vcb[ii];
      lds_dma16<false>(ks, lds_base + buf * TB + ins * 1024);
      lds_dma16<false>(vs, lds_base + (2 + buf) * TB + ins * 1024);
    }
  };
  if (nblk > 0) dma(kb_first, 0);

  // Q and dO fragments (B operands), zero past the real dims and rows
  u32x4 qf[NQS], of[NQS];
  {
    const char* qrow = (const char*)a.q + ((int64_t)b * a.qs[0] + (int64_t)hq * a.qs[1] + (int64_t)iq * a.qs[2]) * 2;
    const char* drow =
        (const char*)a.dout + ((int64_t)b * a.os[0] + (int64_t)hq * a.os[1] + (int64_t)iq * a.os[2]) * 2;
#pragma unroll
    for (int s = 0; s < NQS; ++s) {
      const int d = 16 * s + 8 * hl;
      qf[s] = (row_ok && d < a.dqk) ? *(const u32x4*)(qrow + d * 2) : u32x4{0u, 0u, 0u, 0u};
      of[s] = (row_ok && d < a.dv) ? *(const u32x4*)(drow + d * 2) : u32x4{0u, 0u, 0u, 0u};
    }
  }
  const int64_t wrow = (int64_t)z * a.Rp + rc;
  const float lse2 = row_ok ? a.ws_lse2[wrow] : __builtin_inff();
  const float drow_d = row_ok ? a.ws_d[wrow] : 0.f;
  // this row of the mask array (rows past the entry read its last row)
  const char* mrow = MASKED ? (const char*)a.mask_arr + ((int64_t)b * a.ms[0] + (int64_t)hq * a.ms[1] +
                                                                 (int64_t)iq * a.ms[2]) * a.mes
                                     : nullptr;
  f32x16 acc[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) acc[t] = f32x16{};
  wait_vmcnt<0>();  // block 0 and the register loads have landed
  if (nblk > 1) dma(kb_first + 1, 1);
  // DMA instructions this wave issues per block (K and V each): while block
  // j + 1 is in flight, block j has landed once no more than these remain
  const int dma_w = 2 * max(0, (NI - wave_u + 3) / 4);

  for (int j = 0; j < nblk; ++j) {
    if (j + 1 < nblk) wait_vmcnt_upto<DMA_MAX>(dma_w);
    else wait_vmcnt<0>();
    __syncthreads();
    const SDPA_LDS char* kt_ = smem + (j & 1) * TB;
    const SDPA_LDS char* vt_ = smem + (2 + (j & 1)) * TB;
    const int k0 = (kb_first + j) * BK;
    f32x16 sacc[NKT], pacc[NKT];
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
      sacc[kt] = f32x16{};
      pacc[kt] = f32x16{};
#pragma unroll
      for (int s = 0; s < NQS; ++s) {
        sacc[kt] = E::mma(row_frag<D>(kt_, kt * 32 + col, s, hl), qf[s], sacc[kt]);
        pacc[kt] = E::mma(row_frag<D>(vt_, kt * 32 + col, s, hl), of[s], pacc[kt]);
      }
      // register e: key k0 + 32 kt + 8 (e / 4) + 4 hl + e % 4 of this row;
      // only tiles on a mask edge or past Lk test each key
      const int kw = k0 + kt * 32;
      const bool edge = (kw + 32 > en.Lk) || (a.mask != MASK_NONE && kw + 31 > pmin_w) ||
                        (a.mask == MASK_WINDOW && kw <= pmax_w - a.window);
      if constexpr (MASKED) {
        // Mask array: each group of 4 registers covers 4 consecutive keys,
        // read as one 4-byte (boolean) or 8-byte (additive) load; keys past
        // Lk read the row's first group and are masked anyway.  An additive
        // value joins the exponent in log2 units, as in the forward.
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int kk = kw + 8 * g + 4 * hl;
          const char* pm = mrow + (kk < a.Lk ? kk : 0) * a.mes;
          unsigned mb = 0xffffffffu;
          u32x2 mw = {0u, 0u};
          if (a.ma == MA_BOOL) mb = *(const unsigned*)pm;
          else mw = *(const u32x2*)pm;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int e = 4 * g + t;
            const int key = kk + t;
            bool vis = key < en.Lk;
            if (a.mask != MASK_NONE) vis = vis && key <= pos;
            if (a.mask == MASK_WINDOW) vis = vis && key > pos - a.window;
            float madd = 0.f;
            if (a.ma == MA_BOOL) vis = vis && ((mb >> (8 * t)) & 0xffu) != 0u;
            else madd = E::to_float((unsigned short)(mw[t >> 1] >> (16 * (t & 1)))) * kLog2e;
            const float p = vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kt][e], a.c, madd - lse2)) : 0.f;
            sacc[kt][e] = vis ? p * (pacc[kt][e] - drow_d) : 0.f;  // dS^T (without the scale)
          }
        }
      } else if (edge) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = kw + 8 * (e >> 2) + 4 * hl + (e & 3);
          bool vis = key < en.Lk;
          if (a.mask != MASK_NONE) vis = vis && key <= pos;
          if (a.mask == MASK_WINDOW) vis = vis && key > pos - a.window;
          const float p = vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kt][e], a.c, -lse2)) : 0.f;
          sacc[kt][e] = p * (pacc[kt][e] - drow_d);  // dS^T (without the scale)
        }
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kt][e], a.c, -lse2));
          sacc[kt][e] = p * (pacc[kt][e] - drow_d);
        }
      }
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const u32x4 bf = pack_frag<E>(sacc[kt], s2);
#pragma unroll
        for (int t = 0; t < NDT; ++t) acc[t] = E::mma(tr_frag<D>(kt_, kt * 32 + 16 * s2, t, lane), bf, acc[t]);
      }
    }
    if (j + 2 < nblk) {
      __syncthreads();  // every wave is done with block j's buffers
      dma(kb_first + j + 2, j & 1);
    }
  }

  if (r >= a.R) return;
  // rows past the entry's queries write their gradient, 0 (their P was 0)
  const int iw = row_ok ? iq : r / a.G, hw = row_ok ? hq : kvh * a.G + r % a.G;
  char* orow = (char*)a.grad_q + ((int64_t)b * a.qs[0] + (int64_t)hw * a.qs[1] + (int64_t)iw * a.qs[2]) * 2;
#pragma unroll
  for (int t = 0; t < NDT; ++t) {
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d = t * 32 + 8 * i4 + 4 * hl;
      if (d < a.dqk) {
        u32x2 w;
        w[0] = E::pack2(acc[t][4 * i4 + 0] * a.scale, acc[t][4 * i4 + 1] * a.scale);
        w[1] = E::pack2(acc[t][4 * i4 + 2] * a.scale, acc[t][4 * i4 + 3] * a.scale);
        *(u32x2*)(orow + d * 2) = w;
      }
    }
  }
}

// ---- dK, dV: keys on the lanes, walking the query blocks ----
template <class E, int D, bool MASKED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1))) void bwd_dkdv_kernel(BwdArgs a) {
  using T = Tile<D>;
  constexpr int BQ = 32;  // packed rows per block
  constexpr int NQS = D / 16;
  constexpr int NDT = D / 32;
  constexpr int REG = 128 * T::ROWB;  // K (or V) rows of the tile's 128 keys
  constexpr int TQ = BQ * T::ROWB;    // one Q or dO tile
  constexpr int NIQ = TQ / 1024;
  constexpr int BUF = 2 * TQ + 512;   // Q, dO, then lse2 / D / query index (3 x 128 bytes)
  constexpr int DMA_MAX = 2 * ((NIQ + 3) / 4) + 1;
  static_assert(2 * DMA_MAX <= 63, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) char smem_[2 * REG + 2 * BUF];
  SDPA_LDS char* const smem = (SDPA_LDS char*)smem_;
  const unsigned lds_base = (unsigned)(uintptr_t)smem;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int col = lane & 31, hl = lane >> 5;
  // Tile-major order, heaviest first: under a causal mask the first key
  // tiles are seen by the most queries, so every head's tile 0 goes out
  // before any tile 1, and so on (see the dq kernel).  With kv_parts > 1
  // each (tile, head) is kv_parts workgroups, one per part of its rows.
  const int key_tiles = (a.Lk + 127) / 128;
  const int P = a.kv_parts;
  const int Z = (int)(gridDim.x / (key_tiles * P));
  const int kti = (int)(blockIdx.x / (Z * P));
  const int part = (int)(blockIdx.x / Z) % P;
  const int z = blockIdx.x % Z;
  const int b = z / a.Hkv, kvh = z % a.Hkv;
  const EntryLens en = entry_lens(a, b);
  const int k_wg = kti * 128;
  const int key = k_wg + wave * 32 + col;  // this lane's key
  if (k_wg >= en.Lk || en.R == 0) {
    // No key of the tile is valid, or the entry has no queries (uniform,
    // before any barrier): every gradient of the tile's keys is 0.
    if (key < a.Lk && P > 1) {
      float* zp = a.ws_part + (((int64_t)part * Z + z) * a.Lk + key) * (a.dqk + a.dv);
      for (int d = 4 * hl; d < a.dqk + a.dv; d += 8) *(f32x4*)(zp + d) = f32x4{0.f, 0.f, 0.f, 0.f};
    } else if (key < a.Lk) {
      char* zk = (char*)a.grad_k + ((int64_t)b * a.ks[0] + (int64_t)kvh * a.ks[1] + (int64_t)key * a.ks[2]) * 2;
      char* zv = (char*)a.grad_v + ((int64_t)b * a.vs[0] + (int64_t)kvh * a.vs[1] + (int64_t)key * a.vs[2]) * 2;
      for (int d = 8 * hl; d < a.dqk; d += 16) *(u32x4*)(zk + d * 2) = u32x4{0u, 0u, 0u, 0u};
      for (int d = 8 * hl; d < a.dv; d += 16) *(u32x4*)(zv + d * 2) = u32x4{0u, 0u, 0u, 0u};
    }
    return;
  }

  // packed rows that may see a key of the tile: causal needs pos >= k_wg,
  // a window pos - W < k_wg + 127
  int64_t r_lo = 0, r_hi = en.R;
  if (a.mask != MASK_NONE) r_lo = (int64_t)max(0, k_wg - en.off) * a.G;
  if (a.mask == MASK_WINDOW) {
    const int64_t i_hi = (int64_t)min(en.Lk - 1, k_wg + 127) + a.window - 1 - en.off;  // last query that sees it
    r_hi = min<int64_t>(en.R, i_hi < 0 ? 0 : (i_hi + 1) * a.G);
  }
  int jb0 = (int)(min<int64_t>(r_lo, en.R) / BQ);
  int nblk = r_hi > r_lo ? (int)((r_hi + BQ - 1) / BQ) - jb0 : 0;
  if (P > 1) {
    // this part's share of the blocks (possibly none: it then writes zeros)
    const int lo = (int)((int64_t)nblk * part / P), hi = (int)((int64_t)nblk * (part + 1) / P);
    jb0 += lo;
    nblk = hi - lo;
  }

  // K / V rows past the entry's keys re-read its last key (their P is 0)
  const char* kbase = (const char*)a.k + ((int64_t)b * a.ks[0] + (int64_t)kvh * a.ks[1]) * 2;
  const char* vbase = (const char*)a.v + ((int64_t)b * a.vs[0] + (int64_t)kvh * a.vs[1]) * 2;
  const int64_t kstr = a.ks[2] * 2, vstr = a.vs[2] * 2;
  const SDPA_LDS char* kreg = smem;
  const SDPA_LDS char* vreg = smem + REG;
  dma_rows<D, 128, 4>(lds_base, wave_u, lane, a.dqk / 8,
                      [&](int row) { return kbase + (int64_t)min(k_wg + row, en.Lk - 1) * kstr; });
  dma_rows<D, 128, 4>(lds_base + REG, wave_u, lane, a.dv / 8,
                      [&](int row) { return vbase + (int64_t)min(k_wg + row, en.Lk - 1) * vstr; });

  // Q / dO rows of this lane's DMA instructions: packed row r0 + rq[ii] of
  // each block, i.e. query (r0 + rq) / G of head kvh G + (r0 + rq) % G.  The
  // blocks are fetched in order, one BQ rows after the other, so the
  // (head, query) pair and the element offsets advance by fixed steps
  // instead of a division per row; rows past R read row R - 1.
  constexpr int PWQ = (NIQ + 3) / 4;
  int rq[PWQ], gq[PWQ], cq[PWQ], co[PWQ];
  int64_t qo[PWQ], oo[PWQ];
  const int gq_step = BQ % a.G, iq_step = BQ / a.G;
  const int64_t q_step = (int64_t)iq_step * a.qs[2] + (int64_t)gq_step * a.qs[1];
  const int64_t o_step = (int64_t)iq_step * a.os[2] + (int64_t)gq_step * a.os[1];
  const int64_t q_wrap = a.qs[2] - (int64_t)a.G * a.qs[1], o_wrap = a.os[2] - (int64_t)a.G * a.os[1];
  const int64_t q_head = (int64_t)b * a.qs[0] + (int64_t)kvh * a.G * a.qs[1];
  const int64_t o_head = (int64_t)b * a.os[0] + (int64_t)kvh * a.G * a.os[1];
  const int64_t q_last = q_head + (int64_t)((en.R - 1) % a.G) * a.qs[1] + (int64_t)((en.R - 1) / a.G) * a.qs[2];
  const int64_t o_last = o_head + (int64_t)((en.R - 1) % a.G) * a.os[1] + (int64_t)((en.R - 1) / a.G) * a.os[2];
#pragma unroll
  for (int ii = 0; ii < PWQ; ++ii) {
    const int sl = (ii * 4 + wave_u) * 64 + lane;
    const int row = sl / T::CH;
    const int lch = (sl % T::CH) ^ T::sw(row);
    rq[ii] = row;
    cq[ii] = min(lch, a.dqk / 8 - 1) * 16;
    co[ii] = min(lch, a.dv / 8 - 1) * 16;
    const int rr = jb0 * BQ + row;
    gq[ii] = rr % a.G;
    qo[ii] = q_head + (int64_t)gq[ii] * a.qs[1] + (int64_t)(rr / a.G) * a.qs[2];
    oo[ii] = o_head + (int64_t)gq[ii] * a.os[1] + (int64_t)(rr / a.G) * a.os[2];
  }

  // Block jb into buffer buf; calls come in the order jb0, jb0 + 1, ...
  auto dma_blk = [&](int jb, int buf) __attribute__((always_inline)) {
    const unsigned qb = lds_base + 2 * REG + buf * BUF;
    const int r0 = jb * BQ;
#pragma unroll
    for (int ii = 0; ii < PWQ; ++ii) {
      const int ins = ii * 4 + wave_u;
      if ((ii + 1) * 4 > NIQ && ins >= NIQ) continue;
      const bool in = r0 + rq[ii] < en.R;
      lds_dma16<false>((const char*)a.q + (in ? qo[ii] : q_last) * 2 + cq[ii], qb + ins * 1024);
      lds_dma16<false>((const char*)a.dout + (in ? oo[ii] : o_last) * 2 + co[ii], qb + TQ + ins * 1024);
      gq[ii] += gq_step;
      qo[ii] += q_step;
      oo[ii] += o_step;
      if (gq[ii] >= a.G) {
        gq[ii] -= a.G;
        qo[ii] += q_wrap;
        oo[ii] += o_wrap;
      }
    }
    if (wave_u == 0) {
      // 32 rows of lse2, D and the query index: 8 lanes (16 bytes) each
      if (lane < 24) {
        const int part = lane >> 3, q4 = 4 * (lane & 7);
        const char* src = part == 0 ? (const char*)(a.ws_lse2 + (int64_t)z * a.Rp + r0 + q4)
                          : part == 1 ? (const char*)(a.ws_d + (int64_t)z * a.Rp + r0 + q4)
                                      : (const char*)(a.ws_qi + r0 + q4);
        lds_dma16<false>(src, qb + 2 * TQ);
      }
    }
  };
  if (nblk > 0) dma_blk(jb0, 0);
  f32x16 dk[NDT], dv[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) {
    dk[t] = f32x16{};
    dv[t] = f32x16{};
  }
  wait_vmcnt<0>();  // K, V rows and block 0 have landed
  if (a.dqk < D || a.dv < D) {
    // Padded head dims: zero the K and V columns past the real ones, so the
    // Q and dO columns there (re-read copies of the last real chunk) add
    // nothing to S and dP.  Every wave's K/V DMA must have landed first.
    __syncthreads();
    SDPA_LDS char* kw_ = smem;
    for (int idx = tid; idx < 128 * T::CH; idx += 256) {
      const int row = idx / T::CH, c = idx % T::CH;
      if (8 * c >= a.dqk) *(SDPA_LDS u32x4*)(kw_ + T::off(row, c)) = u32x4{0u, 0u, 0u, 0u};
      if (8 * c >= a.dv) *(SDPA_LDS u32x4*)(kw_ + REG + T::off(row, c)) = u32x4{0u, 0u, 0u, 0u};
    }
  }
  if (nblk > 1) dma_blk(jb0 + 1, 1);
  // DMA instructions this wave issues per block (Q and dO each, plus the
  // lse2 / D / query-index tile on wave 0): while block j + 1 is in flight,
  // block j has landed once no more than these remain
  const int dma_w = 2 * max(0, (NIQ - wave_u + 3) / 4) + (wave_u == 0 ? 1 : 0);
  // First and last packed row of the current block as (query, head in the
  // group) pairs, stepped by BQ rows per block like the DMA rows.
  const int g_step = BQ % a.G, i_step = BQ / a.G;
  int i_first = (jb0 * BQ) / a.G, g_first = (jb0 * BQ) % a.G;
  int i_last = (jb0 * BQ + BQ - 1) / a.G, g_last = (jb0 * BQ + BQ - 1) % a.G;
  const int i_rmax = (en.R - 1) / a.G;
  const int kw = k_wg + wave_u * 32;  // this wave's first key
  // this lane's key column of the mask array, batch entry b
  const char* mkey = MASKED ? (const char*)a.mask_arr + ((int64_t)b * a.ms[0] + (key < a.Lk ? key : 0)) * a.mes
                                     : nullptr;

  for (int j = 0; j < nblk; ++j) {
    if (j + 1 < nblk) wait_vmcnt_upto<DMA_MAX>(dma_w);
    else wait_vmcnt<0>();
    __syncthreads();
    const SDPA_LDS char* qt = smem + 2 * REG + (j & 1) * BUF;
    const SDPA_LDS char* dt = qt + TQ;
    const SDPA_LDS char* sm = qt + 2 * TQ;
    f32x16 sacc = f32x16{}, pacc = f32x16{};
#pragma unroll
    for (int s = 0; s < NQS; ++s) {
      sacc = E::mma(row_frag<D>(qt, col, s, hl), row_frag<D>(kreg, wave * 32 + col, s, hl), sacc);
      pacc = E::mma(row_frag<D>(dt, col, s, hl), row_frag<D>(vreg, wave * 32 + col, s, hl), pacc);
    }
    // register e: packed row r0 + 8 (e / 4) + 4 hl + e % 4 of this lane's
    // key.  Only blocks on a mask edge for this wave's 32 keys, or with keys
    // past the entry's length, test each pair (rows past the entry's
    // queries carry lse2 = +inf, so their P is 0 either way).
    const int r0 = (jb0 + j) * BQ;
    const int pmin_b = i_first + en.off;
    const int pmax_b = (r0 + BQ - 1 < en.R ? i_last : i_rmax) + en.off;
    i_first += i_step;
    g_first += g_step;
    if (g_first >= a.G) {
      g_first -= a.G;
      ++i_first;
    }
    i_last += i_step;
    g_last += g_step;
    if (g_last >= a.G) {
      g_last -= a.G;
      ++i_last;
    }
    const bool edge = (kw + 32 > en.Lk) || (a.mask != MASK_NONE && kw + 31 > pmin_b) ||
                      (a.mask == MASK_WINDOW && kw <= pmax_b - a.window);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int rb = 8 * g + 4 * hl;
      const f32x4 l4 = *(const SDPA_LDS f32x4*)(sm + rb * 4);
      const f32x4 d4 = *(const SDPA_LDS f32x4*)(sm + 128 + rb * 4);
      if constexpr (MASKED) {
        // Mask array: element (packed row, this lane's key) read one by one;
        // the row's (query head, query) come from its query index, rows past
        // R from row R - 1, keys past Lk from key 0 (masked anyway).
        const u32x4 i4 = *(const SDPA_LDS u32x4*)(sm + 256 + rb * 4);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int e = 4 * g + t;
          const int iq = (int)i4[t];
          const int rr = min(r0 + rb + t, a.R - 1);
          const int hq = kvh * a.G + (rr - iq * a.G);
          const char* pm = mkey + ((int64_t)hq * a.ms[1] + (int64_t)iq * a.ms[2]) * a.mes;
          const int pos = iq + en.off;
          bool vis = key < en.Lk;
          if (a.mask != MASK_NONE) vis = vis && key <= pos;
          if (a.mask == MASK_WINDOW) vis = vis && key > pos - a.window;
          float madd = 0.f;
          if (a.ma == MA_BOOL) vis = vis && *(const unsigned char*)pm != 0;
          else madd = E::to_float(*(const unsigned short*)pm) * kLog2e;
          const float p = vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[e], a.c, madd - l4[t])) : 0.f;
          sacc[e] = p;                                  // P
          pacc[e] = vis ? p * (pacc[e] - d4[t]) : 0.f;  // dS (without the scale)
        }
      } else if (edge) {
        const u32x4 i4 = *(const SDPA_LDS u32x4*)(sm + 256 + rb * 4);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int e = 4 * g + t;
          const int pos = (int)i4[t] + en.off;
          bool vis = key < en.Lk;
          if (a.mask != MASK_NONE) vis = vis && key <= pos;
          if (a.mask == MASK_WINDOW) vis = vis && key > pos - a.window;
          const float p = vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[e], a.c, -l4[t])) : 0.f;
          sacc[e] = p;                     // P
          pacc[e] = p * (pacc[e] - d4[t]);  // dS (without the scale)
        }
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int e = 4 * g + t;
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[e], a.c, -l4[t]));
          sacc[e] = p;
          pacc[e] = p * (pacc[e] - d4[t]);
        }
      }
    }
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const u32x4 bp = pack_frag<E>(sacc, s2);
      const u32x4 bs = pack_frag<E>(pacc, s2);
#pragma unroll
      for (int t = 0; t < NDT; ++t) {
        dv[t] = E::mma(tr_frag<D>(dt, 16 * s2, t, lane), bp, dv[t]);
        dk[t] = E::mma(tr_frag<D>(qt, 16 * s2, t, lane), bs, dk[t]);
      }
    }
    if (j + 2 < nblk) {
      __syncthreads();  // every wave is done with block j's buffers
      dma_blk(jb0 + j + 2, j & 1);
    }
  }

  if (key >= a.Lk) return;
  if (P > 1) {
    // partial sums of this part's rows, float32, dK before the scale
    float* wp = a.ws_part + (((int64_t)part * Z + z) * a.Lk + key) * (a.dqk + a.dv);
#pragma unroll
    for (int t = 0; t < NDT; ++t) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = t * 32 + 8 * i4 + 4 * hl;
        if (d < a.dqk)
          *(f32x4*)(wp + d) = f32x4{dk[t][4 * i4], dk[t][4 * i4 + 1], dk[t][4 * i4 + 2], dk[t][4 * i4 + 3]};
        if (d < a.dv)
          *(f32x4*)(wp + a.dqk + d) =
              f32x4{dv[t][4 * i4], dv[t][4 * i4 + 1], dv[t][4 * i4 + 2], dv[t][4 * i4 + 3]};
      }
    }
    return;
  }
  char* krow = (char*)a.grad_k + ((int64_t)b * a.ks[0] + (int64_t)kvh * a.ks[1] + (int64_t)key * a.ks[2]) * 2;
  char* vrow = (char*)a.grad_v + ((int64_t)b * a.vs[0] + (int64_t)kvh * a.vs[1] + (int64_t)key * a.vs[2]) * 2;
#pragma unroll
  for (int t = 0; t < NDT; ++t) {
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d = t * 32 + 8 * i4 + 4 * hl;
      if (d < a.dqk) {
        u32x2 w;
        w[0] = E::pack2(dk[t][4 * i4 + 0] * a.scale, dk[t][4 * i4 + 1] * a.scale);
        w[1] = E::pack2(dk[t][4 * i4 + 2] * a.scale, dk[t][4 * i4 + 3] * a.scale);
        *(u32x2*)(krow + d * 2) = w;
      }
      if (d < a.dv) {
        u32x2 w;
        w[0] = E::pack2(dv[t][4 * i4 + 0], dv[t][4 * i4 + 1]);
        w[1] = E::pack2(dv[t][4 * i4 + 2], dv[t][4 * i4 + 3]);
        *(u32x2*)(vrow + d * 2) = w;
      }
    }
  }
}

// ---- dK, dV from the row parts: their float32 sums in part order ----
// One thread per 4 consecutive columns of one key's [dK | dV] row (Dqk and Dv
// are multiples of 8, so no group straddles the two).
template <class E>
__global__ __launch_bounds__(256) void bwd_kvsum_kernel(BwdArgs a) {
  const int nc = (a.dqk + a.dv) / 4;
  const int64_t per_z = (int64_t)a.Lk * nc;
  const int64_t zn = (int64_t)a.B * a.Hkv;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= zn * per_z) return;
  const int z = (int)(idx / per_z);
  const int64_t rem = idx % per_z;
  const int key = (int)(rem / nc), d = 4 * (int)(rem % nc);
  const int b = z / a.Hkv, kvh = z % a.Hkv;
  const float* src = a.ws_part + ((int64_t)z * a.Lk + key) * (a.dqk + a.dv) + d;
  const int64_t pstride = zn * a.Lk * (a.dqk + a.dv);
  f32x4 acc = *(const f32x4*)src;
  for (int q = 1; q < a.kv_parts; ++q) acc += *(const f32x4*)(src + q * pstride);
  u32x2 w;
  if (d < a.dqk) {
    w[0] = E::pack2(acc[0] * a.scale, acc[1] * a.scale);
    w[1] = E::pack2(acc[2] * a.scale, acc[3] * a.scale);
    char* krow = (char*)a.grad_k + ((int64_t)b * a.ks[0] + (int64_t)kvh * a.ks[1] + (int64_t)key * a.ks[2]) * 2;
    *(u32x2*)(krow + d * 2) = w;
  } else {
    w[0] = E::pack2(acc[0], acc[1]);
    w[1] = E::pack2(acc[2], acc[3]);
    char* vrow = (char*)a.grad_v + ((int64_t)b * a.vs[0] + (int64_t)kvh * a.vs[1] + (int64_t)key * a.vs[2]) * 2;
    *(u32x2*)(vrow + (d - a.dqk) * 2) = w;
  }
}

// The dQ kernel's stream: `s2` with the fork and join events, or s2 = null
// for one stream (the caller's) throughout.
struct DqStream {
  hipStream_t s2 = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};

template <class E, int D>
int launch_bwd_dims(const BwdPlan& p, const BwdArgs& a, hipStream_t s, const DqStream& ds) {
  hipLaunchKernelGGL(bwd_prep_kernel<E>, dim3((unsigned)p.prep_grid), dim3(256), 0, s, a);
  const bool masked = a.ma != MA_NONE;
  hipStream_t sq = s;
  if (ds.s2 && p.dq_grid > 0 && p.dkdv_grid > 0) {
    if (hipEventRecord(ds.fork, s) != hipSuccess || hipStreamWaitEvent(ds.s2, ds.fork, 0) != hipSuccess)
      return SDPA_E_HIP;
    sq = ds.s2;
  }
  if (p.dq_grid > 0) {
    if (masked) hipLaunchKernelGGL((bwd_dq_kernel<E, D, true>), dim3((unsigned)p.dq_grid), dim3(256), 0, sq, a);
    else hipLaunchKernelGGL((bwd_dq_kernel<E, D, false>), dim3((unsigned)p.dq_grid), dim3(256), 0, sq, a);
  }
  if (sq != s && hipEventRecord(ds.join, sq) != hipSuccess) return SDPA_E_HIP;
  if (p.dkdv_grid > 0) {
    if (masked) hipLaunchKernelGGL((bwd_dkdv_kernel<E, D, true>), dim3((unsigned)p.dkdv_grid), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((bwd_dkdv_kernel<E, D, false>), dim3((unsigned)p.dkdv_grid), dim3(256), 0, s, a);
  }
  if (p.kv_parts > 1 && p.sum_grid > 0)
    hipLaunchKernelGGL(bwd_kvsum_kernel<E>, dim3((unsigned)p.sum_grid), dim3(256), 0, s, a);
  if (sq != s && hipStreamWaitEvent(s, ds.join, 0) != hipSuccess) return SDPA_E_HIP;
  return SDPA_OK;
}

template <class E>
int launch_bwd_type(const BwdPlan& p, const BwdArgs& a, hipStream_t s, const DqStream& ds) {
  switch (p.d_pad) {
    case 32: return launch_bwd_dims<E, 32>(p, a, s, ds);
    case 64: return launch_bwd_dims<E, 64>(p, a, s, ds);
    case 96: return launch_bwd_dims<E, 96>(p, a, s, ds);
    case 128: return launch_bwd_dims<E, 128>(p, a, s, ds);
    default: return SDPA_E_HEAD_DIM;
  }
}

}  // namespace dev

namespace {

// One dQ stream (default priority, non-blocking) and its two events per
// device, made on the first backward call on that device outside a graph
// capture and kept until the process ends.  Where they cannot be made, or
// the first call comes under capture, the call runs on the caller's stream
// alone.  The mutex spans the enqueue of a whole call, so concurrent callers
// cannot interleave their records and waits on the shared events.
constexpr int kMaxDevices = 64;
std::mutex g_dq_mu;
int g_dq_state[kMaxDevices] = {0};  // 0 not made yet, 1 ready, -1 unavailable
dev::DqStream g_dq[kMaxDevices];

void make_dq_stream(int d) {
  dev::DqStream ds;
  if (hipStreamCreateWithFlags(&ds.s2, hipStreamNonBlocking) == hipSuccess &&
      hipEventCreateWithFlags(&ds.fork, hipEventDisableTiming) == hipSuccess &&
      hipEventCreateWithFlags(&ds.join, hipEventDisableTiming) == hipSuccess) {
    g_dq[d] = ds;
    g_dq_state[d] = 1;
    return;
  }
  if (ds.join) (void)hipEventDestroy(ds.join);
  if (ds.fork) (void)hipEventDestroy(ds.fork);
  if (ds.s2) (void)hipStreamDestroy(ds.s2);
  (void)hipGetLastError();  // the failure is handled: one stream
  g_dq_state[d] = -1;
}

}  // namespace

int launch_backward(const BwdPlan& p, const BwdArgs& a, void* stream, std::string* err) {
  const hipStream_t s = (hipStream_t)stream;
  int d = -1;
  std::lock_guard<std::mutex> lock(g_dq_mu);
  dev::DqStream ds;
  if (hipGetDevice(&d) == hipSuccess && d >= 0 && d < kMaxDevices) {
    if (g_dq_state[d] == 0) {
      hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
      if (hipStreamIsCapturing(s, &cs) == hipSuccess && cs == hipStreamCaptureStatusNone) make_dq_stream(d);
      (void)hipGetLastError();
    }
    if (g_dq_state[d] == 1) ds = g_dq[d];
  }
  const int rc = p.dtype == SDPA_BF16 ? dev::launch_bwd_type<dev::BF16>(p, a, s, ds)
                                      : dev::launch_bwd_type<dev::F16>(p, a, s, ds);
  if (rc == SDPA_E_HIP) {
    *err = std::string("backward stream fork/join failed: ") + hipGetErrorString(hipGetLastError());
    return rc;
  }
  if (rc != SDPA_OK) {
    *err = "no backward kernel for padded head dim " + std::to_string(p.d_pad);
    return rc;
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    *err = std::string("backward kernel launch failed: ") + hipGetErrorString(e);
    return SDPA_E_HIP;
  }
  return SDPA_OK;
}

}  // namespace sdpa
