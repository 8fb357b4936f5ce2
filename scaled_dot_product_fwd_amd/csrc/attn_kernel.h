// Fused attention forward kernel for gfx950 (CDNA4, wave64, MFMA).
//
// One workgroup owns a tile of packed query rows of one (batch, KV head) and a
// contiguous range of key blocks, and walks that range block by block with an
// online softmax (running row max m and row sum l, rescaled accumulator), so
// the Lq x Lk score matrix never exists (mlx PR #4185 "Add force_fused option
// to scaled_dot_product_attention", Background: with K/V taken in tiles the
// temporary memory does not grow with the key length).
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
// exact for unaligned windows too.
//
// Explicit mask array (MA != MA_NONE): the block's [rows x keys] tile of
// the array rides the same LDS DMA pipeline as K and V and is applied to the
// scores of every block before the running max: a boolean array sends removed
// keys to -inf, an additive one is added to the scaled scores (mlx PR #3552
// "feat(fast): add sliding-window SDPA kernel path", Public API: the mask
// array beside the mask mode).  A row that keeps no key ends with l = 0 and
// writes 0.
//
// Split-K (mlx issue #3826, second and third comments: the block-parallel
// reduction over S): the blocks of the range may be dealt out to `splits`
// workgroups; each writes its unnormalised O with (m, l) and a combine kernel
// merges them by log-sum-exp.  With per-batch key lengths the workgroups of a
// KV head are dealt to the batch entries by their key blocks instead of
// evenly (kv_balance_count).
//
// Lazy rescaling: the reference max m of a row only moves when a block's max
// exceeds it by more than kRescale (log2 units); otherwise the block is
// accumulated against the old reference, so probabilities stay <= 2^kRescale
// and the O/l rescale (Dv multiplies per row) is skipped for most blocks.  The
// result is the same softmax: O, l and m stay mutually consistent.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

#include "sdpa_internal.h"

namespace sdpa {
namespace dev {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define SDPA_LDS __attribute__((address_space(3)))

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;
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
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const f32x2 v = {x, y};  // one v_cvt_pk_bf16_f32, round to nearest even
    return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
  }
  static __device__ __forceinline__ unsigned short to_store(float x) {
    return __builtin_bit_cast(unsigned short, (__bf16)x);
  }
  static __device__ __forceinline__ float to_float(unsigned short h) {
    return __builtin_bit_cast(float, (unsigned)h << 16);
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
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const f32x2 v = {x, y};  // one v_cvt_pk_f16_f32, round to nearest even
    return __builtin_bit_cast(unsigned, __builtin_convertvector(v, f16x2));
  }
  static __device__ __forceinline__ unsigned short to_store(float x) {
    return __builtin_bit_cast(unsigned short, (_Float16)x);
  }
  static __device__ __forceinline__ float to_float(unsigned short h) {
    return (float)__builtin_bit_cast(_Float16, h);
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
template <class E, int DQK, int DV, int NWQ, int NWK, int BKW, int MA = MA_NONE, int NWD = 1>
struct Shape {
  static constexpr int NW = NWQ * NWK * NWD;
  static constexpr int NT = NW * 64;
  static constexpr int BM = NWQ * 32;          // rows per workgroup
  static constexpr int BK = NWK * BKW;         // keys per block
  static constexpr int NKT = BKW / 32;         // 32-key tiles per wave
  static constexpr int NDT = DV / 32;          // 32-wide dv tiles
  static constexpr int NDTW = NDT / NWD;       // dv tiles one wave accumulates
  static constexpr int NQS = DQK / E::KQK;     // QK MFMAs per key tile
  // With the dv split each wave of a pair also takes half of the QK
  // product's depth (its Q columns), and the pair adds its partial scores
  // through LDS: NQSW steps per wave.
  static constexpr int NQSW = NQS / NWD;
  static constexpr int KCH = DQK * E::ES / 16; // 16-byte chunks per K row
  static constexpr int VCH = DV * E::ES / 16;  // 16-byte chunks per V row
  static constexpr int KROW = DQK * E::ES;
  static constexpr int VROW = DV * E::ES;
  static constexpr int KBYTES = BK * KROW;
  static constexpr int VBYTES = BK * VROW;
  static constexpr int BUF = KBYTES + VBYTES;
  static constexpr int KDMA = KBYTES / 1024;   // 1 KB DMA instructions per tile
  static constexpr int VDMA = VBYTES / 1024;
  // Mask array tile: BM rows of BK keys, MES bytes each, kept row-major in
  // 16-byte slots (MNS per row).  Slot ^ msw(row) spreads the 32 rows a wave
  // reads at one key offset over the 256-byte bank window.
  static constexpr int MES = MA == MA_NONE ? 0 : (MA == MA_BOOL ? 1 : E::ES);
  static constexpr int MROWB = BK * MES;
  static constexpr int MNS = MROWB / 16;
  static constexpr int MBYTES = BM * MROWB;
  static constexpr int MDMA = MBYTES / 1024;
  static constexpr int MRPW = MNS >= 16 ? 1 : 16 / cmax(MNS, 1);  // rows per 256-byte window
  static __device__ __forceinline__ int msw(int row) { return MNS ? (row / MRPW) & (MNS - 1) : 0; }
  // Chunk swizzles (16-byte chunks; the LDS serves 256 bytes per cycle).
  // K: the QK operand read has 16 lanes of consecutive rows reading the same
  // logical chunk per cycle; chunk ^ kx(row) puts them in 16 distinct slots
  // of the 256-byte bank window.  V: a transposing read group covers 4
  // consecutive rows (32 bytes each); chunk ^ vy(row) spreads them over the
  // window.  Each swizzle permutes chunks inside aligned groups (KG, VG
  // chunks), so it never leaves the row.  Rows of 10 chunks (head dim 80):
  // 10 r mod 16 takes 8 distinct even slots for r = 0..7 and repeats for
  // r = 8..15, so flipping the chunk's low bit on row bit 3 (pairs of
  // chunks) moves the second eight rows onto the odd slots.
  static constexpr int KG = (KCH % 16 == 0) ? 16 : (KCH % 8 == 0) ? 8 : (KCH % 4 == 0) ? 4 : 2;
  static constexpr int KSH = (KG == 16) ? 0 : (KG == 8) ? 1 : (KG == 4) ? 2 : 3;
  static constexpr int VG = (VCH % 16 == 0) ? 16 : (VCH % 8 == 0) ? 8 : 4;
  static __device__ __forceinline__ int kx(int row) { return (row >> KSH) & (KG - 1); }
  static __device__ __forceinline__ int vy(int row) {
    return VG == 16 ? 4 * (row & 3) : (VG == 8 ? 2 * (row & 3) : 2 * (row & 1));
  }
  // Two K buffers, two V buffers and two mask buffers (see the kernel's
  // block loop); the cross-wave merge below reuses them, and needs a little
  // more than they hold for the smallest head dims.
  static constexpr int MSLOTS = NWQ * (NWK - 1);
  static constexpr int MLB = (MSLOTS * 32 * 8 + 15) / 16 * 16;
  // Partial-score exchange of the dv split: one 32 x 32 float32 tile per
  // wave, stored chunk-major (chunk c of lane l at 1024 c + 16 l).
  static constexpr int XOFF = 2 * BUF + 2 * MBYTES;
  static constexpr int XBYTES = NWD > 1 ? NW * 4096 : 0;
  static constexpr int LDS = cmax(XOFF + XBYTES, MLB + MSLOTS * 32 * (32 + 4) * 4);
  // Families that split the keys over waves (decode, short queries) have one
  // row tile per KV head in practice, so each K/V byte is read once per
  // launch: stream it past the caches.  Prefill row tiles re-read the same
  // K/V from L2.
  static constexpr bool STREAM = NWK > 1;
  // Operand fragments read ahead of their products when the extra registers
  // (4 per fragment) stay within a budget (16-bit types only).
  static constexpr bool HOIST_K = E::ES == 2 && NKT * NQS * 4 <= 48;
  static constexpr bool HOIST_V = NWD == 1 && E::ES == 2 && NKT * (32 / E::KPV) * NDT * 4 <= 48 &&
                                  NQS * 4 + NDT * 16 <= 128;
  // Software-pipelined block loop (QK of the next block overlapping this
  // block's softmax) where two blocks of scores fit next to Q and O:
  // four-wave prefill tiles of the small head dims, and without a mask array
  // of head dims (both) from 192 with 32-key blocks (one wave per SIMD there, so the instruction schedule
  // alone has to overlap the matrix products with the softmax), 16-bit types.
  static constexpr bool PIPE = NWK == 1 && NWD == 1 && E::ES == 2 &&
                               (NQS * 4 + NDT * 16 + 2 * NKT * 16 <= 144 || (DQK >= 192 && DV >= 192 && NKT == 1 && MA == MA_NONE));
  // DMA instructions one block costs the wave that issues the fewest / most.
  static constexpr int DMA_MIN = KDMA / NW + VDMA / NW + MDMA / NW;
  static constexpr int DMA_MAX = (KDMA + NW - 1) / NW + (VDMA + NW - 1) / NW + (MDMA + NW - 1) / NW;
  // Cross-wave merge (NWK > 1), through the idle tile buffers: (m, l) of
  // the waves with wk > 0 first, as [slot][q][2]; then their O in rounds of
  // TPR dv tiles, as [slot][q][MROW] after the (m, l) bytes, TPR as large
  // as fits.
  static constexpr int merge_tiles() {
    for (int t = NDT; t >= 1; --t)
      if (NDT % t == 0 && MLB + MSLOTS * 32 * (t * 32 + 4) * 4 <= LDS) return t;
    return 0;
  }
  static constexpr int TPR = merge_tiles();
  static constexpr int MROW = TPR * 32 + 4;  // +4 floats skew the rows across banks
  static_assert(NWK == 1 || TPR >= 1, "merge scratch must fit the tile buffers");
  static_assert(NWD == 1 || (NWK == 1 && NDT % NWD == 0), "dv split: waves on rows only, whole dv tiles");
  static_assert(NWD == 1 || (NWD == 2 && NKT == 1 && NQSW % (KG / 2) == 0),
                "dv split: wave pairs, one key tile, whole K swizzle groups per half");
  static_assert(DMA_MAX <= 63, "vmcnt range");
  static_assert(BKW % 32 == 0, "BKW must be a multiple of 32");
  static_assert(DQK % E::KQK == 0 && DV % 32 == 0, "bad head-dim tile");
  static_assert(KBYTES % 1024 == 0 && VBYTES % 1024 == 0 && MBYTES % 1024 == 0,
                "tiles must be whole DMA instructions");
  static_assert(LDS <= 160 * 1024, "LDS budget of one workgroup exceeded");
};

// Combine lanes l and l ^ 32 without a trip through LDS: the lane-half swap
// leaves {lower half, lower half} in one result and {upper, upper} in the
// other.
__device__ __forceinline__ float wave_max32(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)sw[0]), __builtin_bit_cast(float, (unsigned)sw[1]));
}
__device__ __forceinline__ float wave_sum32(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)sw[0]) + __builtin_bit_cast(float, (unsigned)sw[1]);
}

// LDS DMA of 16 bytes per lane: lane l's chunk at `src` lands at LDS byte
// address lds + 16 l.  Issued as a single instruction the compiler does not
// track, so it inserts no wait for it anywhere; the kernel waits itself with
// wait_vmcnt.  The instruction has no register result; its address registers
// are consumed at issue.  STREAM marks the load non-temporal: data read once
// per launch should not displace what the caches hold for re-use.
template <bool STREAM>
__device__ __forceinline__ void lds_dma16(const void* src, unsigned lds) {
  if constexpr (STREAM)
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
                 :
                 : "v"(src), "s"(lds)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(lds)
                 : "memory", "m0");
}

// The same with a wave-uniform base address in scalar registers and a 32-bit
// per-lane byte offset (the instruction's scalar-base form: no 64-bit address
// arithmetic per lane and load).
template <bool STREAM>
__device__ __forceinline__ void lds_dma16_s(const char* base, unsigned off, unsigned lds) {
  if constexpr (STREAM)
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                 :
                 : "v"(off), "s"(base), "s"(lds)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(off), "s"(base), "s"(lds)
                 : "memory", "m0");
}

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);  // expcnt, lgkmcnt: no wait
}

template <class E, int DQK, int DV, int NWQ, int NWK, int BKW, int WPE, int MA, int NWD>
__global__ __launch_bounds__(NWQ * NWK * NWD * 64) __attribute__((amdgpu_waves_per_eu(WPE)))
void attn_fwd_kernel(AttnArgs a) {
  using S = Shape<E, DQK, DV, NWQ, NWK, BKW, MA, NWD>;
  using frag = typename E::frag;
  __shared__ __attribute__((aligned(1024))) char smem_[S::LDS];
  // All LDS addressing goes through an LDS-typed pointer, so addresses stay
  // 32-bit and loop-invariant parts fold into the instructions' offsets.
  SDPA_LDS char* const smem = (SDPA_LDS char*)smem_;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wq = wave % NWQ;
  const int wk = (wave / NWQ) % NWK;
  // dv split (NWD > 1, the largest head dims): waves wd = 0..NWD-1 share the
  // same rows, each computes their scores and softmax and accumulates the dv
  // tiles [wd NDTW, (wd + 1) NDTW) of O, so no wave holds the whole O row
  const int wd = wave / (NWQ * NWK);
  const int tw0 = wd * S::NDTW;
  const int col = lane & 31;  // query column of this lane in S^T / O^T
  const int hl = lane >> 5;   // lane half

  // ---- workgroup -> (row tile, split, batch * KV head) ----
  // The hardware deals workgroups to the 8 XCDs round-robin (workgroup w to
  // XCD w % 8) and each XCD has its own L2.  With xcd_group = g, each XCD
  // takes g consecutive work items at a time instead of every 8th one, so
  // neighbouring row tiles, which read nearly the same keys, share an L2.
  // The remap is a permutation of the first multiple of 8 g ids; the
  // remainder keeps its order.
  int id = blockIdx.x;
  if (a.xcd_group > 0) {
    const int span = 8 * a.xcd_group;
    if (id < (int)(gridDim.x / span) * span) {
      const int x = id % 8, slot = id / 8;
      id = ((slot / a.xcd_group) * 8 + x) * a.xcd_group + slot % a.xcd_group;
    }
  }
  int rt, split, z;
  if (a.heavy_first == 2) {
    // Tile-major, heaviest first (causal or window, one split, no XCD
    // grouping): every KV head's longest row tile goes out before any
    // shorter one, so in-order dispatch onto free CUs balances like
    // longest-processing-time-first instead of finishing one head's short
    // tiles while later heads' long tiles still queue.
    const int Z = (int)(gridDim.x / a.row_tiles);
    rt = a.row_tiles - 1 - id / Z;
    split = 0;
    z = id % Z;
  } else {
    rt = id % a.row_tiles;
    id /= a.row_tiles;
    split = id % a.splits;
    z = id / a.splits;
    if (a.heavy_first) rt = a.row_tiles - 1 - rt;
  }
  // Splits of this row tile's key range, and (balanced lengths) the first
  // partial row of its batch entry's workspace segment, in units of R rows.
  int nsp = a.splits;
  int64_t seg = 0;
  if (a.kv_balance > 0) {
    // The B * splits workgroups of KV head z % Hkv go to the batch entries
    // in proportion to their key blocks, so a long entry is not left to the
    // same few workgroups as a short one.  Uniform: before any barrier.
    const int kvh_ = z % a.Hkv;
    const int W = a.B * a.splits;
    const int w = (z / a.Hkv) * a.splits + split;
    const int T = kv_balance_total(a.kv_lens, a.B, a.Lk, a.kv_balance);
    int P = 0, e = 0, s_e = 0;
    for (; e < a.B; ++e) {
      s_e = kv_balance_count(kv_balance_blocks(a.kv_lens, e, a.Lk, a.kv_balance), W, a.B, T);
      if (w < P + s_e) break;
      P += s_e;
    }
    if (e == a.B) return;  // a workgroup the rounding left without work
    split = w - P;
    nsp = s_e;
    z = e * a.Hkv + kvh_;
    seg = (int64_t)kvh_ * W + P;
  }
  const int b = z / a.Hkv;
  const int kvh = z % a.Hkv;

  // ---- this batch entry's lengths ----
  // With per-batch lengths, entry b uses its first Lq queries and Lk keys
  // and query i sits at key position i + Lk - Lq: the K-relative coordinates
  // of mlx PR #3552 "feat(fast): add sliding-window SDPA kernel path"
  // (Implementation) applied to the valid part.  A tile wholly past the
  // entry's queries has nothing to do (uniform: before any barrier or DMA).
  int Lk = a.Lk, Lq = a.Lq;
  if (a.kv_lens) Lk = min(max(a.kv_lens[b], 0), a.Lk);
  if (a.q_lens) Lq = min(max(a.q_lens[b], 0), a.Lq);
  const int R = a.G * Lq;  // packed rows of this entry
  const int off = Lk - Lq;

  // ---- rows of this lane / wave / workgroup ----
  const int r_wg = rt * S::BM;
  if (r_wg >= R) return;
  const int r_wave = r_wg + wq * 32;
  const int r = r_wave + col;
  const bool row_ok = r < R;
  const int iq = r / a.G;
  const int pos = iq + off;  // key position of this row's query
  const int hq = kvh * a.G + r % a.G;

  const int r_last_wg = min(R, r_wg + S::BM) - 1;
  const int pmin_wg = r_wg / a.G + off;
  const int pmax_wg = r_last_wg / a.G + off;
  const int r_last_wave = min(R - 1, r_wave + 31);
  const int pmin_w = min(r_wave, R - 1) / a.G + off;
  const int pmax_w = r_last_wave / a.G + off;

  // ---- key block range of the tile, then of this split ----
  // (a causal tile placed before the first key gets an empty range)
  int k_lo = 0, k_hi = Lk;
  if (a.mask != MASK_NONE) k_hi = min(Lk, pmax_wg + 1);
  if (a.mask == MASK_WINDOW) k_lo = max(0, pmin_wg - a.window + 1);
  const int kb_first = k_lo / S::BK;
  const int kb_end = (k_hi + S::BK - 1) / S::BK;
  const int nb = kb_end - kb_first;
  // Split `split` takes every splits-th block of the range, starting at its
  // own index: at any moment the splits of one head read neighbouring
  // blocks, so the whole grid streams one region of memory together rather
  // than `splits` regions far apart (which maps unevenly onto the HBM
  // channels).  Block j of this workgroup is blk(j).
  const int nblk = split < nb ? (nb - 1 - split) / nsp + 1 : 0;
  auto blk = [&](int j) { return kb_first + split + j * nsp; };

  // ---- LDS DMA of one key block into buffer `buf` ----
  // Each wave issues KPW + VPW DMA instructions per block; lane l of
  // instruction i fills LDS slot 64 i + l (16 bytes) with the chunk that the
  // swizzle puts there.  The per-lane byte offset inside a block is fixed, so
  // it is computed once; only the tail block (rows past Lk) recomputes it,
  // re-reading the last key (masked later) instead of leaving the tensor.
  // Chunks past the real head dim re-read the row's last real chunk; they
  // meet zero Q columns or land in discarded output columns.
  const char* kbase = (const char*)a.k + ((int64_t)b * a.ks[0] + (int64_t)kvh * a.ks[1]) * E::ES;
  const char* vbase = (const char*)a.v + ((int64_t)b * a.vs[0] + (int64_t)kvh * a.vs[1]) * E::ES;
  const int64_t kstr = a.ks[2] * E::ES;
  const int64_t vstr = a.vs[2] * E::ES;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  constexpr int KPW = (S::KDMA + S::NW - 1) / S::NW;  // the last round may leave waves idle
  constexpr int VPW = (S::VDMA + S::NW - 1) / S::NW;
  const int kch_valid = a.dqk * E::ES / 16;  // chunks of real data per row
  const int vch_valid = a.dv * E::ES / 16;
  // (row, byte column) of LDS slot `slot` of a K or V tile
  auto kslot = [&](int slot, int& row, int& colb) {
    row = slot / S::KCH;
    colb = min((slot % S::KCH) ^ S::kx(row), kch_valid - 1) * 16;
  };
  auto vslot = [&](int slot, int& row, int& colb) {
    row = slot / S::VCH;
    colb = min((slot % S::VCH) ^ S::vy(row), vch_valid - 1) * 16;
  };
  unsigned koff[KPW], voff[VPW];
#pragma unroll
  for (int ii = 0; ii < KPW; ++ii) {
    int row, colb;
    kslot((ii * S::NW + wave_u) * 64 + lane, row, colb);
    koff[ii] = (unsigned)(row * kstr) + colb;
  }
#pragma unroll
  for (int ii = 0; ii < VPW; ++ii) {
    int row, colb;
    vslot((ii * S::NW + wave_u) * 64 + lane, row, colb);
    voff[ii] = (unsigned)(row * vstr) + colb;
  }

  // LDS: K tiles in two buffers, then V tiles in two buffers.  Block j's K
  // sits in K buffer j % 2 and its V in V buffer j % 2.
  const unsigned lds_base = (unsigned)(uintptr_t)smem;
  // Block jj of this split starts at key blk(jj) * BK: its K and V rows
  // begin at a wave-uniform address (scalar registers), and each lane adds
  // its fixed 32-bit offset (the planner bounds a block's rows below 2 GiB).
  const char* const kblk0 = kbase + (int64_t)(kb_first + split) * S::BK * kstr;
  const char* const vblk0 = vbase + (int64_t)(kb_first + split) * S::BK * vstr;
  const int64_t kstep = (int64_t)nsp * S::BK * kstr;
  const int64_t vstep = (int64_t)nsp * S::BK * vstr;
  auto dma_k = [&](int jj, int buf) __attribute__((always_inline)) {
    const int k0 = blk(jj) * S::BK;
    const unsigned kl = lds_base + buf * S::KBYTES;
    const char* kb = kblk0 + jj * kstep;
    if (k0 + S::BK <= Lk) {
#pragma unroll
      for (int ii = 0; ii < KPW; ++ii)
        if ((ii + 1) * S::NW <= S::KDMA || ii * S::NW + wave_u < S::KDMA)
          lds_dma16_s<S::STREAM>(kb, koff[ii], kl + (ii * S::NW + wave_u) * 1024);
    } else {
#pragma unroll
      for (int ii = 0; ii < KPW; ++ii) {
        if ((ii + 1) * S::NW > S::KDMA && ii * S::NW + wave_u >= S::KDMA) continue;
        int row, colb;
        kslot((ii * S::NW + wave_u) * 64 + lane, row, colb);
        const int lrow = min(row, Lk - 1 - k0);
        lds_dma16_s<S::STREAM>(kb, (unsigned)(lrow * kstr) + colb, kl + (ii * S::NW + wave_u) * 1024);
      }
    }
  };
  auto dma_v = [&](int jj, int buf) __attribute__((always_inline)) {
    const int k0 = blk(jj) * S::BK;
    const unsigned vl = lds_base + 2 * S::KBYTES + buf * S::VBYTES;
    const char* vb = vblk0 + jj * vstep;
    if (k0 + S::BK <= Lk) {
#pragma unroll
      for (int ii = 0; ii < VPW; ++ii)
        if ((ii + 1) * S::NW <= S::VDMA || ii * S::NW + wave_u < S::VDMA)
          lds_dma16_s<S::STREAM>(vb, voff[ii], vl + (ii * S::NW + wave_u) * 1024);
    } else {
#pragma unroll
      for (int ii = 0; ii < VPW; ++ii) {
        if ((ii + 1) * S::NW > S::VDMA && ii * S::NW + wave_u >= S::VDMA) continue;
        int row, colb;
        vslot((ii * S::NW + wave_u) * 64 + lane, row, colb);
        const int lrow = min(row, Lk - 1 - k0);
        lds_dma16_s<S::STREAM>(vb, (unsigned)(lrow * vstr) + colb, vl + (ii * S::NW + wave_u) * 1024);
      }
    }
  };

  // Mask tile DMA: lane l of instruction i fills slot 64 i + l of the tile,
  // i.e. row (64 i + l) / MNS, physical slot (64 i + l) % MNS, which holds
  // logical slot physical ^ msw(row) of that row.  Rows past the packed rows
  // re-read the last one; slots past Lk in the tail block re-read the slot
  // holding key Lk - 1 (those keys are masked anyway).
  constexpr int MPW = S::MDMA ? (S::MDMA + S::NW - 1) / S::NW : 1;
  const char* mptr[MPW];
  int mls[MPW];
  if constexpr (MA != MA_NONE) {
#pragma unroll
    for (int ii = 0; ii < MPW; ++ii) {
      const int sl = (ii * S::NW + wave_u) * 64 + lane;
      const int row = sl / S::MNS;
      mls[ii] = (sl % S::MNS) ^ S::msw(row);
      const int pr = min(r_wg + row, R - 1);
      const int hr = kvh * a.G + pr % a.G;
      mptr[ii] = (const char*)a.mask_arr +
                 ((int64_t)b * a.ms[0] + (int64_t)hr * a.ms[1] + (int64_t)(pr / a.G) * a.ms[2]) * S::MES +
                 mls[ii] * 16;
    }
  }
  auto dma_m = [&](int blk, int buf) __attribute__((always_inline)) {
    if constexpr (MA != MA_NONE) {
      const int k0 = blk * S::BK;
      const unsigned ml = lds_base + 2 * S::KBYTES + 2 * S::VBYTES + buf * S::MBYTES;
      const int64_t kb = (int64_t)k0 * S::MES;
      const bool tail = k0 + S::BK > Lk;
      const int lmax = tail ? ((Lk - 1 - k0) * S::MES) >> 4 : S::MNS;
#pragma unroll
      for (int ii = 0; ii < MPW; ++ii) {
        if ((ii + 1) * S::NW > S::MDMA && ii * S::NW + wave_u >= S::MDMA) continue;
        const char* src = mptr[ii] + kb;
        if (tail) src += (int64_t)(min(mls[ii], lmax) - mls[ii]) * 16;
        lds_dma16<false>(src, ml + (ii * S::NW + wave_u) * 1024);
      }
    }
  };

  // Prologue: block 0 goes in flight ahead of the Q loads; block 1 follows
  // once both have landed (see below).
  if (nblk > 0) {
    dma_k(0, 0);
    dma_m(blk(0), 0);
    dma_v(0, 0);
  }

  // ---- Q fragments (B operand of S^T = K Q^T), kept in registers ----
  // (with the dv split, this wave's half of the head dim only)
  //
  // The key-split families without a mask array (decode, short queries:
  // bound by the K/V stream) bring Q in by LDS DMA as well, into the V half
  // of buffer 1, which is idle until block 1's V loads.  The compiler waits
  // for none of these loads, so K(1) can go in flight at once, next to
  // block 0 and Q, instead of after them: the stream's first two blocks
  // overlap (a split of one block has nothing to overlap and loads Q
  // straight into registers).  Q rows of the tile: row-major, 16-byte
  // chunks; rows past the entry's re-read its last one, chunks past the real
  // head dim the row's last real chunk (both are zeroed below).
  constexpr int QROWB = DQK * E::ES;
  constexpr int QBYTES = S::BM * QROWB;
  constexpr bool QDMA_OK = S::STREAM && MA == MA_NONE && E::ES == 2 && NWD == 1 && QBYTES <= S::VBYTES &&
                           QBYTES % 1024 == 0;
  const bool qdma = QDMA_OK && nblk > 1;  // uniform
  frag qf[S::NQSW];
  if constexpr (QDMA_OK) {
    if (qdma) {
      constexpr int QCH = QROWB / 16, QI = QBYTES / 1024, QPW = (QI + S::NW - 1) / S::NW;
      const int qch_valid = a.dqk * E::ES / 16;
      const unsigned ql = lds_base + 2 * S::KBYTES + S::VBYTES;
#pragma unroll
      for (int ii = 0; ii < QPW; ++ii) {
        const int ins = ii * S::NW + wave_u;
        if ((ii + 1) * S::NW > QI && ins >= QI) continue;
        const int slot = ins * 64 + lane;
        const int rr = min(r_wg + slot / QCH, R - 1);
        const int hr = kvh * a.G + rr % a.G;
        const char* src = (const char*)a.q +
                          ((int64_t)b * a.qs[0] + (int64_t)hr * a.qs[1] + (int64_t)(rr / a.G) * a.qs[2]) * E::ES +
                          min(slot % QCH, qch_valid - 1) * 16;
        lds_dma16<false>(src, ql + ins * 1024);
      }
      dma_k(1, 1);
      // K(0), V(0) and Q have landed once no more than this wave's K(1) loads
      // remain (its count rounded down: waves with one more wait for it too)
      wait_vmcnt<S::KDMA / S::NW>();
      __syncthreads();
      const SDPA_LDS char* qt = smem + 2 * S::KBYTES + S::VBYTES + (wq * 32 + col) * QROWB;
#pragma unroll
      for (int s = 0; s < S::NQSW; ++s) {
        const int d = s * E::KQK + hl * E::EPL;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (row_ok && d < a.dqk) v = *(const SDPA_LDS u32x4*)(qt + d * 2);
        qf[s] = v;
      }
    }
  }
  if (!qdma) {
    const char* qrow = (const char*)a.q +
                       ((int64_t)b * a.qs[0] + (int64_t)hq * a.qs[1] + (int64_t)iq * a.qs[2]) * E::ES;
#pragma unroll
    for (int s = 0; s < S::NQSW; ++s) {
      const int d = (wd * S::NQSW + s) * E::KQK + hl * E::EPL;
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
    // Block 0 and the Q loads must have landed.  Waiting for everything
    // here also tells the compiler the Q loads are complete, so it puts no
    // load wait of its own inside the loop (which would also stall on the
    // DMA in flight there).
    wait_vmcnt<0>();
  }

  // The loop below assumes a positive scale.  A negative one is folded into
  // Q (negating a rounded value is exact): s * c = (-s) * (-c).  A zero scale
  // makes every visible key equally likely: Q = 0 with scale 1 gives exactly
  // that, and masked keys still reach -inf.
  float c = a.c;
  float sn = a.scale;  // the same factor in natural-log units
  if (c < 0.f) {
    c = -c;
    sn = -sn;
#pragma unroll
    for (int s = 0; s < S::NQSW; ++s) {
      if constexpr (E::ES == 2) qf[s] ^= 0x80008000u;
      else qf[s] = -qf[s];
    }
  } else if (c == 0.f) {
    c = 1.f;
    sn = 1.f;
#pragma unroll
    for (int s = 0; s < S::NQSW; ++s) {
      if constexpr (E::ES == 2) qf[s] = u32x4{0u, 0u, 0u, 0u};
      else qf[s] = 0.f;
    }
  }
  // Factor from the scores in the accumulators to log2 units.  An additive
  // mask is added in natural-log units (s scale + m, one fma), after which
  // the factor is log2 e.
  const float cs = MA == MA_ADD ? kLog2e : c;

  // Loop-invariant parts of the LDS operand addresses (16-bit types).  The
  // K swizzle only involves the lane's row inside a 32-key tile and the V
  // swizzle only the lane bits of the row, so per block every read is one
  // register plus a constant.
  constexpr int SPG = S::KG / 2;  // head-dim steps per K swizzle group
  constexpr int TPG = S::VG / 4;  // dv tiles per V swizzle group
  int koffl[SPG], voffl[TPG];
  if constexpr (E::ES == 2) {
    const int xk = S::kx(col);
#pragma unroll
    for (int sl = 0; sl < SPG; ++sl)
      koffl[sl] = col * S::KROW + 16 * ((2 * sl + hl) ^ xk) + wd * (S::NQSW / SPG) * 16 * S::KG;
    const int g = lane >> 4, t16 = lane & 15;
    const int x = 2 * (g & 1) + ((t16 & 3) >> 1);
    const int y = S::vy(t16 >> 2);
#pragma unroll
    for (int tl = 0; tl < TPG; ++tl)
      voffl[tl] = (4 * (g >> 1) + (t16 >> 2)) * S::VROW + 16 * ((4 * tl + x) ^ y) + 8 * (t16 & 1);
  }

  f32x16 oacc[S::NDTW];
#pragma unroll
  for (int t = 0; t < S::NDTW; ++t) oacc[t] = f32x16{};
  float m_ref = kNegInf;  // reference max of this row, log2 units (same in both lane halves)
  float l_run = 0.f;      // this lane's share of the row sum (halves add up at the end)

  // Block 1 goes in flight once block 0 and Q have landed (waited for
  // above).  With Q by DMA, K(1) is in flight already and V(1) follows once
  // every wave has read its Q.
  if (qdma) {
    __syncthreads();  // every wave has its Q fragments: V buffer 1 is free
    dma_v(1, 1);
  } else if (nblk > 1) {
    dma_k(1, 1);
    dma_m(blk(1), 1);
    dma_v(1, 1);
  }

  // ---- S^T = K Q^T of one block (this wave's BKW keys) ----
  auto qk = [&](int j, f32x16 (&sacc)[S::NKT]) __attribute__((always_inline)) {
    const SDPA_LDS char* kl = smem + (j & 1) * S::KBYTES;
    if constexpr (S::HOIST_K) {
      // Every K fragment of the block is read before the first product, so
      // the reads overlap each other instead of each product waiting for
      // its own.
      frag kf[S::NKT][S::NQSW];
#pragma unroll
      for (int kt = 0; kt < S::NKT; ++kt) {
        const SDPA_LDS char* ktile = kl + (wk * BKW + kt * 32) * S::KROW;
#pragma unroll
        for (int s = 0; s < S::NQSW; ++s)
          kf[kt][s] = *(const SDPA_LDS u32x4*)(ktile + koffl[s % SPG] + 16 * S::KG * (s / SPG));
      }
#pragma unroll
      for (int kt = 0; kt < S::NKT; ++kt) {
        sacc[kt] = f32x16{};
#pragma unroll
        for (int s = 0; s < S::NQSW; ++s) sacc[kt] = E::mma(kf[kt][s], qf[s], sacc[kt]);
      }
      return;
    }
#pragma unroll
    for (int kt = 0; kt < S::NKT; ++kt) {
      sacc[kt] = f32x16{};
      const SDPA_LDS char* ktile = kl + (wk * BKW + kt * 32) * S::KROW;
#pragma unroll
      for (int s = 0; s < S::NQSW; ++s) {
        frag af;
        if constexpr (E::ES == 2) {
          // chunk (2 s + hl) ^ kx(row) of row col: 8 elements
          af = *(const SDPA_LDS u32x4*)(ktile + koffl[s % SPG] + 16 * S::KG * (s / SPG));
        } else {
          const int d = 2 * s + hl;
          af = *(const SDPA_LDS float*)(ktile + col * S::KROW + (((d >> 2) ^ S::kx(col)) << 4) + (d & 3) * 4);
        }
        sacc[kt] = E::mma(af, qf[s], sacc[kt]);
      }
    }
  };

  // V operand of the PV product for key tile kt, key step s2, dv tile t.
  auto vread = [&](int j, int kt, int s2, int t) __attribute__((always_inline)) -> frag {
    const SDPA_LDS char* vl = smem + 2 * S::KBYTES + (j & 1) * S::VBYTES;
    const int kbase_t = wk * BKW + kt * 32;  // first key of this tile inside the block
    if constexpr (E::ES == 2) {
      // Transposing read: lane t16 of group g supplies the address of 4 dv
      // values of one key; the hardware hands lane i of the group element
      // i%4 of the chunk addressed by lane 4j + i/4, i.e. the 4 keys
      // (j = 0..3) of dv column 16*(g%2) + i.
      const SDPA_LDS char* vb = vl + (kbase_t + 16 * s2) * S::VROW + voffl[t % TPG] + 16 * S::VG * (t / TPG);
      const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SDPA_LDS i16x4*)vb);
      const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SDPA_LDS i16x4*)(vb + 8 * S::VROW));
      const u32x2 h0 = __builtin_bit_cast(u32x2, v0), h1 = __builtin_bit_cast(u32x2, v1);
      u32x4 f;
      f[0] = h0[0];
      f[1] = h0[1];
      f[2] = h1[0];
      f[3] = h1[1];
      return f;
    } else {
      const int row = kbase_t + 8 * (s2 >> 2) + 4 * hl + (s2 & 3);
      const int dv = 32 * t + col;
      const int cc = (dv >> 2) ^ S::vy(row);
      return *(const SDPA_LDS float*)(vl + row * S::VROW + cc * 16 + (dv & 3) * 4);
    }
  };

  // ---- does a boolean mask array keep any key of block j for these rows? ----
  // A block the array removes entirely adds nothing to the softmax: the wave
  // skips its products and exponentials.  Reads the same elements as
  // mask_max below; wave-uniform.  Always true otherwise: additive arrays are
  // mostly dense biases, for which the check would only cost time.
  auto mask_live = [&](int j) __attribute__((always_inline)) -> bool {
    if constexpr (MA != MA_BOOL) {
      return true;
    } else {
      const int mrow = wq * 32 + col;
      const SDPA_LDS char* mt = smem + 2 * S::KBYTES + 2 * S::VBYTES + (j & 1) * S::MBYTES + mrow * S::MROWB;
      const int sw = S::msw(mrow);
      bool keep = false;
#pragma unroll
      for (int kt = 0; kt < S::NKT; ++kt) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int byte = (wk * BKW + kt * 32 + 8 * g + 4 * hl) * S::MES;
          const SDPA_LDS char* pa = mt + (((byte >> 4) ^ sw) << 4) + (byte & 15);
          keep |= *(const SDPA_LDS unsigned*)pa != 0u;
        }
      }
      return __builtin_amdgcn_ballot_w64(keep) != 0;
    }
  };

  // ---- edge blocks: the diagonal, a window edge, the Lk tail ----
  // (wave-uniform: decided from this wave's first and last row)
  auto edge_of = [&](int j) __attribute__((always_inline)) -> bool {
    const int kw = blk(j) * S::BK + wk * BKW;  // first key of this wave's slice
    return (kw + BKW > Lk) || (a.mask != MASK_NONE && kw + BKW - 1 > pmin_w) ||
           (a.mask == MASK_WINDOW && kw <= pmax_w - a.window);
  };
  // Per-element mask of an edge block: keys outside this row's visible range
  // [lo, hi] go to -inf.  The key of register e in tile kt is
  // kw + 32 kt + 4 hl + off(e) with off(e) = 8 (e / 4) + e % 4.
  auto mask_edge = [&](int j, f32x16 (&sacc)[S::NKT]) __attribute__((always_inline)) {
    const int kw = blk(j) * S::BK + wk * BKW;
    int hi = Lk - 1, lo = 0;
    if (a.mask != MASK_NONE) hi = min(hi, pos);
    if (a.mask == MASK_WINDOW) lo = max(lo, pos - a.window + 1);
#pragma unroll
    for (int kt = 0; kt < S::NKT; ++kt) {
      const int base = kw + kt * 32 + 4 * hl;
      const unsigned span = (unsigned)(hi - lo);  // visible iff 0 <= key - lo <= span
      const int first = lo - base;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int off = 8 * (e >> 2) + (e & 3);
        if ((unsigned)(off - first) > span || hi < lo) sacc[kt][e] = kNegInf;
      }
    }
  };
  // Fold the block max into the running max: online softmax with lazy
  // rescaling (scale c > 0); the reference max moves only when the block max
  // exceeds it by more than kRescale.
  auto fold_max = [&](f32x16 (&sacc)[S::NKT]) __attribute__((always_inline)) {
    float mx = kNegInf;
#pragma unroll
    for (int kt = 0; kt < S::NKT; ++kt)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[kt][e]);
    mx = wave_max32(mx);
    const float mxs = mx * cs;  // block max in log2 units (-inf if all masked)
    const bool need = mxs > m_ref + kRescale;
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(need) != 0, 0)) [[unlikely]] {
      const float m_new = need ? mxs : m_ref;
      const float alpha = need ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.0f;
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < S::NDTW; ++t) oacc[t] *= alpha;
      m_ref = m_new;
    }
  };

  // ---- mask edge blocks and fold the block max into the running max ----
  auto mask_max = [&](int j, f32x16 (&sacc)[S::NKT]) __attribute__((always_inline)) {
    if constexpr (MA != MA_NONE) {
      // This lane's row of the block's mask tile: register e of tile kt is
      // key wk BKW + 32 kt + 8 (e / 4) + 4 hl + e % 4 of the block, so each
      // group of 4 registers reads 4 consecutive elements.
      const int mrow = wq * 32 + col;
      const SDPA_LDS char* mt = smem + 2 * S::KBYTES + 2 * S::VBYTES + (j & 1) * S::MBYTES + mrow * S::MROWB;
      const int sw = S::msw(mrow);
#pragma unroll
      for (int kt = 0; kt < S::NKT; ++kt) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int byte = (wk * BKW + kt * 32 + 8 * g + 4 * hl) * S::MES;
          const SDPA_LDS char* pa = mt + (((byte >> 4) ^ sw) << 4) + (byte & 15);
          if constexpr (MA == MA_BOOL) {
            // bytes are 0 or 1: bit 0 of byte t, sign-extended, selects
            // between the score and -inf bit by bit (bfe + bfi)
            const unsigned w = *(const SDPA_LDS unsigned*)pa;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const unsigned keep = (unsigned)((int)(w << (31 - 8 * t)) >> 31);
              // copy out first: a bit cast of a vector element in place
              // reads element 0 with this compiler
              const float sv = sacc[kt][4 * g + t];
              const unsigned sb = __builtin_bit_cast(unsigned, sv);
              sacc[kt][4 * g + t] = __builtin_bit_cast(float, (sb & keep) | (0xFF800000u & ~keep));
            }
          } else {
            float mv[4];
            if constexpr (E::ES == 4) {
              const f32x4 w = *(const SDPA_LDS f32x4*)pa;
              mv[0] = w[0]; mv[1] = w[1]; mv[2] = w[2]; mv[3] = w[3];
            } else {
              const u32x2 w = *(const SDPA_LDS u32x2*)pa;
#pragma unroll
              for (int t = 0; t < 4; ++t) {
                const unsigned short h = (unsigned short)(w[t >> 1] >> (16 * (t & 1)));
                mv[t] = E::to_float(h);
              }
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) sacc[kt][4 * g + t] = __builtin_fmaf(sacc[kt][4 * g + t], sn, mv[t]);
          }
        }
      }
    }
    if (edge_of(j)) mask_edge(j, sacc);
    fold_max(sacc);
  };

  // ---- probabilities of a block against the reference max ----
  auto expo = [&](f32x16 (&sacc)[S::NKT]) __attribute__((always_inline)) {
    const float msub = (m_ref == kNegInf) ? 0.f : m_ref;
#pragma unroll
    for (int kt = 0; kt < S::NKT; ++kt) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kt][e], cs, -msub));
        sacc[kt][e] = p;
        l_run += p;
      }
    }
  };

  // ---- O^T += V^T P^T of block j (V fragments optionally read ahead) ----
  using vfrag_t = frag[S::HOIST_V ? S::NKT : 1][S::HOIST_V ? 32 / E::KPV : 1][S::HOIST_V ? S::NDT : 1];
  auto vhoist = [&](int j, vfrag_t& vf) __attribute__((always_inline)) {
    if constexpr (S::HOIST_V) {
#pragma unroll
      for (int kt = 0; kt < S::NKT; ++kt)
#pragma unroll
        for (int s2 = 0; s2 < 32 / E::KPV; ++s2)
#pragma unroll
          for (int t = 0; t < S::NDT; ++t) vf[kt][s2][t] = vread(j, kt, s2, t);  // NWD == 1 here
    }
  };
  auto pv = [&](int j, f32x16 (&sacc)[S::NKT], vfrag_t& vf) __attribute__((always_inline)) {
#pragma unroll
    for (int kt = 0; kt < S::NKT; ++kt) {
#pragma unroll
      for (int s2 = 0; s2 < 32 / E::KPV; ++s2) {
        frag bf;
        if constexpr (E::ES == 2) {
          u32x4 pk;
#pragma unroll
          for (int w = 0; w < 4; ++w) pk[w] = E::pack2(sacc[kt][8 * s2 + 2 * w], sacc[kt][8 * s2 + 2 * w + 1]);
          bf = pk;
        } else {
          bf = sacc[kt][s2];
        }
#pragma unroll
        for (int t = 0; t < S::NDTW; ++t) {
          if constexpr (S::HOIST_V) oacc[t] = E::mma(vf[kt][s2][t], bf, oacc[t]);
          else oacc[t] = E::mma(vread(j, kt, s2, tw0 + t), bf, oacc[t]);
        }
      }
    }
  };

  if constexpr (!S::PIPE) {
    // Block j sits in buffer pair j % 2.  Iteration j waits for block j
    // (block j + 1 stays in flight), computes it, and sends block j + 2 to
    // the same pair as soon as every wave is done with each half: K right
    // after the QK products, V after the PV products.  So the next block is
    // always in flight during the compute and two are while the wave waits:
    // the stream never drains between blocks.  (Where two blocks would
    // overflow the 63-entry vector-memory counter, K waits for the end too
    // and part of block j + 1 lands first.)
    constexpr bool KEARLY = 2 * S::DMA_MAX <= 63;
    static_assert(NWD == 1 || KEARLY, "the dv split's score exchange uses the barrier after QK");
    f32x16 sacc[S::NKT];
    bool live_prev = true;
    // A wave whose 32 rows all lie past the packed rows (a short query set
    // in a multi-wave row tile) only helps with the loads.
    const bool wave_rows = r_wave < R;
    for (int j = 0; j < nblk; ++j) {
      if (j + 1 < nblk) wait_vmcnt<S::DMA_MIN>();  // only block j + 1 may still be in flight
      else wait_vmcnt<0>();
      __syncthreads();  // every wave's share of block j has landed
      // A boolean array's block is checked every 4th block while blocks are
      // live and at every block after a removed one: dense masks pay for a
      // quarter of the checks, a live run costs at most 3 unchecked blocks.
      bool live = wave_rows;
      if (MA == MA_BOOL && wave_rows && (!live_prev || (j & 3) == 0)) live = mask_live(j);
      live_prev = live;
      if (live) qk(j, sacc);
      if constexpr (NWD > 1) {
        // dv split: this wave's scores cover half of the head dim; leave
        // them for the other wave of the pair (same rows, same keys, same
        // register layout), whose half comes back after the barrier.
        if (live) {
          SDPA_LDS char* xw = smem + S::XOFF + wave * 4096 + lane * 16;
#pragma unroll
          for (int c = 0; c < 4; ++c)
            *(SDPA_LDS f32x4*)(xw + c * 1024) =
                f32x4{sacc[0][4 * c], sacc[0][4 * c + 1], sacc[0][4 * c + 2], sacc[0][4 * c + 3]};
        }
      }
      if constexpr (KEARLY) {
        if (NWD > 1 || j + 2 < nblk) {
          __syncthreads();  // every wave is done with K(j) (and the partial scores are in LDS)
          if (j + 2 < nblk) dma_k(j + 2, j & 1);
        }
      }
      if constexpr (NWD > 1) {
        if (live) {
          // the same sum in both waves of the pair: a + b = b + a exactly
          const SDPA_LDS char* xr = smem + S::XOFF + (wave ^ (NWQ * NWK)) * 4096 + lane * 16;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const f32x4 o = *(const SDPA_LDS f32x4*)(xr + c * 1024);
#pragma unroll
            for (int i = 0; i < 4; ++i) sacc[0][4 * c + i] += o[i];
          }
        }
      }
      if (live) {
        vfrag_t vf;
        vhoist(j, vf);  // in flight during the softmax
        mask_max(j, sacc);
        expo(sacc);
        pv(j, sacc, vf);
      }
      if (j + 2 < nblk) {
        if constexpr (!KEARLY) wait_vmcnt<63 - S::DMA_MAX>();
        __syncthreads();  // every wave is done with V(j) and the mask tile of j
        if constexpr (!KEARLY) dma_k(j + 2, j & 1);
        dma_m(blk(j + 2), j & 1);
        dma_v(j + 2, j & 1);
      }
    }
  } else {
    // Software-pipelined loop: the QK products of block j + 1 are issued
    // between the exponentials of block j and its PV products, so the
    // matrix cores work while the vector unit computes probabilities (inside
    // one block the products wait for the probabilities, so only a
    // neighbouring block's products can run beside them).  K runs two blocks
    // ahead of V: K(j + 1) and V(j) are consumed in step j, after which
    // their buffers take K(j + 3) and V(j + 2).  Step j waits for K(j + 1)
    // and V(j); what may still be in flight is K(j + 2) and V(j + 1).
    f32x16 sa[S::NKT], sb[S::NKT];
    bool live_cur = true;  // the mask array keeps a key of the block in `cur`
    if (nblk > 0) {
      __syncthreads();  // block 0 (waited for above) is visible to every wave
      live_cur = mask_live(0);
      qk(0, sa);
      mask_max(0, sa);
      if (nblk > 2) {
        __syncthreads();  // every wave is done with K(0) and the mask tile of 0
        dma_k(2, 0);
        dma_m(blk(2), 0);
      }
    }
    // `more` (block j + 1 exists) is a literal at every call, so the
    // compute of a step is one branch-free stretch the scheduler can
    // interleave.
    auto step = [&](int j, f32x16 (&cur)[S::NKT], f32x16 (&nxt)[S::NKT], const bool more)
        __attribute__((always_inline)) {
      if (j + 2 < nblk) wait_vmcnt<S::DMA_MIN>();
      else if (more) wait_vmcnt<S::VDMA / S::NW>();
      else wait_vmcnt<0>();
      __syncthreads();  // K(j + 1) and V(j) have landed for every wave
      // The products of block j + 1 always run (they overlap this block's
      // exponentials); whether the array keeps any of its keys is read here
      // and decides, in the next step, whether its exponentials and PV
      // products run.  Constant true without a boolean array.
      // (checked as in the plain loop: every 4th block, or after a removed one)
      bool ln = true;
      if (MA == MA_BOOL && more && (!live_cur || ((j + 1) & 3) == 0)) ln = mask_live(j + 1);
      if constexpr (MA == MA_NONE && DQK <= 64 && DV <= 64) {
        // Small head dims without a mask array: the step is one straight
        // stretch of code, so the scheduler can put the next block's max and
        // the row sums beside the matrix products.  Whether block j + 1 needs
        // the per-element mask is decided first, and each case has its own
        // copy of the step (at larger head dims the two copies no longer fit
        // the register file).
        auto body = [&](auto EDGE) __attribute__((always_inline)) {
          vfrag_t vf;
          vhoist(j, vf);
          expo(cur);
          if (more) qk(j + 1, nxt);
          pv(j, cur, vf);
          if (more) {
            if constexpr (decltype(EDGE)::value) mask_edge(j + 1, nxt);
            fold_max(nxt);
          }
        };
        if (more && edge_of(j + 1)) body(std::true_type{});
        else body(std::false_type{});
      } else if (MA != MA_BOOL || live_cur) {
        // Large head dims: ask the scheduler to interleave the exponentials
        // with the matrix products (one of LLVM's fixed interleaving
        // strategies for exponential-plus-MFMA code; measured 5-12% faster
        // on the D=256 prefill workloads, none better at the small dims).
        if constexpr (DQK >= 192 && DV >= 192 && MA == MA_NONE) __builtin_amdgcn_iglp_opt(3);
        vfrag_t vf;
        vhoist(j, vf);
        expo(cur);
        if (more) qk(j + 1, nxt);
        pv(j, cur, vf);
        if (more) mask_max(j + 1, nxt);
      } else {
        if (more) {
          qk(j + 1, nxt);
          mask_max(j + 1, nxt);
        }
      }
      live_cur = ln;
      if (j + 2 < nblk) {
        __syncthreads();  // every wave is done with K(j + 1), its mask tile and V(j)
        if (j + 3 < nblk) {
          dma_k(j + 3, (j + 1) & 1);
          dma_m(blk(j + 3), (j + 1) & 1);
        }
        dma_v(j + 2, j & 1);
      }
    };
    int j = 0;
    for (; j + 2 < nblk; j += 2) {
      step(j, sa, sb, true);
      step(j + 1, sb, sa, true);
    }
    if (j + 1 < nblk) {
      step(j, sa, sb, true);
      step(j + 1, sb, sa, false);
    } else if (j < nblk) {
      step(j, sa, sb, false);
    }
  }

  // ---- epilogue ----
  float l_row = wave_sum32(l_run);  // both halves' keys

  if constexpr (NWK > 1) {
    // Merge the NWK key slices of the same rows once every wave is done with
    // the tile buffers: waves wk > 0 leave their partial (m, l, O) in LDS,
    // wave wk == 0 folds them into its own registers.
    SDPA_LDS float* mml = (SDPA_LDS float*)smem;            // [MSLOTS][32][2]
    SDPA_LDS float* mo = (SDPA_LDS float*)(smem + S::MLB);  // [MSLOTS][32][MROW]
    const int slot = wq * (NWK - 1) + (wk - 1);
    __syncthreads();
    if (wk > 0 && hl == 0) {
      mml[(slot * 32 + col) * 2 + 0] = m_ref;
      mml[(slot * 32 + col) * 2 + 1] = l_row;
    }
    __syncthreads();
    float sc[NWK];  // weight of each slice's partial in the merged row
    if (wk == 0) {
      float M = m_ref;
#pragma unroll
      for (int w = 1; w < NWK; ++w) M = fmaxf(M, mml[((wq * (NWK - 1) + w - 1) * 32 + col) * 2]);
      const float Mu = (M == kNegInf) ? 0.f : M;
      sc[0] = __builtin_amdgcn_exp2f(m_ref - Mu);
      l_row *= sc[0];
#pragma unroll
      for (int w = 1; w < NWK; ++w) {
        const int sl = (wq * (NWK - 1) + w - 1) * 32 + col;
        sc[w] = __builtin_amdgcn_exp2f(mml[sl * 2] - Mu);
        l_row += sc[w] * mml[sl * 2 + 1];
      }
#pragma unroll
      for (int t = 0; t < S::NDT; ++t) oacc[t] *= sc[0];
      m_ref = M;
    }
#pragma unroll
    for (int t0 = 0; t0 < S::NDT; t0 += S::TPR) {
      if (t0 > 0) __syncthreads();  // the previous round has been read
      if (wk > 0) {
        SDPA_LDS float* myo = mo + (slot * 32 + col) * S::MROW;
#pragma unroll
        for (int t = 0; t < S::TPR; ++t) {
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const int d = t * 32 + 8 * i4 + 4 * hl;
            *(SDPA_LDS f32x4*)(myo + d) = f32x4{oacc[t0 + t][4 * i4 + 0], oacc[t0 + t][4 * i4 + 1],
                                                oacc[t0 + t][4 * i4 + 2], oacc[t0 + t][4 * i4 + 3]};
          }
        }
      }
      __syncthreads();
      if (wk == 0) {
#pragma unroll
        for (int w = 1; w < NWK; ++w) {
          const SDPA_LDS float* po = mo + ((wq * (NWK - 1) + w - 1) * 32 + col) * S::MROW;
#pragma unroll
          for (int t = 0; t < S::TPR; ++t) {
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
              const f32x4 v4 = *(const SDPA_LDS f32x4*)(po + t * 32 + 8 * i4 + 4 * hl);
              oacc[t0 + t][4 * i4 + 0] += sc[w] * v4[0];
              oacc[t0 + t][4 * i4 + 1] += sc[w] * v4[1];
              oacc[t0 + t][4 * i4 + 2] += sc[w] * v4[2];
              oacc[t0 + t][4 * i4 + 3] += sc[w] * v4[3];
            }
          }
        }
      }
    }
    if (wk > 0) return;
  }

  if (!row_ok) return;
  if (a.splits == 1) {
    // l = 0 only for a row left without keys (by a mask array or its
    // entry's lengths): it writes 0 and lse = -inf
    const float inv = l_row > 0.f ? 1.0f / l_row : 0.f;
    char* orow = (char*)a.o + ((int64_t)b * a.os[0] + (int64_t)hq * a.os[1] + (int64_t)iq * a.os[2]) * E::ES;
#pragma unroll
    for (int t = 0; t < S::NDTW; ++t) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = (tw0 + t) * 32 + 8 * i4 + 4 * hl;
        if (d < a.dv) {
          if constexpr (E::ES == 2) {
            u32x2 w;
            w[0] = E::pack2(oacc[t][4 * i4 + 0] * inv, oacc[t][4 * i4 + 1] * inv);
            w[1] = E::pack2(oacc[t][4 * i4 + 2] * inv, oacc[t][4 * i4 + 3] * inv);
            *(u32x2*)(orow + d * 2) = w;
          } else {
            *(float4*)(orow + d * 4) = make_float4(oacc[t][4 * i4 + 0] * inv, oacc[t][4 * i4 + 1] * inv,
                                                   oacc[t][4 * i4 + 2] * inv, oacc[t][4 * i4 + 3] * inv);
          }
        }
      }
    }
    if (a.lse && hl == 0 && wd == 0) a.lse[((int64_t)b * a.Hq + hq) * a.Lq + iq] = (m_ref + log2f(l_row)) * kLn2;
    return;
  }

  // ---- split plan: this split's partial (O, m, l) ----
  // partial row: [z][r][split], or with balanced lengths the entry's segment
  // [seg R, (seg + nsp) R) of its KV head, laid out [r][split]
  const int64_t ws_row = a.kv_balance > 0 ? seg * a.R + (int64_t)r * nsp + split
                                          : ((int64_t)z * a.R + r) * a.splits + split;
  float* wo = a.ws_o + ws_row * a.dv;
#pragma unroll
  for (int t = 0; t < S::NDTW; ++t) {
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d = (tw0 + t) * 32 + 8 * i4 + 4 * hl;
      if (d < a.dv)
        *(float4*)(wo + d) = make_float4(oacc[t][4 * i4 + 0], oacc[t][4 * i4 + 1], oacc[t][4 * i4 + 2],
                                         oacc[t][4 * i4 + 3]);
    }
  }
  if (hl == 0 && wd == 0) *(float2*)(a.ws_ml + ws_row * 2) = make_float2(m_ref, l_row);
}

}  // namespace dev
}  // namespace sdpa
