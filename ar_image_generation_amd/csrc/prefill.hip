// band_prefill_attn: causal, keep-set-masked attention over whole sequences,
// bf16 in, fp32 accumulation, on the matrix cores (v_mfma_f32_16x16x32_bf16).
//
// Workgroup = 4 waves = 128 query rows of one (batch, head); wave w owns
// the 16-row blocks w and w + 4 (64 rows apart).  The 64-key tiles that hold
// a kept pair (listed once per query tile by prefill_tiles_kernel) stream K
// and V into a two-stage LDS ring by direct global->LDS copies, the next
// tile in flight while the current one is computed.  A workgroup takes at
// most 80 KiB of LDS, so two share a CU: while one waits at its per-tile
// barrier the other's matrix work keeps the CU busy.  Scores are computed
// transposed, S^T = K Q^T (A = K from LDS, B = Q^T from registers), so that
// the MFMA result gives every lane one query row and four keys of each
// 16-key block.  That lane-per-row layout is kept for the
// whole softmax: the running max/sum are per lane (combined over the four
// lanes of a row by lane swaps), the probabilities P^T are already in the B
// operand layout of the second product, and the output is accumulated
// transposed, O^T += V^T P^T (A = V^T by transposing LDS reads of row-major
// V), so the online rescale is one multiply per lane register.
//
// Sparsity: only listed key tiles are visited.  Keys below the prompt end
// come in tiles on multiples of 64, keys past it in window tiles aligned so
// that each 16-row block's kept run on a diagonal starts on a 16-key block
// of the tile.  A tile in which every wave's two row blocks hold their kept
// pairs in at most two of its four 16-key blocks is computed on those two
// only (half the products, exponentials and LDS operand reads); with the
// row blocks 64 rows apart, raster widths dividing 64 make the two row
// blocks meet the same diagonal runs, so window tiles are such tiles.  A
// wave none of whose rows keeps a key of the tile only takes part in the
// copies and barriers; a wave whose blocks are all wholly kept applies no
// mask; otherwise each row gets a 64-bit keep word over the tile's keys
// (causal, prompt and window bits) and every score keeps its bit or becomes
// -inf.
// (Skipping single 16x16 blocks inside a wave behind uniform branches
// measured slower: it breaks the interleaving of the unrolled products.)
// Workgroups are numbered so that all query tiles of one (batch, head)
// share an XCD (hardware deals workgroups to the 8 XCDs round-robin), which
// keeps the prompt keys/values every tile re-reads in that XCD's L2, and so
// that the last query tiles -- the longest under a causal mask -- start
// first.
#include "common.h"

#include <type_traits>

namespace da {


struct PrefillArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;                       // [batch][heads][n] or null
  int64_t sq[3], sk[3], sv[3], so[3];   // element strides (batch, head, position)
  const int32_t* prompt_len;        // [batch]
  const int32_t* tile_count;        // [batch][n_qt]
  const int4* tile_list;            // [batch][n_qt][max_tiles][2]: (key tile, need lo, need hi, 0),
                                    // (full lo, full hi, 0, 0)
  int batch, heads, kv_heads, n, n_qt, max_tiles;
  int mode, W, B, G;
  float qscale;                     // scale * log2(e)
  float inv_g;                      // 1 / G
};

// Query tile: NWAVE waves x RB_MAX row blocks of 16 rows (wave w: blocks w,
// w + NWAVE); key tile: BN keys.
constexpr int RB_MAX = 2;
constexpr int NWAVE = 4;
static_assert(NWAVE * 8 <= 32, "the LDS list keeps 8 full-block bits per wave in 32 bits");
constexpr int BM_ROWS = NWAVE * 16 * RB_MAX;
constexpr int NTHREADS = NWAVE * 64;

constexpr int BN = 64;              // keys per tile
constexpr float kLog2eP = 1.4426950408889634f;
constexpr float kLn2P = 0.6931471805599453f;

// Does any pair (i, j), i in [ilo, ihi], j in [jlo, jhi], pass the causal
// keep rule?  (Exact; used to skip tiles and blocks.)
__device__ inline bool range_has_kept(int ilo, int ihi, int jlo, int jhi, int P, int mode, int W,
                                      int B, int G) {
  if (jlo > ihi) return false;                   // causal
  if (mode == DA_MODE_DENSE) return true;
  if (jlo < P) return true;                      // a prompt key under the diagonal
  const int dlo = ilo - jhi > 0 ? ilo - jhi : 0;
  const int dhi = ihi - jlo < W ? ihi - jlo : W;
  if (dlo > dhi) return false;
  if (mode == DA_MODE_BAND) return dlo <= B;
  if (2 * (int64_t)B + 1 >= G) return true;
  const int r = dlo % G;
  if (r <= B || r >= G - B) return true;
  return dlo - r + G - B <= dhi;                 // next band start
}

// Is every pair in the range kept (no element mask needed)?
__device__ inline bool range_all_kept(int ilo, int jhi, int P, int mode) {
  if (jhi > ilo) return false;                   // causal: every key <= every row
  return mode == DA_MODE_DENSE || jhi < P;
}

// s_waitcnt immediate that waits until at most n vector-memory operations
// of this wave are outstanding (expcnt and lgkmcnt left unconstrained).
constexpr int vmcnt_imm(int n) { return (n & 0xf) | ((n >> 4) << 14) | (0x7 << 4) | (0xf << 8); }

// Non-negative x mod G through a float reciprocal (exact for |x| < 2^22).
__device__ inline int mod_g(int x, int G, float inv_g) {
  int r = x - G * (int)floorf((float)x * inv_g);
  r += r < 0 ? G : 0;
  r -= r >= G ? G : 0;
  return r;
}

// Bits lo..hi of a 64-bit word, clipped to 0..63; 0 when the range is empty.
__device__ inline uint64_t bit_range(int lo, int hi) {
  lo = lo < 0 ? 0 : lo;
  hi = hi > 63 ? 63 : hi;
  const int len = hi - lo;
  const uint64_t m = (~uint64_t(0) >> (63 - (len < 0 ? 0 : len))) << (lo > 63 ? 0 : lo);
  return len < 0 ? 0 : m;
}

// Largest raster width the row-diagonal prefill supports: its band pattern
// (one 64-bit word per residue mod G) lives in LDS.
constexpr int GMAX = 1016;

// Sequences of up to 64 * MAX_LIST tokens.  A query tile lists at most
// ceil(n / 64) + 3 key tiles: prompt tiles below the prompt end, window
// tiles from at most 15 keys before it (LDS copy, 8 bytes an entry; with
// the ring and the band pattern a workgroup stays within 80 KiB, so two
// share a CU).
constexpr int MAX_LIST = 1024;
constexpr int LIST_EXTRA = 3;
constexpr int LIST_CAP = MAX_LIST + LIST_EXTRA;

// A tile's copies global -> LDS (global_load_lds_dwordx4: lane l's 16
// bytes land at M0 + 16 l), K and V alternating, DPW of each for this
// wave.  Issued as one block of inline assembly so that the compiler does
// not treat them as pending LDS writes that every later LDS read must wait
// for: the ring's own waits (vmcnt + barrier) order the stages.  Each
// address is a uniform 64-bit base (SGPRs) plus the lane's 32-bit byte
// offset, so the copies need no per-lane address arithmetic.  The
// compiler's hazard checks do not see inside the block, so it carries its
// own wait states: 5 before the first copy (a VALU write of any SGPR
// operand, 5 before a memory instruction reads it) and 1 after each M0
// write (SALU write of M0, 1 before an LDS DMA).
__device__ inline const void* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  return (const void*)(uintptr_t)(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32)) << 32) |
                                  (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v));
}
#define DA_DMA_PAIR(u)                                                        \
  "s_mov_b32 m0, %[mk" #u "]\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[k" #u "], %[kb]\n\t" \
  "s_mov_b32 m0, %[mv" #u "]\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[v" #u "], %[vb]\n\t"
template <int DPW>
__device__ inline void dma_tile(const void* kbase, const void* vbase, const uint32_t (&ko)[DPW],
                                const uint32_t (&vo)[DPW], uint32_t lk, uint32_t lv) {
  static_assert(DPW == 2 || DPW == 4, "2 or 4 copies of K and of V a wave");
  if constexpr (DPW == 4) {
    __asm__ volatile("s_nop 4\n\t" DA_DMA_PAIR(0) DA_DMA_PAIR(1) DA_DMA_PAIR(2) DA_DMA_PAIR(3)
                     :
                     : [kb] "s"(kbase), [vb] "s"(vbase), [k0] "v"(ko[0]), [k1] "v"(ko[1]), [k2] "v"(ko[2]),
                       [k3] "v"(ko[3]), [v0] "v"(vo[0]), [v1] "v"(vo[1]), [v2] "v"(vo[2]), [v3] "v"(vo[3]),
                       [mk0] "s"(lk), [mk1] "s"(lk + 1024), [mk2] "s"(lk + 2048), [mk3] "s"(lk + 3072),
                       [mv0] "s"(lv), [mv1] "s"(lv + 1024), [mv2] "s"(lv + 2048), [mv3] "s"(lv + 3072)
                     : "memory", "m0");
  } else {
    __asm__ volatile("s_nop 4\n\t" DA_DMA_PAIR(0) DA_DMA_PAIR(1)
                     :
                     : [kb] "s"(kbase), [vb] "s"(vbase), [k0] "v"(ko[0]), [k1] "v"(ko[1]), [v0] "v"(vo[0]),
                       [v1] "v"(vo[1]), [mk0] "s"(lk), [mk1] "s"(lk + 1024), [mv0] "s"(lv), [mv1] "s"(lv + 1024)
                     : "memory", "m0");
  }
}
#undef DA_DMA_PAIR

// K and V tiles sit in LDS row-major with 16-byte chunk p of row r at
// position p ^ swz(r) (common.h), so that neither the K operand reads nor
// the transposing V reads meet a bank conflict.

// ---------------------------------------------------------------- tile lists
// For query tile qt of batch b: the key tiles (BN keys) holding a kept pair,
// each with two 64-bit masks over (wave, row block, 16-key block) -- bit
// w*8 + rb*4 + kq: that block has a kept pair / every pair is kept.  Two
// grids of key tiles:
//  * prompt tiles at multiples of BN, for keys below the prompt end (DENSE:
//    every key), masked by the causal rule alone;
//  * window tiles for keys at or past the prompt end, starting on keys
//    congruent to i0 - B mod 16.  A 16-row block at rows r0..r0+15 keeps, on
//    the diagonal k G of its window, the keys r0 - kG - B .. r0 - kG + 15 + B
//    (causal: up to r0 - kG + 15), so with that alignment the run starts on a
//    16-key block of the tile and, for B <= 8, fills at most two blocks.
// A tile in which every wave's rows (row blocks w and w + 4, 64 rows apart)
// need at most two of the four key blocks is a "half" tile: each wave
// computes only those two blocks, shared by its row blocks, at half the
// matrix, softmax and LDS-read work.  The list holds the whole tiles
// first, then the half tiles, so that the attention kernel runs them in two
// loops (the order of the online softmax's steps does not change its
// result beyond rounding).
// One wave per (b, qt); lane = candidate key tile; a ballot keeps the order.
__global__ void __launch_bounds__(64) prefill_tiles_kernel(PrefillArgs a) {
  const int lane = threadIdx.x;
  const int b = blockIdx.x / a.n_qt;
  const int qt = blockIdx.x % a.n_qt;
  const int n = a.n;
  const int P = clampi(a.prompt_len[b], 0, n);
  const int i0 = qt * BM_ROWS;
  const int i_last = i0 + BM_ROWS - 1 < n - 1 ? i0 + BM_ROWS - 1 : n - 1;
  const bool dense = a.mode == DA_MODE_DENSE;
  int4* out = const_cast<int4*>(a.tile_list) + ((int64_t)b * a.n_qt + qt) * a.max_tiles * 2;
  // prompt grid: keys below pe
  const int pe = dense ? i_last + 1 : (P < i_last + 1 ? P : i_last + 1);
  const int n_pro = (pe + BN - 1) / BN;
  // window grid: tiles from wb (congruent to i0 - B mod 16, at most 15
  // before the first key past the prompt a row of the tile can keep)
  // through the last row
  int n_win = 0, wb = 0;
  if (!dense) {
    const int reach = a.mode == DA_MODE_BAND ? (a.B < a.W ? a.B : a.W) : a.W;
    const int wlo = i0 - reach > P ? i0 - reach : P;
    wb = wlo - ((wlo - (i0 - a.B)) & 15);
    n_win = wlo <= i_last ? (i_last - wb) / BN + 1 : 0;
  }
  int count = 0, n_whole = 0;
  for (int pass = 0; pass < 2; ++pass) {        // whole tiles, then half tiles
    for (int base = 0; base < n_pro + n_win; base += 64) {
      const int c = base + lane;
      const bool win = c >= n_pro;
      const int j0 = win ? wb + (c - n_pro) * BN : c * BN;
      uint64_t need = 0, full = 0;
      bool half = true;                          // every wave needs <= 2 key blocks
      if (c < n_pro + n_win) {
        for (int w = 0; w < NWAVE; ++w) {
          unsigned uni = 0;                        // key blocks any of the wave's rows needs
          for (int rb = 0; rb < RB_MAX; ++rb) {
            const int rlo = i0 + w * 16 + rb * NWAVE * 16;
            if (rlo > i_last) continue;
            const int rhi = rlo + 15 < i_last ? rlo + 15 : i_last;
            for (int kq = 0; kq < 4; ++kq) {
              const int jlo = j0 + 16 * kq, jhi = jlo + 15;
              const uint64_t bit = uint64_t(1) << (w * 8 + rb * 4 + kq);
              bool has, all;
              if (!win) {
                has = jlo <= rhi && (dense || jlo < P);
                all = rhi == rlo + 15 && jhi <= rlo && (dense || jhi < P);
              } else {
                const int jl = jlo > P ? jlo : P;
                has = jl <= jhi && range_has_kept(rlo, rhi, jl, jhi, P, a.mode, a.W, a.B, a.G);
                all = false;
              }
              if (has) { need |= bit; uni |= 1u << kq; }
              if (all) full |= bit;
            }
          }
          half = half && __popc(uni) <= 2;
        }
      }
      const bool keep = need != 0 && half == (pass == 1);
      const uint64_t bal = __ballot(keep);
      const int slot = count + __popcll(bal & ((uint64_t(1) << lane) - 1));
      if (keep && slot < a.max_tiles) {
        full &= need;
        out[2 * slot] = make_int4(j0, (int)(uint32_t)need, (int)(uint32_t)(need >> 32), win ? 1 : 0);
        out[2 * slot + 1] = make_int4((int)(uint32_t)full, (int)(uint32_t)(full >> 32), 0, 0);
      }
      count += __popcll(bal);
    }
    if (pass == 0) n_whole = count;
  }
  count = count < a.max_tiles ? count : a.max_tiles;
  n_whole = n_whole < count ? n_whole : count;
  if (lane == 0) const_cast<int32_t*>(a.tile_count)[(int64_t)b * a.n_qt + qt] = count | (n_whole << 16);
}

// ---------------------------------------------------------------- attention
template <int HD, int MODE>
__global__ void __launch_bounds__(NTHREADS) __attribute__((amdgpu_waves_per_eu(2))) prefill_kernel(PrefillArgs a) {
  constexpr int RB = RB_MAX;
  constexpr int NC = HD / 32;          // 32-wide contraction chunks of the head dim
  constexpr int NB = HD / 16;          // 16-wide output blocks of the head dim
  constexpr int CPR = HD / 8;          // 16-byte chunks per key row
  constexpr int RPI = 64 / CPR;        // key rows per 1 KiB wave transfer
  constexpr int TILE = BN * HD;        // elements of one K (or V) tile
  constexpr int DPW = BN * CPR / NTHREADS;  // 1 KiB transfers per wave per tile, K (same for V)
  constexpr int NS = 2;                // LDS ring stages: current tile, next tile

  // ring of NS stages, each a K tile then a V tile, row-major, 16-byte
  // chunk p of row r holding the row's chunk p ^ swz(r) (bank spreading)
  __shared__ __attribute__((aligned(1024))) uint16_t ring[NS * 2 * TILE];
  // row-diagonal band pattern: bit c of bp[r] says whether a key c places
  // before a query at residue r (mod G) lies within B of a multiple of G
  __shared__ uint64_t bp[MODE == DA_MODE_ROWDIAG ? GMAX : 1];
  // this query tile's list, read from LDS so that no list read waits behind
  // the tile DMA in flight: x = (first key + 16) | window tile << 17 |
  // (wave w's blocks all wholly kept) << (18 + w), y = the need bits (8 per
  // wave: row block rb, key block kq at bit 8w + 4rb + kq -- the block holds
  // a kept pair)
  __shared__ int2 tl[LIST_CAP];
  static_assert(sizeof(ring) + sizeof(bp) + sizeof(tl) <= 80 * 1024 - 32,
                "two workgroups a CU: at most 80 KiB of LDS each (160 KiB a CU), with a few bytes for the compiler's own");

  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);   // uniform: scalar branches
  const int lane = t & 63;
  const int lr = lane & 15;
  const int lg = lane >> 4;

  const int n_bh = a.batch * a.heads;
  // all query tiles of (b, h) on one XCD; the last (longest: most listed
  // key tiles under a causal mask) query tiles start first, so the short
  // ones fill in at the end of the grid
  const int bh = blockIdx.x % n_bh;
  const int qt = a.n_qt - 1 - (int)(blockIdx.x / n_bh);
  const int b = bh / a.heads;
  const int h = bh % a.heads;
  const int hk = h / (a.heads / a.kv_heads);
  const int i0 = qt * BM_ROWS;
  const int n = a.n;
  const int i_last = i0 + BM_ROWS - 1 < n - 1 ? i0 + BM_ROWS - 1 : n - 1;
  const int W = a.W, Bw = a.B, G = a.G;

  const int64_t lid = (int64_t)b * a.n_qt + qt;
  const int4* list = a.tile_list + lid * a.max_tiles * 2;
  // one round trip before the first tile's copies: the list length (and
  // its number of whole tiles, listed first), its first entry and this
  // thread's entry, the prompt length
  const int cw = __builtin_amdgcn_readfirstlane(a.tile_count[lid]);   // uniform loop bounds
  const int cnt = clampi(cw & 0xffff, 0, a.max_tiles);
  const int n_whole = clampi((int)((uint32_t)cw >> 16), 0, cnt);
  const int4 first = list[0];
  int4 mine0 = make_int4(0, 0, 0, 0), mine1 = make_int4(0, 0, 0, 0);
  if (t < a.max_tiles) {
    mine0 = list[2 * t];
    mine1 = list[2 * t + 1];
  }
  const int P = __builtin_amdgcn_readfirstlane(clampi(a.prompt_len[b], 0, n));   // uniform: scalar mask terms

  const uint16_t* qb = a.q + b * a.sq[0] + h * a.sq[1];
  const uint16_t* kb = (const uint16_t*)uniform_ptr(a.k + b * a.sk[0] + hk * a.sk[1]);
  const uint16_t* vb = (const uint16_t*)uniform_ptr(a.v + b * a.sv[0] + hk * a.sv[1]);

  // ---- this wave's query rows: blocks w and w + 4 of the tile, 64 rows
  // apart (RS), so that on a raster width dividing 64 both meet a window
  // tile's diagonal runs in the same key blocks; lane lr of block rb holds
  // row wi0 + RS*rb + lr; its Q^T operand chunks stay in registers
  constexpr int RS = NWAVE * 16;
  const int wi0 = i0 + wave * 16;
  bf16x8 qv[RB][NC];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int i = wi0 + RS * rb + lr;
    const uint16_t* qrow = qb + (int64_t)(i < n ? i : n - 1) * a.sq[2];
#pragma unroll
    for (int c = 0; c < NC; ++c)
      qv[rb][c] = *reinterpret_cast<const bf16x8*>(qrow + 32 * c + lg * 8);
  }

  // DMA of the key tile starting at key j0 into ring stage st: this wave's
  // DPW transfers of K and of V; lane l of transfer u fills LDS chunk l of
  // its 1 KiB block.  This lane's row of each transfer and its byte offsets
  // from the tile's first row (fixed per lane; under 4 GiB, checked on the
  // host); rows before key 0 or past the last key read the nearest key
  // instead (no mask keeps them)
  int dma_row[DPW], dma_c8[DPW];
  uint32_t dko[DPW], dvo[DPW];
#pragma unroll
  for (int u = 0; u < DPW; ++u) {
    const int blk = wave * DPW + u;                   // 1 KiB block of the tile
    const int row = blk * RPI + lane / CPR;
    const int chunk = (lane % CPR) ^ swz<CPR>(row);
    dma_row[u] = row;
    dma_c8[u] = chunk * 8;
    dko[u] = (uint32_t)(((int64_t)row * a.sk[2] + chunk * 8) * 2);
    dvo[u] = (uint32_t)(((int64_t)row * a.sv[2] + chunk * 8) * 2);
  }
  // LDS byte address of this wave's first 1 KiB block of ring stage 0 (K)
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)ring) + wave * DPW * 1024;
  auto issue = [&](int j0, int st) __attribute__((always_inline)) {
    j0 = __builtin_amdgcn_readfirstlane(j0);
    const uint32_t lk = lds0 + st * 2 * TILE * 2, lv = lk + TILE * 2;
    if (j0 >= 0 && j0 + BN <= n) {
      dma_tile<DPW>(kb + (int64_t)j0 * a.sk[2], vb + (int64_t)j0 * a.sv[2], dko, dvo, lk, lv);
    } else {
      const int jb = j0 > 0 ? j0 : 0;                 // j0 <= n - 1
      uint32_t ko[DPW], vo[DPW];
#pragma unroll
      for (int u = 0; u < DPW; ++u) {
        const int r = clampi(j0 + dma_row[u], 0, n - 1) - jb;   // 0 .. 63
        ko[u] = (uint32_t)(((int64_t)r * a.sk[2] + dma_c8[u]) * 2);
        vo[u] = (uint32_t)(((int64_t)r * a.sv[2] + dma_c8[u]) * 2);
      }
      dma_tile<DPW>(kb + (int64_t)jb * a.sk[2], vb + (int64_t)jb * a.sv[2], ko, vo, lk, lv);
    }
  };
  auto entry_j0 = [&](int x) { return clampi(x, -15, n - 1); };
  if (cnt > 0) issue(entry_j0(__builtin_amdgcn_readfirstlane(first.x)), 0);

  auto pack = [&](int4 e0, int4 e1) {
    int allfull = 0;
#pragma unroll
    for (int w = 0; w < NWAVE; ++w) allfull |= (((uint32_t)e1.x >> (8 * w)) & 0xffu) == 0xffu ? 1 << w : 0;
    return make_int2((entry_j0(e0.x) + 16) | ((e0.w & 1) << 17) | (allfull << 18), e0.y);
  };
  if (t < cnt) tl[t] = pack(mine0, mine1);
  for (int e = t + NTHREADS; e < cnt; e += NTHREADS) tl[e] = pack(list[2 * e], list[2 * e + 1]);

  if constexpr (MODE == DA_MODE_ROWDIAG) {
    // band centres of residue r within reach of bits 0..63: r - kG for
    // every k with r - kG in [-B, 63 + B]
    for (int r = t; r < G; r += NTHREADS) {
      uint64_t w = 0;
      if (2 * (int64_t)Bw + 1 >= G) {
        w = ~uint64_t(0);
      } else {
        int c0 = r;
        while (c0 - G >= -Bw) c0 -= G;
        for (; c0 <= 63 + Bw; c0 += G) w |= bit_range(c0 - Bw, c0 + Bw);
      }
      bp[r] = w;
    }
  }

  float mq[RB], ls[RB];                // running reference max (scaled), partial sum
  f32x4 o[RB][NB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    mq[rb] = -INFINITY;
    ls[rb] = 0.f;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) o[rb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int vt_row = 4 * lg + (lr >> 2);
  const int vt_sub = (lr & 3);
  const int my_i0 = wi0 + lr;          // this lane's row in block 0 (block rb adds RS rb)

  // Keep word of this lane's row in block rb over the tile's keys j0..j0+63
  // (bit c: key j0 + c at distance x - c).  Prompt tiles: the causal bits
  // (and below the prompt end); window tiles: the window rule at or past
  // the prompt end.  A window tile past the prompt, below every row's
  // diagonal and inside every row's window needs only the band pattern.
  auto keep_word = [&](int rb, int j0, bool win, bool inner) __attribute__((always_inline)) -> uint64_t {
    const int x = my_i0 + RS * rb - j0;
    if (!win) {
      if constexpr (MODE == DA_MODE_DENSE) return bit_range(0, x);
      else return bit_range(0, (x < P - j0 - 1 ? x : P - j0 - 1));
    }
    if constexpr (MODE == DA_MODE_ROWDIAG) {
      const uint64_t band = bp[mod_g(x, G, a.inv_g)];
      return inner ? band : band & bit_range(x - W, x) & bit_range(P - j0, 63);
    } else {
      return bit_range(x - (Bw < W ? Bw : W), x) & bit_range(P - j0, 63);
    }
  };

  // One step over NQ of the staged tile's 16-key blocks: blk[..] (all four,
  // or the two holding the wave's kept pairs), shared by its row blocks.
  // S^T = K Q^T (A = K from LDS), masks, online softmax, O^T += V^T P^T
  // over pairs of blocks (A = V^T by transposing LDS reads).  Rows 16
  // apart share the swizzle, so a block's LDS addresses are a per-lane base
  // plus 16 q rows.
  auto body = [&](auto nq, const uint16_t* st0, const int (&blk)[4], bool masked, int j0, bool win,
                  bool inner) __attribute__((always_inline)) {
    constexpr int NQ = decltype(nq)::value;
    f32x4 sc[RB][NQ];
#pragma unroll
    for (int hq = 0; hq < NQ; ++hq) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) sc[rb][hq] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int pos = (4 * c + lg) ^ swz<CPR>(lr);
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(st0 + (16 * blk[hq] + lr) * HD + pos * 8);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          sc[rb][hq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qv[rb][c], sc[rb][hq], 0, 0, 0);
      }
    }
    if (masked) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const uint64_t keep = keep_word(rb, j0, win, inner);
#pragma unroll
        for (int hq = 0; hq < NQ; ++hq) {
          const uint32_t wd = (uint32_t)(keep >> (16 * blk[hq] + 4 * lg));
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int32_t m = (int32_t)(wd << (31 - r)) >> 31;
            sc[rb][hq][r] = __int_as_float((__float_as_int(sc[rb][hq][r]) & m) | (~m & (int32_t)0xff800000));
          }
        }
      }
    }

    float mts[RB];
    bool grow = false;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float mt = -INFINITY;
#pragma unroll
      for (int hq = 0; hq < NQ; ++hq)
#pragma unroll
        for (int r = 0; r < 4; ++r) mt = fmaxf(mt, sc[rb][hq][r]);
      mts[rb] = max_over_row_groups(mt) * a.qscale;
      grow = grow || mts[rb] > mq[rb] + 8.f;
    }
    if (__any(grow)) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const float mn = fmaxf(mq[rb], mts[rb]);
        const float alpha = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(mq[rb] - mn);
        ls[rb] *= alpha;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int r = 0; r < 4; ++r) o[rb][nb][r] *= alpha;
        mq[rb] = mn;
      }
    }
    bf16x8 pb[RB][NQ / 2];           // P^T of the step's 32-key pairs of blocks
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float mref = mq[rb] == -INFINITY ? 0.f : mq[rb];
#pragma unroll
      for (int cc = 0; cc < NQ / 2; ++cc)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sc[rb][2 * cc + e / 4][e % 4], a.qscale, -mref));
          ls[rb] += p;
          pb[rb][cc][e] = (__bf16)p;
        }
    }
    // O^T += V^T P^T: the pair's blocks give the product's 32 keys
#pragma unroll
    for (int cc = 0; cc < NQ / 2; ++cc) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        typedef short v4i16 __attribute__((ext_vector_type(4)));
        typedef short v8i16 __attribute__((ext_vector_type(8)));
        const int chunk = 2 * nb + (vt_sub >> 1);
        const int lane_off = vt_row * HD + ((chunk ^ swz<CPR>(vt_row)) * 8) + (vt_sub & 1) * 4;
        const uint16_t* plo = st0 + TILE + 16 * blk[2 * cc] * HD + lane_off;
        const uint16_t* phi = st0 + TILE + 16 * blk[2 * cc + 1] * HD + lane_off;
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(plo));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(phi));
        const v8i16 w = v8i16{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        const bf16x8 vf = __builtin_bit_cast(bf16x8, w);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          o[rb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb[rb][cc], o[rb][nb], 0, 0, 0);
      }
    }
  };

  // One listed tile a step, tile t in stage t % NS.  At the top of step idx
  // tile idx has landed and every wave is done with step idx-1, whose stage
  // then receives tile idx+1 -- fetched while this step computes.  The
  // DMA is invisible to the compiler's waits: each wave waits for its own
  // part (vmcnt), then the barrier covers every wave's part.
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();                     // tile 0 landed, list and band pattern written
  // the step body takes its ring stage as a constant (the loop runs two
  // steps an iteration), so every LDS address is a fixed per-lane base
  // plus an immediate offset
  auto step = [&](int idx, auto stage, auto nq) __attribute__((always_inline)) {
    constexpr int ST = decltype(stage)::value;
    constexpr int NQ = decltype(nq)::value;
    if (idx > 0) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // tile idx (this wave's part)
      __builtin_amdgcn_s_barrier();               // everyone's part; step idx-1 done
      __asm__ volatile("" ::: "memory");
    }
    if (idx + 1 < cnt) issue((tl[idx + 1].x & 0x1ffff) - 16, (ST + 1) % NS);
    const int2 e = tl[idx];
    const int ex = __builtin_amdgcn_readfirstlane(e.x);
    const unsigned need8 = ((uint32_t)__builtin_amdgcn_readfirstlane(e.y) >> (wave * 8)) & 0xffu;
    // a wave without a kept pair in this tile only takes part in the copies
    // and barriers
    if (need8 == 0) return;
    const int j0 = (ex & 0x1ffff) - 16;
    const bool win = (ex >> 17) & 1;
    const uint16_t* st0 = ring + ST * 2 * TILE;
    const bool inner = MODE == DA_MODE_ROWDIAG && win && j0 >= P && wi0 - j0 >= BN - 1 &&
                       wi0 + RS * (RB - 1) + 15 - j0 <= W;
    if constexpr (NQ == 2) {
      // the (at most) two key blocks holding the wave's kept pairs; with one,
      // a second it has no kept pair in
      const unsigned m4 = (need8 | (need8 >> 4)) & 0xfu;
      const int q0 = m4 ? __builtin_ctz(m4) : 0;
      const unsigned rest = m4 & (m4 - 1);
      const int blk[4] = {q0, rest ? __builtin_ctz(rest) : (q0 + 1) & 3, 0, 0};
      body(nq, st0, blk, true, j0, win, inner);
    } else {
      const int blk[4] = {0, 1, 2, 3};
      const bool allfull = (ex >> (18 + wave)) & 1;
      body(nq, st0, blk, !allfull, j0, win, inner);
    }
  };
  // tiles from..to-1 (all whole or all half), tile idx in ring stage idx % 2
  auto run = [&](auto nq, int from, int to) __attribute__((always_inline)) {
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    if (from & 1) {
      for (int idx = from; idx < to; idx += 2) {
        step(idx, S1{}, nq);
        if (idx + 1 < to) step(idx + 1, S0{}, nq);
      }
    } else {
      for (int idx = from; idx < to; idx += 2) {
        step(idx, S0{}, nq);
        if (idx + 1 < to) step(idx + 1, S1{}, nq);
      }
    }
  };
  static_assert(NS == 2, "two steps an iteration, one per stage");
  run(std::integral_constant<int, 4>{}, 0, n_whole);
  run(std::integral_constant<int, 2>{}, n_whole, cnt);

  // ---- normalise and store: lane holds row wi0+RS*rb+lr, dims 16nb + 4lg + r
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float L = ls[rb];
    L = sum_over_row_groups(L);
    const int i = wi0 + RS * rb + lr;
    if (i > i_last) continue;
    const float inv = 1.f / L;
    uint16_t* orow = a.o + b * a.so[0] + h * a.so[1] + (int64_t)i * a.so[2];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const uint32_t w0 = f32_to_bf16(o[rb][nb][0] * inv) | (f32_to_bf16(o[rb][nb][1] * inv) << 16);
      const uint32_t w1 = f32_to_bf16(o[rb][nb][2] * inv) | (f32_to_bf16(o[rb][nb][3] * inv) << 16);
      *reinterpret_cast<uint2*>(orow + 16 * nb + 4 * lg) = make_uint2(w0, w1);
    }
    if (a.lse && lg == 0)
      a.lse[((int64_t)b * a.heads + h) * n + i] = (mq[rb] + log2f(L)) * kLn2P;
  }
}
}  // namespace da

using namespace da;

static int n_query_tiles(int n) { return (n + BM_ROWS - 1) / BM_ROWS; }
static int max_key_tiles(int n) { return (n + BN - 1) / BN + LIST_EXTRA; }

extern "C" int64_t da_prefill_tiles_bytes(int32_t batch, int32_t n) {
  if (batch < 0 || n < 0) return fail(DA_EINVAL, "batch=%d n=%d", batch, n);
  clear_error();
  const int64_t lists = (int64_t)batch * n_query_tiles(n);
  return ((lists * 4 + 15) / 16) * 16 + lists * max_key_tiles(n) * 32;
}

static void fill_common(PrefillArgs& a, const da_mask* m, int32_t batch, int32_t n,
                        const int32_t* prompt_len, const void* tiles) {
  a.prompt_len = prompt_len;
  a.batch = batch;
  a.n = n;
  a.mode = m->mode;
  // Distances between a row and a key of one sequence are below n, so a
  // window or band of n or more keeps what an unbounded one keeps: W and B
  // are clamped to n, which keeps every row/key offset computation (x - W,
  // c + B, ...) far inside the int range and every band loop short.
  a.W = m->W < n ? m->W : n;
  a.B = m->B < n ? m->B : n;
  a.G = m->G;
  a.inv_g = 1.f / (float)m->G;
  a.n_qt = n_query_tiles(n);
  a.max_tiles = max_key_tiles(n);
  const int64_t lists = (int64_t)batch * a.n_qt;
  a.tile_count = reinterpret_cast<const int32_t*>(tiles);
  a.tile_list = reinterpret_cast<const int4*>(reinterpret_cast<const char*>(tiles) +
                                              ((lists * 4 + 15) / 16) * 16);
}

extern "C" int da_prefill_tiles_build(const da_mask* m, int32_t batch, int32_t n,
                                      const int32_t* prompt_len, void* tiles, int64_t tiles_bytes,
                                      void* stream) {
  int rc = check_mask(m);
  if (rc) return rc;
  if (!m->causal) return fail(DA_ENOTSUP, "prefill needs a causal mask");
  if (batch < 0 || n < 0) return fail(DA_EINVAL, "batch=%d n=%d", batch, n);
  const int64_t need = da_prefill_tiles_bytes(batch, n);
  if (batch > 0 && n > 0 && (!prompt_len || !tiles))
    return fail(DA_EINVAL, "prompt_len and tiles must be non-NULL");
  if (tiles_bytes < need) return fail(DA_ECAPACITY, "tiles buffer %lld bytes < %lld", (long long)tiles_bytes, (long long)need);
  if ((uintptr_t)tiles % 16) return fail(DA_EINVAL, "tiles buffer not 16-byte aligned");
  clear_error();
  if (batch == 0 || n == 0) return DA_OK;
  PrefillArgs a{};
  fill_common(a, m, batch, n, prompt_len, tiles);
  const int64_t blocks = (int64_t)batch * a.n_qt;
  hipLaunchKernelGGL(prefill_tiles_kernel, dim3((unsigned)blocks), dim3(64), 0, (hipStream_t)stream, a);
  return check_launch("prefill_tiles_kernel");
}

extern "C" int da_band_prefill_attn(const da_mask* m, da_dtype dtype, int32_t batch, int32_t heads,
                                    int32_t kv_heads, int32_t n, int32_t head_dim,
                                    const void* q, const void* k, const void* v, void* out,
                                    const int64_t* strides, const int32_t* prompt_len,
                                    const void* tiles, int64_t tiles_bytes, float scale, float* lse,
                                    void* stream) {
  int rc = check_mask(m);
  if (rc) return rc;
  if (!m->causal) return fail(DA_ENOTSUP, "prefill needs a causal mask");
  if (dtype != DA_BF16) return fail(DA_ENOTSUP, "prefill runs on bf16 inputs (dtype %d)", (int)dtype);
  if (!(scale > 0.f) || scale == INFINITY) return fail(DA_EINVAL, "scale must be positive and finite (%g)", (double)scale);
  if (head_dim != 64 && head_dim != 128) return fail(DA_ENOTSUP, "head_dim %d not in {64, 128}", head_dim);
  if ((int64_t)n > (int64_t)BN * MAX_LIST)
    return fail(DA_ENOTSUP, "prefill supports sequences of up to %d tokens (n=%d)", BN * MAX_LIST, n);
  if (m->mode == DA_MODE_ROWDIAG && m->G > GMAX)
    return fail(DA_ENOTSUP, "row-diagonal prefill supports G <= %d (G=%d)", GMAX, m->G);
  if (batch < 0 || heads < 1 || kv_heads < 1 || heads % kv_heads || n < 0)
    return fail(DA_EINVAL, "batch=%d heads=%d kv_heads=%d n=%d", batch, heads, kv_heads, n);
  if (!strides) return fail(DA_EINVAL, "strides is NULL");
  if (batch > 0 && n > 0 && (!q || !k || !v || !out || !prompt_len || !tiles))
    return fail(DA_EINVAL, "q, k, v, out, prompt_len and tiles must be non-NULL");
  for (int i = 0; i < 12; ++i)
    if (strides[i] < 0 || (strides[i] * 2) % 16) return fail(DA_EINVAL, "stride %d must be a non-negative multiple of 8 elements", i);
  // a key tile's rows are addressed by 32-bit byte offsets from its first row
  if (((int64_t)(BN - 1) * strides[5] + head_dim) * 2 > UINT32_MAX ||
      ((int64_t)(BN - 1) * strides[8] + head_dim) * 2 > UINT32_MAX)
    return fail(DA_ENOTSUP, "key/value position stride too large (%lld, %lld elements)",
                (long long)strides[5], (long long)strides[8]);
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out | (uintptr_t)tiles) % 16)
    return fail(DA_EINVAL, "q, k, v, out and tiles must be 16-byte aligned");
  const int64_t need = da_prefill_tiles_bytes(batch, n);
  if (tiles_bytes < need)
    return fail(DA_ECAPACITY, "tiles buffer %lld bytes < %lld for batch %d, n %d", (long long)tiles_bytes,
                (long long)need, batch, n);
  clear_error();
  if (batch == 0 || n == 0) return DA_OK;
  PrefillArgs a{};
  a.q = reinterpret_cast<const uint16_t*>(q);
  a.k = reinterpret_cast<const uint16_t*>(k);
  a.v = reinterpret_cast<const uint16_t*>(v);
  a.o = reinterpret_cast<uint16_t*>(out);
  a.lse = lse;
  for (int i = 0; i < 3; ++i) {
    a.sq[i] = strides[i];
    a.sk[i] = strides[3 + i];
    a.sv[i] = strides[6 + i];
    a.so[i] = strides[9 + i];
  }
  fill_common(a, m, batch, n, prompt_len, tiles);
  a.heads = heads;
  a.kv_heads = kv_heads;
  a.qscale = scale * kLog2eP;
  const int64_t blocks = (int64_t)a.n_qt * batch * heads;
  if (blocks > 0x7fffffff) return fail(DA_ENOTSUP, "grid too large");
  void (*fn)(PrefillArgs);
  switch (m->mode) {
    case DA_MODE_DENSE: fn = head_dim == 128 ? prefill_kernel<128, DA_MODE_DENSE> : prefill_kernel<64, DA_MODE_DENSE>; break;
    case DA_MODE_BAND: fn = head_dim == 128 ? prefill_kernel<128, DA_MODE_BAND> : prefill_kernel<64, DA_MODE_BAND>; break;
    default: fn = head_dim == 128 ? prefill_kernel<128, DA_MODE_ROWDIAG> : prefill_kernel<64, DA_MODE_ROWDIAG>; break;
  }
  hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(NTHREADS), 0, (hipStream_t)stream, a);
  return check_launch("prefill_kernel");
}
