// sparse_decode_attn: split-KV decode attention over listed (kept) keys.
//
// Grid: one 256-thread workgroup per (query, kv head, chunk of `split`
// listed keys).  Each K/V row (head_dim elements, 128-512 bytes) is read by
// LPR = row_bytes / 16 consecutive lanes with one 16-byte load each, so one
// wave instruction moves 1 KiB and the rows of a run are contiguous in
// memory.  Rows are taken in tiles of NP passes (NP * 256 / LPR rows); a
// chunk of at most three tiles has all of them in flight at once, longer
// chunks keep two in flight while the older one is reduced.  Before the first
// tile, every index of the chunk, then (paged caches) every block-table
// entry, is read in one round trip each and turned into a row offset in LDS,
// so no K/V load waits on more than the loads issued before it.  The kernel
// is bound by HBM bandwidth on the kept bytes and uses each byte once, so
// K/V go straight to registers; LDS only carries the row offsets and the
// cross-wave softmax/output reduction.
//
// All hq/hkv query heads that share a kv head are served by the same
// workgroup, so each kept row is read once.  Scores are q . k scaled by
// log2(e)/sqrt(d) (folded into q) and summed across a row's lanes with DPP;
// the chunk's max, sum and sum p*v follow.  A query whose list fits one
// chunk writes its normalised output directly.  Otherwise each chunk stores
// a (max, sum, unnormalised o) partial and merge_kernel combines them by
// log-sum-exp.  (Merging inside the decode kernel by the last-arriving chunk
// needs agent-scope fences, which write back and invalidate the whole L2 of
// the XCD on this part: measured far slower than a second launch.)
//
// Mask form (FORM 1, 2): instead of reading lists, every lane computes the
// entries of its rows from the query's position, prompt length and the
// mask -- the list builder's entries in the builder's order, from the
// keep-set's closed form (KeepCF) -- so keep-set build and attention are one
// launch; the lists can be written out as well, and the new token's K/V rows
// can be appended to the cache at its position before they are read.
//
// Every index read from device memory (request, position, page) is clamped
// into the cache extents the host passes, so no list content can make the
// kernel read outside the cache.
#include "common.h"

#include <mutex>
#include <type_traits>

namespace da {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  int64_t page_stride, head_stride, slot_stride;
  const int32_t* block_table;
  int bt_stride, ps_shift, ps_mask;
  int n_seq, n_pages, max_len;      // extents for clamping
  const int32_t* seq;
  const int32_t* count;
  const int32_t* idx;
  // keep-set computed in the kernel (mask form): positions, prompt lengths,
  // the mask, and optional list outputs (count may be null: no lists)
  const int32_t* pos;
  const int32_t* prompt;
  int mode, W, B, G;
  int32_t* count_out;
  int32_t* idx_out;
  // KV append (mask form): the new token's K and V rows [n_q][hkv][HD], or null
  const void* k_new;
  const void* v_new;
  int n_q, hq, hkv, cap, split, max_split;
  float qscale;           // scale * log2(e)
  void* out;
  float* lse;
  float* ws_o;            // [n_q][hq][max_split][HD]
  float* ws_ml;           // [n_q][hq][max_split][2]
  int32_t* ws_cnt;        // [n_q][hkv] keep-set sizes (mask form, several chunks)
  const int32_t* mcount;  // the sizes the merge reads: count [n_q] (lists) or ws_cnt
  int mcount_per_head;    // mcount indexed by (query, kv head) instead of query
  int list_heads;         // list form: lists per query, 1 or hkv (list q*hkv + g per kv head)
  const int32_t* head_wb; // mask form: per-query-head (W, B) [hq][2], or null
};

// Workspace layout: partial outputs, then partial (max, sum) pairs, then
// (mask form) each query's keep-set size for the merge.
struct WsLayout {
  int64_t o_off, ml_off, cnt_off, bytes;
};

static inline int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

static WsLayout ws_layout(int64_t n_q, int64_t hq, int64_t hd, int64_t ns) {
  WsLayout w{0, 0, 0, 0};
  if (ns <= 1) return w;
  const int64_t rows = n_q * hq * ns;
  w.o_off = 0;
  w.ml_off = align256(rows * hd * 4);
  w.cnt_off = w.ml_off + align256(rows * 2 * 4);
  w.bytes = w.cnt_off + align256(n_q * hq * 4);
  return w;
}


template <bool BF16, int EPL>
__device__ inline void store_out(void* base, int64_t off, const float* x) {
  if constexpr (BF16) {
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = f32_to_bf16(x[2 * e]) | (f32_to_bf16(x[2 * e + 1]) << 16);
    *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(base) + off) = u32x4{w[0], w[1], w[2], w[3]};
  } else {
    *reinterpret_cast<u32x4*>(reinterpret_cast<float*>(base) + off) =
        u32x4{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3])};
  }
}

// One tile = NP passes of the workgroup = NP * (256 / LPR) listed rows.
template <bool BF16, int HD, int NP>
struct Tile {
  static constexpr int ES = BF16 ? 2 : 4;
  static constexpr int EPL = 16 / ES;
  static constexpr int LPR = HD * ES / 16;
  static constexpr int RPP = 256 / LPR;
  static constexpr int ROWS = NP * RPP;
  u32x4 k[NP], v[NP];

  // Issues the K and V loads of tile t (no waits), nontemporal: each kept
  // byte is read once (measured 6-8 % faster than cached loads).  Slots past
  // the chunk read position 0's row (always valid, and shared, so it costs
  // cache hits).
  __device__ inline void load(const char* kb, const char* vb, const int64_t* off, int64_t off0,
                              int t, int rsub, int nrows) {
    int64_t o[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int r = t * ROWS + p * RPP + rsub;
      o[p] = off[r < nrows ? r : nrows - 1];
      o[p] = r < nrows ? o[p] : off0;
    }
    // all LDS reads first, then all global loads: one LDS wait per tile
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      k[p] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kb + o[p] * ES));
      v[p] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vb + o[p] * ES));
    }
  }
};

// q . k over this lane's 16-byte chunk: bf16 pairs through v_dot2, fp32 by FMA.
template <bool BF16>
__device__ inline float chunk_dot(const u32x4 q, const u32x4 k, const float* qf) {
  if constexpr (BF16) {
    typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
    float d = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // copy to scalars first: bit-casting a vector element directly makes
      // this compiler read element 0 for every e
      const uint32_t qe = q[e], ke = k[e];
      d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qe),
                                          __builtin_bit_cast(bf16x2, ke), d, false);
    }
    return d;
  } else {
    float d = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) d = fmaf(qf[e], __uint_as_float(k[e]), d);
    return d;
  }
}

// Workgroup barrier that orders LDS only: global loads in flight stay in
// flight (a plain __syncthreads also waits for every outstanding load).
__device__ inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Element offset of position j of request sq (contiguous or paged cache).
__device__ inline int64_t row_offset(const DecodeArgs& a, const int32_t* bt, int sq, int j) {
  j = clampi(j, 0, a.max_len - 1);
  if (bt)
    return (int64_t)clampi(bt[j >> a.ps_shift], 0, a.n_pages - 1) * a.page_stride +
           (int64_t)(j & a.ps_mask) * a.slot_stride;
  return (int64_t)sq * a.page_stride + (int64_t)j * a.slot_stride;
}

// A query's keep-set in closed form (mask form of the decode kernel).
// Entries 0 .. Pc-1 are the prompt positions (DENSE: every position up to
// the query); the window entries follow in ascending position, i.e. in
// descending offset d = i - j over the kept offsets in [0, dmax], dmax =
// i - max(i - W, Pc).  The kept offsets are, for the band rule, 0 .. B,
// and for the row-diagonal rule those within B of a multiple of G: exactly
// the d with (d + B) mod G <= 2B -- runs of 2B + 1 offsets, period G, the
// first starting at -B -- or every offset when 2B + 1 >= G.  So the count of
// kept offsets in [0, x] is, with y = x + B, (y div G)(2B + 1) + min(y mod G,
// 2B) + 1 - B, and the m-th kept offset (1-based, ascending) is
// ((m + B - 1) div (2B + 1)) G + (m + B - 1) mod (2B + 1) - B.
struct KeepCF {
  int i, Pc, T;        // query position, prompt entries, window entries
  int periodic;        // 1: row-diagonal runs; 0: offsets 0 .. T-1 all kept
  uint32_t B, G, run;  // run = 2B + 1

  __device__ int size() const { return Pc + T; }
  // position of entry e, 0 <= e < size()
  __device__ int entry(int e) const {
    if (e < Pc) return e;
    const uint32_t m = (uint32_t)(T - (e - Pc));   // 1-based ascending rank of the offset
    if (!periodic) return i - (int)(m - 1);
    const uint32_t nn = m + B - 1;
    return i - (int)((nn / run) * G + nn % run - B);
  }
};

__device__ inline KeepCF keep_cf(int mode, int i, int P, int W, int B, int G, bool bad) {
  KeepCF k{};
  k.i = i;
  if (bad) return k;
  const int L = i + 1;
  if (mode == DA_MODE_DENSE) {
    k.Pc = L;
    return k;
  }
  k.Pc = P < L ? P : L;
  const int wlo = i - W > k.Pc ? i - W : k.Pc;
  const int dmax = i - wlo;                  // -1: the prompt reaches the query
  if (dmax < 0) return k;
  if (mode == DA_MODE_BAND) {
    k.T = (dmax < B ? dmax : B) + 1;
  } else if (2 * (int64_t)B + 1 >= G) {
    k.T = dmax + 1;
  } else {
    k.periodic = 1;
    k.B = (uint32_t)B;
    k.G = (uint32_t)G;
    k.run = 2 * (uint32_t)B + 1;
    const uint32_t y = (uint32_t)dmax + (uint32_t)B;
    const uint32_t ym = y % k.G;
    k.T = (int)((y / k.G) * k.run + (ym < 2 * k.B ? ym : 2 * k.B) + 1 - k.B);
  }
  return k;
}

// FORM: 0 = listed keys; 1 = keep-set from the mask; 2 = from the mask with
// a window and band per kv head.
template <bool BF16, int HD, int GRP, int NP, int FORM>
//
// The arguments a workgroup needs before its first memory reads -- the
// query's position and prompt length arrays (list form: the counts and the
// lists), its request array, the grid decomposition, K, V and q -- come
// first and one by one; all but q fit the 14 kernel-argument SGPRs the
// hardware preloads at launch (the library is built with kernel-argument
// preloading), so the position/request reads start without first waiting
// for the argument block.  The full argument block follows; its loads
// overlap those reads.
__global__ void __launch_bounds__(256) decode_kernel(const int32_t* m0_p, const int32_t* m1_p,
                                                     const int32_t* seq_p, int hkv_p, int max_split_p,
                                                     int cap_p, int split_p, const void* k_p,
                                                     const void* v_p, const void* q_p, DecodeArgs a) {
  constexpr bool MASKED = FORM >= 1;
  constexpr bool PERHEAD = FORM == 2;
  using TL = Tile<BF16, HD, NP>;
  constexpr int ES = TL::ES;
  constexpr int EPL = TL::EPL;
  constexpr int LPR = TL::LPR;
  constexpr int RPP = TL::RPP;
  constexpr int ROWS = TL::ROWS;

  extern __shared__ int64_t rowoff[];     // [split] element offset of each listed row
  __shared__ float red_m[4][GRP];
  __shared__ float red_l[4][GRP];
  __shared__ float red_o[4][GRP][HD];

  const int t = threadIdx.x;
  const int wave = t >> 6;
  const int c = t % LPR;
  const int rsub = t / LPR;

  const int bid = blockIdx.x;
  const int s = bid % max_split_p;
  const int qg = bid / max_split_p;
  const int qi = qg / hkv_p;
  const int g = qg % hkv_p;
  // mask form: the query's position, prompt length and request, read first
  // and together (the empty asm keeps later memory operations, and the
  // waits they bring, behind these three reads)
  int i_m = 0, P_m = 0, sq_m = 0;
  if constexpr (MASKED) {
    i_m = m0_p[qi];
    P_m = m1_p[qi];
    sq_m = seq_p[qi];
    // the argument-block fields the first addresses need, read alongside
    __asm__ volatile("" ::"s"(a.head_stride), "s"(a.page_stride),
                     "s"(a.slot_stride), "s"(a.n_seq), "s"(a.max_len), "s"(a.mode), "s"(a.W), "s"(a.B),
                     "s"(a.G) : "memory");
  }
  const int r0 = s * split_p;
  const int lim = cap_p - r0 < split_p ? cap_p - r0 : split_p;   // >= 1

  // ---- stage 0: query slices, list entries, count and request in one
  // round trip (every load unconditional and in bounds)
  u32x4 qw[GRP];
#pragma unroll
  for (int h = 0; h < GRP; ++h) {
    const int64_t qoff = (((int64_t)qi * hkv_p + g) * GRP + h) * HD + c * EPL;   // hq = hkv GRP
    qw[h] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(q_p) + qoff * ES);
  }
  constexpr int IPT = 4;                  // list entries per thread per round
  int cnt, nrows, sq;
  const int32_t* bt;
  int64_t off0;
  const char* kb = reinterpret_cast<const char*>(k_p) + ((int64_t)g * a.head_stride + c * EPL) * ES;
  const char* vb = reinterpret_cast<const char*>(v_p) + ((int64_t)g * a.head_stride + c * EPL) * ES;
  TL b0, b1;
  // mask form: the chunk row of the appended token, or -1; the keep-set's
  // closed form
  int sub_row = -1;
  KeepCF kc{};
  __shared__ u32x4 newrow[2 * LPR];       // mask form, KV append: the new K, V rows
  // mask form: keep-set size; KV append state (the new rows travel in nkv)
  int n_keep = 0, qpos = 0;
  bool appending = false, stores = false;
  u32x4 nkv = u32x4{0u, 0u, 0u, 0u};
  // KV append: lanes 0 .. 2 LPR-1 store the new K / V row at position qpos
  // (positions outside the cache are not written).  This workgroup's own
  // use of the row reads the LDS copy, so no load has to wait for the store.
  auto store_new_row = [&]() {
    if (t < 2 * LPR) {
      const int64_t o = row_offset(a, bt, sq, qpos);
      char* base = reinterpret_cast<char*>(const_cast<void*>(t < LPR ? a.k : a.v));
      *reinterpret_cast<u32x4*>(base + ((int64_t)g * a.head_stride + c * EPL + o) * ES) = nkv;
    }
  };
  if constexpr (!MASKED) {
    // the query's list, or with one list per kv head this kv head's
    const int lrow = a.list_heads > 1 ? qg : qi;
    const int32_t* myidx = m1_p + (int64_t)lrow * cap_p + r0;
    int jj[IPT];
#pragma unroll
    for (int u = 0; u < IPT; ++u) {
      const int r = u * 256 + t;
      jj[u] = myidx[r < lim ? r : lim - 1];
    }
    cnt = m0_p[lrow];
    const int sq_raw = seq_p[qi];
    // compiler-only barrier: keeps the loads above ahead of the count test
    // (they would otherwise be sunk behind it), with the argument-block
    // fields the row offsets need read alongside; emits nothing
    __asm__ volatile("" ::"s"(a.head_stride), "s"(a.page_stride), "s"(a.slot_stride), "s"(a.n_seq),
                     "s"(a.max_len) : "memory");
    cnt = cnt < a.cap ? cnt : a.cap;
    if (r0 >= cnt) return;
    nrows = cnt - r0 < a.split ? cnt - r0 : a.split;
    sq = clampi(sq_raw, 0, a.n_seq - 1);

    // ---- stage 1: element offset of every listed row into LDS
    bt = a.block_table ? a.block_table + (int64_t)sq * a.bt_stride : nullptr;
    off0 = bt ? (int64_t)clampi(bt[0], 0, a.n_pages - 1) * a.page_stride
              : (int64_t)sq * a.page_stride;
    for (int base = 0; base < nrows; base += IPT * 256) {
      if (base > 0) {
#pragma unroll
        for (int u = 0; u < IPT; ++u) {
          const int r = base + u * 256 + t;
          jj[u] = myidx[r < lim ? r : lim - 1];
        }
      }
#pragma unroll
      for (int u = 0; u < IPT; ++u) jj[u] = clampi(jj[u], 0, a.max_len - 1);
      int64_t o[IPT];
      if (bt) {
        int pg[IPT];
#pragma unroll
        for (int u = 0; u < IPT; ++u) pg[u] = bt[jj[u] >> a.ps_shift];
#pragma unroll
        for (int u = 0; u < IPT; ++u)
          o[u] = (int64_t)clampi(pg[u], 0, a.n_pages - 1) * a.page_stride +
                 (int64_t)(jj[u] & a.ps_mask) * a.slot_stride;
      } else {
#pragma unroll
        for (int u = 0; u < IPT; ++u) o[u] = (int64_t)sq * a.page_stride + (int64_t)jj[u] * a.slot_stride;
      }
#pragma unroll
      for (int u = 0; u < IPT; ++u) {
        const int r = base + u * 256 + t;
        if (r < nrows) rowoff[r] = o[u];
      }
    }
    __syncthreads();
  } else {
    // ---- keep-set in the kernel, in closed form: entry e of the query's
    // keep-set is e itself for the prompt part (or, DENSE, every key up to
    // the query) and the (T - (e - Pc))-th kept offset d counted from the
    // query for the window part (keep_cf), so every lane computes the
    // positions of its own rows with no scan, barrier or memory read: the
    // same entries in the same order as the list builder's scan.  With a
    // contiguous cache every K/V load of the chunk is issued right after the
    // query's position, prompt length and request arrive; a paged cache
    // first reads the block-table entries of the chunk's rows (one round
    // trip) into LDS row offsets.  With list outputs the kv-head-0
    // workgroups also write the entries of their chunk.
    const int i = i_m;
    const int P = P_m;
    const int sq_raw = sq_m;
    // the mask's window and band, or this head's own (negative read as 0;
    // per-head masks reach this kernel with one query head per kv head)
    int Wm = a.W, Bm = a.B;
    if constexpr (PERHEAD) {
      Wm = a.head_wb[2 * g] > 0 ? a.head_wb[2 * g] : 0;
      Bm = a.head_wb[2 * g + 1] > 0 ? a.head_wb[2 * g + 1] : 0;
    }
    // KV append: lanes 0 .. LPR-1 carry the new token's K chunk of this kv
    // head, lanes LPR .. 2 LPR-1 its V chunk
    appending = a.k_new != nullptr;
    if (appending && t < 2 * LPR) {
      const void* src = t < LPR ? a.k_new : a.v_new;
      const int64_t off = ((int64_t)qi * a.hkv + g) * HD + c * EPL;
      nkv = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(src) + off * ES);
    }
    __asm__ volatile("" ::: "memory");
    sq = clampi(sq_raw, 0, a.n_seq - 1);
    bt = a.block_table ? a.block_table + (int64_t)sq * a.bt_stride : nullptr;
    off0 = bt ? (int64_t)clampi(bt[0], 0, a.n_pages - 1) * a.page_stride
              : (int64_t)sq * a.page_stride;
    const bool bad = i < 0 || P < 0;
    qpos = i;
    stores = appending && !bad && i < a.max_len;
    kc = keep_cf(a.mode, i, P, Wm, Bm, a.G, bad);
    const int n = kc.size();
    n_keep = n;
    cnt = n < a.cap ? n : a.cap;
    // the new row is entry n - 1 of the keep-set (position i is always kept);
    // it is attended unless the list was cut at cap
    if (stores && n <= a.cap && n - 1 >= r0 && n - 1 < r0 + lim) sub_row = n - 1 - r0;
    if (r0 >= cnt) {
      // nothing to attend; the lists, sizes and the appended row are still due
      if (a.count_out != nullptr && g == 0 && s == 0 && t == 0) a.count_out[qi] = n;
      if (a.ws_cnt && s == 0 && t == 0) a.ws_cnt[(int64_t)qi * a.hkv + g] = n;
      if (stores && a.max_split == 1) store_new_row();
      return;
    }
    nrows = cnt - r0 < a.split ? cnt - r0 : a.split;
    if (bt) {
      // ---- stage 1 (paged): element offset of every row of the chunk
      for (int base = 0; base < nrows; base += IPT * 256) {
        int jj[IPT], pg[IPT];
#pragma unroll
        for (int u = 0; u < IPT; ++u) {
          const int r = base + u * 256 + t;
          jj[u] = clampi(kc.entry(r0 + (r < nrows ? r : nrows - 1)), 0, a.max_len - 1);
        }
#pragma unroll
        for (int u = 0; u < IPT; ++u) pg[u] = bt[jj[u] >> a.ps_shift];
#pragma unroll
        for (int u = 0; u < IPT; ++u) {
          const int r = base + u * 256 + t;
          if (r < nrows)
            rowoff[r] = (int64_t)clampi(pg[u], 0, a.n_pages - 1) * a.page_stride +
                        (int64_t)(jj[u] & a.ps_mask) * a.slot_stride;
        }
      }
      __syncthreads();
    }
  }

  // ---- query slices as fp32 (the fp32 path; bf16 uses the packed words)
  float qf[GRP][4];
#pragma unroll
  for (int h = 0; h < GRP; ++h)
#pragma unroll
    for (int e = 0; e < 4; ++e) qf[h][e] = __uint_as_float(qw[h][e]) * a.qscale;
  const float sscale = BF16 ? a.qscale : 1.f;

  // ---- stage 2: tiles of ROWS rows, two in flight; per-thread online softmax
  float m[GRP], l[GRP], acc[GRP][EPL];
#pragma unroll
  for (int h = 0; h < GRP; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }
  const int nt = (nrows + ROWS - 1) / ROWS;

  auto process = [&](const TL& buf, int tt) {
    u32x4 kx[NP], vx4[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      kx[p] = buf.k[p];
      vx4[p] = buf.v[p];
    }
    if constexpr (MASKED) {
      if (sub_row >= 0) {                     // the appended row: its LDS copy
#pragma unroll
        for (int p = 0; p < NP; ++p)
          if (tt * ROWS + p * RPP + rsub == sub_row) {
            kx[p] = newrow[c];
            vx4[p] = newrow[LPR + c];
          }
      }
    }
    float sc[NP][GRP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const bool valid = tt * ROWS + p * RPP + rsub < nrows;
#pragma unroll
      for (int h = 0; h < GRP; ++h) {
        const float d = group_sum<LPR>(chunk_dot<BF16>(qw[h], kx[p], qf[h])) * sscale;
        sc[p][h] = valid ? d : -INFINITY;
      }
    }
    float mref[GRP];
#pragma unroll
    for (int h = 0; h < GRP; ++h) {
      float mt = sc[0][h];
#pragma unroll
      for (int p = 1; p < NP; ++p) mt = fmaxf(mt, sc[p][h]);
      const float mn = fmaxf(m[h], mt);
      mref[h] = mn == -INFINITY ? 0.f : mn;     // no valid row seen yet
      const float f = exp2f(m[h] - mref[h]);
      l[h] *= f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] *= f;
      m[h] = mn;
    }
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      float vx[EPL];
      unpack<EPL>(vx4[p], vx);
#pragma unroll
      for (int h = 0; h < GRP; ++h) {
        const float w = exp2f(sc[p][h] - mref[h]);
        l[h] += w;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(w, vx[e], acc[h][e]);
      }
    }
  };

  // Row r of the chunk: its element offset from the keep-set's closed form
  // (mask form, contiguous cache) or from LDS; slots past the chunk read
  // the request's first row (always valid, and shared, so cache hits).
  const bool direct = MASKED && bt == nullptr;
  auto load = [&](TL& b, int tt) {
    if (direct) {
      int64_t o[NP];
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int r = tt * ROWS + p * RPP + rsub;
        const int j = clampi(kc.entry(r0 + (r < nrows ? r : 0)), 0, a.max_len - 1);
        o[p] = r < nrows ? (int64_t)sq * a.page_stride + (int64_t)j * a.slot_stride : off0;
      }
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        b.k[p] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kb + o[p] * ES));
        b.v[p] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vb + o[p] * ES));
      }
    } else {
      b.load(kb, vb, rowoff, off0, tt, rsub, nrows);
    }
  };
  // mask form: work that no load waits for, done once the first loads are
  // in flight -- list outputs, keep-set sizes for the merge, the appended
  // row's store and its LDS copy
  auto after_issue = [&]() {
    if constexpr (MASKED) {
      const int lim_e = r0 + lim;                     // entries of this chunk: [r0, lim_e)
      if (a.count_out != nullptr && g == 0) {
        int32_t* my_out = a.idx_out + (int64_t)qi * a.cap;
        const int hi = n_keep < lim_e ? n_keep : lim_e;
        for (int e = r0 + t; e < hi; e += 256) my_out[e] = kc.entry(e);
        if (s == 0 && t == 0) a.count_out[qi] = n_keep;
      }
      if (a.ws_cnt && s == 0 && t == 0) a.ws_cnt[(int64_t)qi * a.hkv + g] = n_keep;
      // KV append: one chunk -- this one -- or, with several, the chunk that
      // attends the last entry (position i itself when the list is not cut)
      if (stores && (a.max_split == 1 || (cnt - 1) / a.split == s)) store_new_row();
      if (appending) {
        if (t < 2 * LPR) newrow[t] = nkv;
        lds_barrier();
      }
    }
  };
  if (nt <= 3) {
    // short chunk: every tile in flight at once, none loaded past the end
    // (the two-buffer loop below always issues one tile of lookahead)
    TL b2;
    load(b0, 0);
    load(b1, 1);
    load(b2, 2);
    after_issue();
    process(b0, 0);
    if (nt > 1) process(b1, 1);
    if (nt > 2) process(b2, 2);
  } else {
    load(b0, 0);
    after_issue();
    for (int tt = 0; tt < nt; tt += 2) {
      load(b1, tt + 1);
      process(b0, tt);
      if (tt + 1 >= nt) break;
      load(b0, tt + 2);
      process(b1, tt + 1);
    }
  }

  // ---- combine the row slots of each wave (lanes with the same chunk c)
#pragma unroll
  for (int h = 0; h < GRP; ++h) {
    float M = m[h];
#pragma unroll
    for (int o = LPR; o < 64; o <<= 1) M = fmaxf(M, __shfl_xor(M, o));
    const float f = exp2f(m[h] - (M == -INFINITY ? 0.f : M));
    l[h] *= f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] *= f;
#pragma unroll
    for (int o = LPR; o < 64; o <<= 1) {
      l[h] += __shfl_xor(l[h], o);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] += __shfl_xor(acc[h][e], o);
    }
    m[h] = M;
  }
  if ((t & 63) < LPR) {
#pragma unroll
    for (int h = 0; h < GRP; ++h) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) red_o[wave][h][c * EPL + e] = acc[h][e];
      if (c == 0) {
        red_m[wave][h] = m[h];
        red_l[wave][h] = l[h];
      }
    }
  }
  __syncthreads();

  // ---- combine the four waves; one thread per (head, 16-byte chunk)
  if (t < GRP * LPR) {
    const int h = t / LPR;
    const int cc = t % LPR;
    float M = fmaxf(fmaxf(red_m[0][h], red_m[1][h]), fmaxf(red_m[2][h], red_m[3][h]));
    float fw[4];
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      fw[w] = exp2f(red_m[w][h] - M);          // M is finite: the chunk has rows
      L = fmaf(fw[w], red_l[w][h], L);
    }
    float o[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e)
      o[e] = fw[0] * red_o[0][h][cc * EPL + e] + fw[1] * red_o[1][h][cc * EPL + e] +
             fw[2] * red_o[2][h][cc * EPL + e] + fw[3] * red_o[3][h][cc * EPL + e];
    const int64_t row = (int64_t)qi * a.hq + g * GRP + h;
    if (cnt <= a.split) {
      const float inv = 1.f / L;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] *= inv;
      store_out<BF16, EPL>(a.out, row * HD + cc * EPL, o);
      if (a.lse && cc == 0) a.lse[row] = (M + log2f(L)) * kLn2;
    } else {
      float* dst = a.ws_o + (row * a.max_split + s) * HD + cc * EPL;
#pragma unroll
      for (int e = 0; e < EPL; e += 4)
        *reinterpret_cast<float4*>(dst + e) = make_float4(o[e], o[e + 1], o[e + 2], o[e + 3]);
      if (cc == 0) {
        a.ws_ml[(row * a.max_split + s) * 2] = M;
        a.ws_ml[(row * a.max_split + s) * 2 + 1] = L;
      }
    }
  }
}

// Matrix-core form of decode_kernel for bf16 caches whose kv heads serve
// a group of GRP >= 2 query heads.  The group's queries against the kept
// rows are a small dense contraction: scores S^T = K Q^T (16 rows x 16
// columns, the GRP query heads in the first columns) and O^T += V^T P^T,
// on v_mfma_f32_16x16x32_bf16 and v_mfma_f32_16x16x16_bf16.  The matrix
// cores then do the dot products and the P.V sums that would otherwise be
// most of the vector work per kept byte (measured: the vector form's
// arithmetic, not its loads, set its speed on the GQA workloads).
//
// Layout.  Each wave takes blocks of 16 kept rows (wave w: blocks w, w+4,
// ...), loaded as whole rows (RPI rows a wave instruction, 16 bytes a lane)
// into registers and staged in a 4 KiB LDS area of the wave: K comes back
// as the A operand of S^T = K Q^T (lane l: row l % 16, dims 32c + 8 (l/16)
// .. + 8), V comes back transposed (ds_read_b64_tr_b16) as the A operand
// V^T.  The score result gives lane l the scores of rows 4 (l/16) + r,
// r = 0..3, for query head l % 16 -- the layout of the B operand P^T of the
// second product, so the softmax runs in place.  The next block's K and V
// are in flight while a block is computed; loads are nontemporal (each
// byte is read once).  The online
// softmax keeps a reference max per query head that moves only when the
// block max passes it by more than 2^8 (log2 domain), so the output
// accumulators are rescaled rarely.  Rows (element offsets, and positions
// for per-head masks) come from an LDS table filled at the start, the same
// entries in the same order as decode_kernel reads.  The four waves' states
// meet in LDS at the end, as in decode_kernel, whose output and partial
// formats are kept (the merge kernel serves both).
template <int HD, int GRP, int FORM, bool APPEND>
__global__ void __launch_bounds__(256) decode_mfma_kernel(const int32_t* m0_p, const int32_t* m1_p,
                                                          const int32_t* seq_p, int hkv_p,
                                                          int max_split_p, int cap_p, int split_p,
                                                          const void* k_p, const void* v_p,
                                                          const void* q_p, DecodeArgs a) {
  static_assert(GRP >= 2 && GRP <= 16, "query heads of a group are matrix-core columns");
  constexpr bool MASKED = FORM >= 1;
  constexpr bool PERHEAD = FORM == 2;
  constexpr int NC = HD / 32;         // 32-dim contraction steps of S^T = K Q^T
  constexpr int NB = HD / 16;         // 16-dim output blocks of O^T
  constexpr int CPR = HD / 8;         // 16-byte chunks per row
  constexpr int LPR = CPR;            // output combine: threads per head (8 elements each)

  extern __shared__ int64_t rowoff[];                 // [split] element offsets (+ positions)
  __shared__ float red_m[4][GRP];
  __shared__ float red_l[4][GRP];
  // per-wave V staging during the loop; the waves' outputs afterwards
  constexpr int VST = 16 * HD;                        // bf16 elements per wave
  constexpr int RED = GRP * HD * 2;                   // fp32 outputs per wave, in bf16 units
  __shared__ __attribute__((aligned(16))) uint16_t stage[4 * (VST > RED ? VST : RED)];
  __shared__ u32x4 newrow[2 * CPR];                   // KV append: the new K, V rows

  const int t = threadIdx.x;
  const int wave = t >> 6;
  const int lane = t & 63;
  const int lr = lane & 15;
  const int lg = lane >> 4;

  const int bid = blockIdx.x;
  const int s = bid % max_split_p;
  const int qg = bid / max_split_p;
  const int qi = qg / hkv_p;
  const int g = qg % hkv_p;
  int i_m = 0, P_m = 0, sq_m = 0, cnt_l = 0;
  if constexpr (MASKED) {
    i_m = m0_p[qi];
    P_m = m1_p[qi];
    sq_m = seq_p[qi];
  } else {
    // the query's list, or with one list per kv head this kv head's
    cnt_l = m0_p[a.list_heads > 1 ? qg : qi];
    sq_m = seq_p[qi];
  }
  const int r0 = s * split_p;
  const int lim = cap_p - r0 < split_p ? cap_p - r0 : split_p;   // >= 1

  // ---- stage 0: the group's query rows into LDS as 16 rows (rows past the
  // group zero), chunks swizzled like the V staging; lane l reads its B
  // operand Q^T (query head l % 16) from there for each block
  __shared__ __attribute__((aligned(16))) uint16_t qsh[16 * HD];
  for (int e = t; e < 16 * CPR; e += 256) {
    const int h = e / CPR, ch = e % CPR;
    u32x4 w = u32x4{0u, 0u, 0u, 0u};
    if (h < GRP)
      w = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(q_p) +
                                          (((int64_t)qi * hkv_p + g) * GRP + h) * HD + ch * 8);
    *reinterpret_cast<u32x4*>(qsh + h * HD + ((ch ^ swz<CPR>(h)) * 8)) = w;
  }
  // per-head masks: this lane's head's window and band, and the group's
  // widest, whose keep-set contains every head's
  int Wh = a.W, Bh = a.B, Wg = a.W, Bg = a.B;
  if constexpr (PERHEAD) {
    const int32_t* wb = a.head_wb + 2 * (int64_t)g * GRP;
    Wg = 0;
    Bg = 0;
#pragma unroll
    for (int h = 0; h < GRP; ++h) {
      const int w = wb[2 * h] > 0 ? wb[2 * h] : 0, b = wb[2 * h + 1] > 0 ? wb[2 * h + 1] : 0;
      Wg = w > Wg ? w : Wg;
      Bg = b > Bg ? b : Bg;
      if (h == lr) {
        Wh = w;
        Bh = b;
      }
    }
  }
  const char* kb = reinterpret_cast<const char*>(k_p) + (int64_t)g * a.head_stride * 2;
  const char* vb = reinterpret_cast<const char*>(v_p) + (int64_t)g * a.head_stride * 2;

  int cnt, nrows;
  const int sq = clampi(sq_m, 0, a.n_seq - 1);
  const int32_t* bt = a.block_table ? a.block_table + (int64_t)sq * a.bt_stride : nullptr;
  KeepCF kc{};
  int n_keep = 0, sub_row = -1;
  bool appending = false, stores = false;
  u32x4 nkv = u32x4{0u, 0u, 0u, 0u};
  auto store_new_row = [&]() {
    if (t < 2 * CPR) {
      const int64_t o = row_offset(a, bt, sq, i_m);
      char* base = reinterpret_cast<char*>(const_cast<void*>(t < CPR ? a.k : a.v));
      *reinterpret_cast<u32x4*>(base + ((int64_t)g * a.head_stride + (t % CPR) * 8 + o) * 2) = nkv;
    }
  };
  if constexpr (MASKED) {
    // KV append: a kernel of its own (the code, unused, cost a step ~1 us)
    appending = APPEND && a.k_new != nullptr;
    if (appending && t < 2 * CPR) {
      const void* src = t < CPR ? a.k_new : a.v_new;
      const int64_t off = ((int64_t)qi * a.hkv + g) * HD + (t % CPR) * 8;
      nkv = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(src) + off);
    }
    const bool bad = i_m < 0 || P_m < 0;
    stores = appending && !bad && i_m < a.max_len;
    kc = keep_cf(a.mode, i_m, P_m, Wg, Bg, a.G, bad);
    n_keep = kc.size();
    cnt = n_keep < a.cap ? n_keep : a.cap;
    if (stores && n_keep <= a.cap && n_keep - 1 >= r0 && n_keep - 1 < r0 + lim) sub_row = n_keep - 1 - r0;
    if (r0 >= cnt) {
      if (a.count_out != nullptr && g == 0 && s == 0 && t == 0) a.count_out[qi] = n_keep;
      if (a.ws_cnt && s == 0 && t == 0) a.ws_cnt[(int64_t)qi * a.hkv + g] = n_keep;
      if (stores && a.max_split == 1) store_new_row();
      return;
    }
  } else {
    cnt = cnt_l < a.cap ? cnt_l : a.cap;
    if (r0 >= cnt) return;
  }
  nrows = cnt - r0 < a.split ? cnt - r0 : a.split;

  // ---- stage 1: element offset (and, per-head masks, position) of every
  // row of the chunk into LDS, one round trip for the list entries or
  // block-table entries; with them, before any K/V load is issued, every
  // store the step owes besides its output: the lists (kv-head-0
  // workgroups write the entries of their chunk), the keep-set size for the
  // merge, and the appended row (in the cache and, for this workgroup's own
  // use, in LDS).  No store or conditional load then sits among the K/V
  // loads, so the compiler's wait counts for them stay exact.
  __shared__ int64_t app_off;
  const bool lists_out = MASKED && a.count_out != nullptr && g == 0;
  int32_t* my_out = lists_out ? a.idx_out + (int64_t)qi * a.cap + r0 : nullptr;
  if constexpr (MASKED) {
    if (stores && t == 0) app_off = row_offset(a, bt, sq, i_m);
    if (lists_out && s == 0 && t == 0) a.count_out[qi] = n_keep;
    if (a.ws_cnt && s == 0 && t == 0) a.ws_cnt[(int64_t)qi * a.hkv + g] = n_keep;
    if (appending && t < 2 * CPR) newrow[t] = nkv;
  }
  // (positions follow the offsets: the table holds min(split, cap) rows)
  int32_t* rowpos = reinterpret_cast<int32_t*>(rowoff + (split_p < cap_p ? split_p : cap_p));
  {
    // IPT rows a thread a round; only as many rows as the chunk has are
    // computed (a closed-form entry costs an integer division)
    const int32_t* myidx = MASKED ? nullptr : m1_p + (int64_t)(a.list_heads > 1 ? qg : qi) * cap_p + r0;
    auto fill = [&](auto ipt) {
      constexpr int IPT = decltype(ipt)::value;
      for (int base = 0; base < nrows; base += IPT * 256) {
        int jj[IPT];
#pragma unroll
        for (int u = 0; u < IPT; ++u) {
          const int r = base + u * 256 + t;
          const int rc = r < nrows ? r : nrows - 1;
          int j;
          if constexpr (MASKED) j = kc.entry(r0 + rc);
          else j = myidx[rc];
          jj[u] = clampi(j, 0, a.max_len - 1);
          if constexpr (PERHEAD) {
            if (r < nrows) rowpos[r] = j;
          }
          if (lists_out && r < nrows) my_out[r] = j;
        }
        int64_t o[IPT];
        if (bt) {
          int pg[IPT];
#pragma unroll
          for (int u = 0; u < IPT; ++u) pg[u] = bt[jj[u] >> a.ps_shift];
#pragma unroll
          for (int u = 0; u < IPT; ++u)
            o[u] = (int64_t)clampi(pg[u], 0, a.n_pages - 1) * a.page_stride +
                   (int64_t)(jj[u] & a.ps_mask) * a.slot_stride;
        } else {
#pragma unroll
          for (int u = 0; u < IPT; ++u) o[u] = (int64_t)sq * a.page_stride + (int64_t)jj[u] * a.slot_stride;
        }
#pragma unroll
        for (int u = 0; u < IPT; ++u) {
          const int r = base + u * 256 + t;
          if (r < nrows) rowoff[r] = o[u];
        }
      }
    };
    if (nrows <= 256) fill(std::integral_constant<int, 1>{});
    else if (nrows <= 512) fill(std::integral_constant<int, 2>{});
    else fill(std::integral_constant<int, 4>{});
  }
  __syncthreads();
  if constexpr (MASKED) {
    // KV append: one chunk -- this one -- or, with several, the chunk that
    // attends the last entry (position i itself when the list is not cut)
    if (stores && (a.max_split == 1 || (cnt - 1) / a.split == s) && t < 2 * CPR) {
      char* base = reinterpret_cast<char*>(const_cast<void*>(t < CPR ? a.k : a.v));
      *reinterpret_cast<u32x4*>(base + ((int64_t)g * a.head_stride + (t % CPR) * 8 + app_off) * 2) = nkv;
    }
  }

  // B operand chunk c of S^T = K Q^T: query head l % 16, dims 32c + 8 (l / 16)
  auto qop = [&](int c, int lr_, int lg_) {
    return *reinterpret_cast<const bf16x8*>(qsh + lr_ * HD + (((4 * c + lg_) ^ swz<CPR>(lr_)) * 8));
  };
  // KV append: scores of the new K row for this lane's query head, on the
  // matrix core with the same operand layout as every block's rows
  float s_new = 0.f;
  if constexpr (MASKED) {
    if (sub_row >= 0) {
      f32x4 sn = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c)
        sn = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, newrow[4 * c + lg]), qop(c, lr, lg),
                                                     sn, 0, 0, 0);
      s_new = sn[0];
    }
  }

  const int nblk = (nrows + 15) / 16;
  uint16_t* vst = stage + wave * (VST > RED ? VST : RED);

  // ---- stage 2: blocks of 16 rows, the next one in flight per wave
  float m = -INFINITY, lsum = 0.f;
  f32x4 o[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One K and one V buffer: the next block's K is issued as soon as this
  // block's K is staged, its V once this block's V is staged, so every wave
  // has a block of loads in flight while it computes; sixteen waves a CU
  // then hold 128 KiB of reads in flight.  Loads are whole rows, RPI rows an
  // instruction (lane l: row c RPI + l / CPR, 16-byte chunk l % CPR): rows
  // read in 64-byte pieces, as the matrix-core operand layout would have
  // them, measured 28 % slower on the same data.
  constexpr int RPI = 64 / CPR;
  const int nrow_l = lane / CPR, nchk_l = lane % CPR;
  u32x4 kk[NC], vv[NC];
  auto row_bytes = [&](int blk, int c) {
    const int row = blk * 16 + c * RPI + nrow_l;
    return rowoff[row < nrows ? row : nrows - 1] * 2 + nchk_l * 16;
  };
  auto load_k = [&](int blk) {
#pragma unroll
    for (int c = 0; c < NC; ++c)
      kk[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kb + row_bytes(blk, c)));
  };
  auto load_v = [&](int blk) {
#pragma unroll
    for (int c = 0; c < NC; ++c)
      vv[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vb + row_bytes(blk, c)));
  };
  // a block's rows as loaded to the wave's staging area, row-major with
  // swizzled chunks
  auto stage_rows = [&](uint16_t* st, const u32x4 (&x)[NC], int lane_) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int r = c * RPI + lane_ / CPR;
      *reinterpret_cast<u32x4*>(st + r * HD + (((lane_ % CPR) ^ swz<CPR>(r)) * 8)) = x[c];
    }
  };
  auto process = [&](int blk) {
    // LDS addresses (query operand, V staging, transposing reads) are taken
    // from an offset the compiler cannot see as loop-invariant, so they are
    // recomputed per block instead of being held in registers through the
    // loop (which spilled)
    int zo = 0;
    __asm__ volatile("" : "+v"(zo));
    uint16_t* const vsw = vst;
    // lane coordinates the compiler cannot see as loop-invariant: every LDS
    // offset derived from them is recomputed per block (a few integer ops)
    // instead of being held in registers through the loop
    const int lane_z = lane + zo, lr_z = lane_z & 15, lg_z = lane_z >> 4;
    // K through the staging area into the A operand of S^T = K Q^T (lane l:
    // row l % 16, dims 32c + 8 (l / 16) .. + 8)
    stage_rows(vsw, kk, lane_z);
    // the refill of this K buffer stays behind the stores that read it (an
    // empty asm that orders memory: hoisted above them, the loads would
    // force a copy of the buffer and a wait for every load in flight)
    __asm__ volatile("" ::: "memory");
    load_k(blk + 4);
    f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const bf16x8 ka =
          *reinterpret_cast<const bf16x8*>(vsw + lr_z * HD + (((4 * c + lg_z) ^ swz<CPR>(lr_z)) * 8));
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qop(c, lr_z, lg_z), sc, 0, 0, 0);
    }
    // V over the K rows (the operand reads above precede these stores: LDS
    // operations of a wave run in order)
    stage_rows(vsw, vv, lane_z);
    if constexpr (MASKED) {
      // KV append: the new token's row is row sub_row % 16 of its block.
      // Its V row goes over the staged one, and its scores are the ones
      // computed from its K row at the start (the same products on the same
      // matrix core, so the same values).  The block test is uniform.
      if (sub_row >= 0 && (sub_row >> 4) == blk) {
        const int rr = sub_row & 15;
        if (lr == rr) {
#pragma unroll
          for (int c = 0; c < NC; ++c)
            *reinterpret_cast<u32x4*>(vsw + lr_z * HD + (((4 * c + lg_z) ^ swz<CPR>(lr_z)) * 8)) =
                newrow[CPR + 4 * c + lg];
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[r] = (lg == (rr >> 2) && r == (rr & 3)) ? s_new : sc[r];
      }
    }
    // likewise the refill of the V buffer stays behind its staging stores
    __asm__ volatile("" : "+v"(sc)::"memory");
    load_v(blk + 4);
    float sv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = blk * 16 + 4 * lg + r;
      bool keep = row < nrows;
      if constexpr (PERHEAD) {
        const int j = rowpos[row < nrows ? row : 0];
        const int64_t d = (int64_t)i_m - j;
        keep = keep && (a.mode == DA_MODE_DENSE || j < P_m || (d <= Wh && window_keep(a.mode, d, Bh, a.G)));
      }
      sv[r] = keep ? sc[r] * a.qscale : -INFINITY;
    }
    const float mt = max_over_row_groups(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
    if (__any(mt > m + 8.f)) {
      const float mn = fmaxf(m, mt);
      const float alpha = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m - mn);
      lsum *= alpha;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[nb][r] *= alpha;
      m = mn;
    }
    const float mref = m == -INFINITY ? 0.f : m;
    v4i16 pb;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float p = __builtin_amdgcn_exp2f(sv[r] - mref);
      lsum += p;
      pb[r] = __builtin_bit_cast(short, (__bf16)p);
    }
    // O^T += V^T P^T, one 16-dim block at a time
    const int vr = 4 * lg_z + (lr_z >> 2);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const uint16_t* pv = vsw + vr * HD + (((2 * nb + ((lr_z & 3) >> 1)) ^ swz<CPR>(vr)) * 8) + (lr_z & 1) * 4;
      const v4i16 av = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(pv));
      o[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, pb, o[nb], 0, 0, 0);
    }
  };
  // Every load is issued unconditionally (blocks past the chunk read its
  // last row again: cache hits), so the compiler's wait counts never merge
  // paths with different numbers of loads in flight.
  if (wave < nblk) {
    load_k(wave);
    load_v(wave);
    for (int blk = wave; blk < nblk; blk += 4) process(blk);
  }

  // ---- combine: per query head the wave's max, sum and output, then the
  // four waves (LDS), then the output or the chunk's partial
  lsum = sum_over_row_groups(lsum);
  __syncthreads();                      // every wave done with its V staging
  float* redo = reinterpret_cast<float*>(stage) + wave * (GRP * HD);
  if (lr < GRP) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) redo[lr * HD + 16 * nb + 4 * lg + r] = o[nb][r];
    if (lg == 0) {
      red_m[wave][lr] = m;
      red_l[wave][lr] = lsum;
    }
  }
  __syncthreads();
  if (t < GRP * LPR) {
    const int h = t / LPR;
    const int cc = t % LPR;
    const float* ro = reinterpret_cast<const float*>(stage);
    float M = fmaxf(fmaxf(red_m[0][h], red_m[1][h]), fmaxf(red_m[2][h], red_m[3][h]));
    const float Mr = M == -INFINITY ? 0.f : M;
    float fw[4];
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      fw[w] = exp2f(red_m[w][h] - Mr);
      L = fmaf(fw[w], red_l[w][h], L);
    }
    float ov[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) x = fmaf(fw[w], ro[(w * GRP + h) * HD + cc * 8 + e], x);
      ov[e] = x;
    }
    const int64_t row = (int64_t)qi * a.hq + g * GRP + h;
    if (cnt <= a.split) {
      const float inv = 1.f / L;
#pragma unroll
      for (int e = 0; e < 8; ++e) ov[e] *= inv;
      store_out<true, 8>(a.out, row * HD + cc * 8, ov);
      if (a.lse && cc == 0) a.lse[row] = (M + log2f(L)) * kLn2;
    } else {
      float* dst = a.ws_o + (row * a.max_split + s) * HD + cc * 8;
#pragma unroll
      for (int e = 0; e < 8; e += 4)
        *reinterpret_cast<float4*>(dst + e) = make_float4(ov[e], ov[e + 1], ov[e + 2], ov[e + 3]);
      if (cc == 0) {
        a.ws_ml[(row * a.max_split + s) * 2] = M;
        a.ws_ml[(row * a.max_split + s) * 2 + 1] = L;
      }
    }
  }
}

// Log-sum-exp merge of the chunk partials of one (query, head): one wave.
// Lanes first read the chunks' (max, sum) pairs in parallel, then every lane
// accumulates its HD/64 output elements over the chunks.
template <bool BF16, int HD>
__global__ void __launch_bounds__(64) merge_kernel(DecodeArgs a) {
  constexpr int EPT = HD / 64;
  const int row = blockIdx.x;           // query * hq + head
  const int qi = row / a.hq;
  const int lane = threadIdx.x;
  int cnt = a.mcount[a.mcount_per_head ? (int64_t)qi * a.hkv + (row % a.hq) / (a.hq / a.hkv) : qi];
  cnt = cnt < a.cap ? cnt : a.cap;
  if (cnt <= a.split) return;           // written directly by decode_kernel
  const int ns = (cnt + a.split - 1) / a.split;
  const float* ml = a.ws_ml + (int64_t)row * a.max_split * 2;
  float M = -INFINITY;
  for (int k = lane; k < ns; k += 64) M = fmaxf(M, ml[2 * k]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  float L = 0.f;
  for (int k = lane; k < ns; k += 64) L += exp2f(ml[2 * k] - M) * ml[2 * k + 1];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) L += __shfl_xor(L, o);
  float o[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) o[e] = 0.f;
  const float* src = a.ws_o + (int64_t)row * a.max_split * HD + lane * EPT;
#pragma unroll 4
  for (int k = 0; k < ns; ++k) {
    const float w = exp2f(ml[2 * k] - M);
#pragma unroll
    for (int e = 0; e < EPT; ++e) o[e] = fmaf(w, src[(int64_t)k * HD + e], o[e]);
  }
  const float inv = 1.f / L;
  if constexpr (BF16) {
    uint16_t* dst = reinterpret_cast<uint16_t*>(a.out) + (int64_t)row * HD + lane * EPT;
#pragma unroll
    for (int e = 0; e < EPT; ++e) dst[e] = (uint16_t)f32_to_bf16(o[e] * inv);
  } else {
    float* dst = reinterpret_cast<float*>(a.out) + (int64_t)row * HD + lane * EPT;
#pragma unroll
    for (int e = 0; e < EPT; ++e) dst[e] = o[e] * inv;
  }
  if (a.lse && lane == 0) a.lse[row] = (M + log2f(L)) * kLn2;
}

typedef void (*decode_fn)(const int32_t*, const int32_t*, const int32_t*, int, int, int, int,
                          const void*, const void*, const void*, DecodeArgs);  // ..., k, v, q, args
typedef void (*merge_fn)(DecodeArgs);

// Tile depth: NP passes per tile (two tiles in flight per workgroup).
template <bool BF16, int HD, int GRP, int FORM>
static decode_fn pick_np(int np) {
  if (np <= 2) return decode_kernel<BF16, HD, GRP, 2, FORM>;
  if (np == 3) return decode_kernel<BF16, HD, GRP, 3, FORM>;
  return decode_kernel<BF16, HD, GRP, 4, FORM>;
}

template <bool BF16, int HD, int FORM>
static decode_fn pick_grp(int grp, int np) {
  switch (grp) {
    case 1: return pick_np<BF16, HD, 1, FORM>(np);
    case 2: return pick_np<BF16, HD, 2, FORM>(np);
    case 4: return pick_np<BF16, HD, 4, FORM>(np);
    default: return pick_np<BF16, HD, 8, FORM>(np);
  }
}

// Matrix-core kernel for bf16 groups of 2, 4 or 8 query heads a kv head.
template <int FORM, bool APPEND>
static decode_fn pick_mfma_a(int head_dim, int grp) {
  if (head_dim == 64)
    return grp == 2 ? decode_mfma_kernel<64, 2, FORM, APPEND>
                    : grp == 4 ? decode_mfma_kernel<64, 4, FORM, APPEND> : decode_mfma_kernel<64, 8, FORM, APPEND>;
  return grp == 2 ? decode_mfma_kernel<128, 2, FORM, APPEND>
                  : grp == 4 ? decode_mfma_kernel<128, 4, FORM, APPEND> : decode_mfma_kernel<128, 8, FORM, APPEND>;
}

template <int FORM>
static decode_fn pick_mfma(int head_dim, int grp, bool append) {
  if constexpr (FORM == 0) return pick_mfma_a<0, false>(head_dim, grp);
  else return append ? pick_mfma_a<FORM, true>(head_dim, grp) : pick_mfma_a<FORM, false>(head_dim, grp);
}

static bool use_mfma(da_dtype dtype, int grp) { return dtype == DA_BF16 && grp >= 2; }

template <int FORM>
static decode_fn pick_kernel(da_dtype dtype, int head_dim, int grp, int np) {
  if (dtype == DA_BF16)
    return head_dim == 64 ? pick_grp<true, 64, FORM>(grp, np) : pick_grp<true, 128, FORM>(grp, np);
  return head_dim == 64 ? pick_grp<false, 64, FORM>(grp, np) : pick_grp<false, 128, FORM>(grp, np);
}

// Workgroups of `k` (256 threads, `lds` bytes of dynamic LDS) the current
// device holds at once, 0 if unknown.  Cached: the answer depends only on the
// kernel, the LDS size and the device.
static int64_t resident_blocks(decode_fn k, size_t lds) {
  struct Entry { decode_fn k; size_t lds; int dev; int64_t n; };
  static std::mutex mu;
  static Entry cache[64];
  static int used = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  for (int e = 0; e < used; ++e)
    if (cache[e].k == k && cache[e].lds == lds && cache[e].dev == dev) return cache[e].n;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(k), 256, lds) !=
          hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  const int64_t n = (int64_t)cus * per_cu;
  if (used < 64) cache[used++] = Entry{k, lds, dev, n};
  return n;
}

// Tile depth (2, 3 or 4 passes) for chunks of `chunk` rows; `kernel_for(np)`
// gives the kernel of each depth, `grid` the workgroups of the launch.
// Row slots past a chunk's end still issue their (redundant) loads, and on
// this part the per-CU load path is what such slots cost, so among the
// candidates the depth leaving the fewest empty slots wins, ties going to the
// deeper tile.  A chunk that fits in three tiles at some depth has every tile
// in flight at once: the candidates are those depths.  Longer chunks stream
// through the two-buffer loop, where a grid that is resident all at once
// measured faster than a deeper tile (1024 workgroups of 300-row chunks, four
// query heads a kv head: 2 passes at 121 VGPRs, 4 workgroups a CU, 5-7 %
// faster than 3 or 4 passes at 3 or 2): the candidates are the depths whose
// kernel holds the whole grid at once, or all depths if none does.
template <typename KernelFor>
static int tile_depth(int chunk, int rows_per_pass, int64_t grid, size_t lds, KernelFor kernel_for) {
  auto pick = [&](auto ok) {
    int best = 0;
    int64_t best_slots = INT64_MAX;
    for (int np = 4; np >= 2; --np) {
      const int64_t tile = (int64_t)np * rows_per_pass;
      const int64_t slots = (chunk + tile - 1) / tile * tile;
      if (ok(np, slots / tile) && slots < best_slots) {
        best_slots = slots;
        best = np;
      }
    }
    return best;
  };
  int np = pick([](int, int64_t tiles) { return tiles <= 3; });
  if (np) return np;
  np = pick([&](int d, int64_t) { return resident_blocks(kernel_for(d), lds) >= grid; });
  if (np) return np;
  return pick([](int, int64_t) { return true; });
}

// Longest chunk one workgroup takes: its row offsets live in LDS (8 B each).
constexpr int kMaxSplit = 4096;

static int64_t n_splits(int32_t cap, int32_t split) { return (int64_t(cap) + split - 1) / split; }

// Checks the arguments shared by both decode entry points and fills `a`;
// DA_OK or a negative status (nothing launched).
static int prepare_decode(DecodeArgs& a, const void* q, da_dtype dtype, int32_t n_q, int32_t hq,
                          int32_t hkv, int32_t head_dim, float scale, const da_kv_cache* kv,
                          const int32_t* seq, int32_t cap, int32_t split, void* out, float* lse,
                          void* workspace, int64_t ws_bytes) {
  if (n_q < 0) return fail(DA_EINVAL, "n_q=%d < 0", n_q);
  if (hq < 1 || hkv < 1 || hq % hkv) return fail(DA_EINVAL, "hq=%d hkv=%d: need hq %% hkv == 0", hq, hkv);
  if (!kv) return fail(DA_EINVAL, "kv descriptor is NULL");
  if (cap < 1 || split < 1) return fail(DA_EINVAL, "cap=%d split=%d must be >= 1", cap, split);
  if (dtype != DA_F32 && dtype != DA_BF16) return fail(DA_ENOTSUP, "dtype %d not supported", (int)dtype);
  if (head_dim != 64 && head_dim != 128) return fail(DA_ENOTSUP, "head_dim %d not in {64, 128}", head_dim);
  const int grp = hq / hkv;
  if (grp != 1 && grp != 2 && grp != 4 && grp != 8)
    return fail(DA_ENOTSUP, "hq/hkv=%d not in {1, 2, 4, 8}", grp);
  if (split > kMaxSplit) return fail(DA_ENOTSUP, "split=%d > %d", split, kMaxSplit);
  if (kv->block_table) {
    if (!is_pow2(kv->page_size)) return fail(DA_EINVAL, "page_size=%d not a power of two", kv->page_size);
    if (kv->bt_stride < 1) return fail(DA_EINVAL, "bt_stride=%d < 1", kv->bt_stride);
  }
  if (kv->page_stride < 0 || kv->head_stride < 0 || kv->slot_stride < 0)
    return fail(DA_EINVAL, "negative cache stride");
  if (kv->n_seq < 1 || kv->n_pages < 1 || kv->max_len < 1)
    return fail(DA_EINVAL, "cache extents n_seq=%d n_pages=%d max_len=%d must be >= 1",
                kv->n_seq, kv->n_pages, kv->max_len);
  if (kv->block_table && (int64_t)kv->max_len > (int64_t)kv->bt_stride * kv->page_size)
    return fail(DA_EINVAL, "max_len=%d exceeds bt_stride * page_size", kv->max_len);
  if (!kv->block_table && kv->n_pages < kv->n_seq)
    return fail(DA_EINVAL, "contiguous cache: n_pages must cover n_seq");
  if (n_q > 0 && (!q || !out || !seq || !kv->k || !kv->v))
    return fail(DA_EINVAL, "q, out, seq, kv->k and kv->v must be non-NULL");
  const int esz = dtype == DA_BF16 ? 2 : 4;
  if (((kv->page_stride | kv->head_stride | kv->slot_stride) * esz) % 16 ||
      ((uintptr_t)kv->k | (uintptr_t)kv->v | (uintptr_t)q | (uintptr_t)out) % 16)
    return fail(DA_EINVAL, "cache rows, q and out must be 16-byte aligned");
  const int64_t ns = n_splits(cap, split);
  const WsLayout wl = ws_layout(n_q, hq, head_dim, ns);
  if (wl.bytes > 0 && (!workspace || ws_bytes < wl.bytes))
    return fail(DA_ECAPACITY, "workspace %lld bytes < %lld needed", (long long)ws_bytes, (long long)wl.bytes);
  if (wl.bytes > 0 && (uintptr_t)workspace % 256) return fail(DA_EINVAL, "workspace not 256-byte aligned");
  const int64_t blocks = int64_t(n_q) * hkv * ns;
  if (blocks > 0x7fffffff) return fail(DA_ENOTSUP, "grid of %lld workgroups too large", (long long)blocks);

  a = DecodeArgs{};
  a.list_heads = 1;
  a.q = q;
  a.k = kv->k;
  a.v = kv->v;
  a.page_stride = kv->page_stride;
  a.head_stride = kv->head_stride;
  a.slot_stride = kv->slot_stride;
  a.block_table = kv->block_table;
  a.bt_stride = kv->bt_stride;
  a.ps_shift = kv->block_table ? ilog2(kv->page_size) : 0;
  a.ps_mask = kv->block_table ? kv->page_size - 1 : 0x7fffffff;
  a.n_seq = kv->block_table ? kv->n_seq : kv->n_pages;
  a.n_pages = kv->n_pages;
  a.max_len = kv->max_len;
  a.seq = seq;
  a.n_q = n_q;
  a.hq = hq;
  a.hkv = hkv;
  a.cap = cap;
  a.split = split;
  a.max_split = (int)ns;
  a.qscale = scale * kLog2e;
  a.out = out;
  a.lse = lse;
  char* ws = reinterpret_cast<char*>(workspace);
  a.ws_o = wl.bytes ? reinterpret_cast<float*>(ws + wl.o_off) : nullptr;
  a.ws_ml = wl.bytes ? reinterpret_cast<float*>(ws + wl.ml_off) : nullptr;
  a.ws_cnt = wl.bytes ? reinterpret_cast<int32_t*>(ws + wl.cnt_off) : nullptr;
  return DA_OK;
}

// Launches the decode kernel (and, when a list spans several chunks, the
// merge) for prepared arguments.
template <int FORM>
static int launch_decode(const DecodeArgs& a, da_dtype dtype, int head_dim, void* stream) {
  const int esz = dtype == DA_BF16 ? 2 : 4;
  const int chunk = a.split < a.cap ? a.split : a.cap;
  const int64_t blocks = int64_t(a.n_q) * a.hkv * a.max_split;
  const int grp = a.hq / a.hkv;
  decode_fn dk;
  size_t lds;
  if (use_mfma(dtype, grp)) {
    // row table in LDS: offsets, and positions for per-head masks
    lds = (size_t)chunk * (sizeof(int64_t) + (FORM == 2 ? sizeof(int32_t) : 0));
    dk = pick_mfma<FORM>(head_dim, grp, a.k_new != nullptr);
  } else {
    // row offsets in LDS: every list, and the mask form of a paged cache
    lds = FORM >= 1 && !a.block_table ? 0 : (size_t)chunk * sizeof(int64_t);
    const int np = tile_depth(chunk, 256 / (head_dim * esz / 16), blocks, lds, [&](int d) {
      return pick_kernel<FORM>(dtype, head_dim, grp, d);
    });
    dk = pick_kernel<FORM>(dtype, head_dim, grp, np);
  }
  const merge_fn mk = dtype == DA_BF16 ? (head_dim == 64 ? merge_kernel<true, 64> : merge_kernel<true, 128>)
                                       : (head_dim == 64 ? merge_kernel<false, 64> : merge_kernel<false, 128>);
  const int32_t* m0 = FORM >= 1 ? a.pos : a.count;
  const int32_t* m1 = FORM >= 1 ? a.prompt : a.idx;
  hipLaunchKernelGGL(dk, dim3((unsigned)blocks), dim3(256), lds, (hipStream_t)stream, m0, m1, a.seq,
                     a.hkv, a.max_split, a.cap, a.split, a.k, a.v, a.q, a);
  int rc = check_launch("decode_kernel");
  if (rc || a.max_split <= 1) return rc;
  hipLaunchKernelGGL(mk, dim3((unsigned)(int64_t(a.n_q) * a.hq)), dim3(64), 0, (hipStream_t)stream, a);
  return check_launch("merge_kernel");
}

}  // namespace da

using namespace da;

extern "C" int64_t da_decode_workspace_bytes(int32_t n_q, int32_t hq, int32_t head_dim,
                                             int32_t cap, int32_t split) {
  if (n_q < 0 || hq < 1 || head_dim < 1 || cap < 1 || split < 1)
    return fail(DA_EINVAL, "workspace sizing: invalid sizes");
  clear_error();
  return ws_layout(n_q, hq, head_dim, n_splits(cap, split)).bytes;
}

extern "C" int da_sparse_decode_attn(const void* q, da_dtype dtype, int32_t n_q, int32_t hq,
                                     int32_t hkv, int32_t head_dim, float scale,
                                     const da_kv_cache* kv, const int32_t* seq,
                                     const int32_t* count, const int32_t* idx, int32_t cap,
                                     int32_t list_heads, int32_t split, void* out, float* lse,
                                     void* workspace, int64_t ws_bytes, void* stream) {
  DecodeArgs a;
  int rc = prepare_decode(a, q, dtype, n_q, hq, hkv, head_dim, scale, kv, seq, cap, split, out, lse,
                          workspace, ws_bytes);
  if (rc) return rc;
  if (n_q > 0 && (!count || !idx)) return fail(DA_EINVAL, "count and idx must be non-NULL");
  if (list_heads != 1 && list_heads != hkv)
    return fail(DA_EINVAL, "list_heads=%d must be 1 or hkv=%d", list_heads, hkv);
  clear_error();
  if (n_q == 0) return DA_OK;
  a.count = count;
  a.idx = idx;
  a.list_heads = list_heads;
  a.mcount = count;                     // the merge reads the lists' counts
  a.mcount_per_head = list_heads > 1;
  a.ws_cnt = nullptr;
  return launch_decode<0>(a, dtype, head_dim, stream);
}

namespace da {

// Scratch memory of the allocation-free entry point: the decode workspace
// (chunk partials and keep-set sizes) in a file-scope device array, one
// copy per GPU, alive until the process ends.  Host code never uses the
// array's name as an address: the device address of each GPU's copy comes
// from hipGetSymbolAddress, taken once per device with that device current.
constexpr int64_t kScratchBytes = int64_t(32) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;

// This device's scratch address, or nullptr with the error recorded.
static void* scratch_ptr() {
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    fail(DA_EHIP, "scratch: no current device (or device id >= %d)", kMaxDevices);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      fail(DA_EHIP, "scratch: hipGetSymbolAddress: %s", hipGetErrorString(e));
      return nullptr;
    }
    ptrs[dev] = p;
  }
  return ptrs[dev];
}

}  // namespace da

extern "C" int64_t da_decode_scratch_bytes(void) { return kScratchBytes; }

extern "C" int da_sparse_decode_attn_masked(const da_mask* m, const void* q, da_dtype dtype,
                                            int32_t n_q, int32_t hq, int32_t hkv, int32_t head_dim,
                                            float scale, const da_kv_cache* kv, const int32_t* seq,
                                            const int32_t* pos, const int32_t* prompt_len,
                                            const int32_t* head_wb,
                                            const void* k_new, const void* v_new,
                                            int32_t cap, int32_t split, int32_t* count, int32_t* idx,
                                            void* out, float* lse, void* workspace, int64_t ws_bytes,
                                            void* stream) {
  int rc = check_mask(m);
  if (rc) return rc;
  if (!m->causal) return fail(DA_ENOTSUP, "decode needs a causal mask");
  DecodeArgs a;
  rc = prepare_decode(a, q, dtype, n_q, hq, hkv, head_dim, scale, kv, seq, cap, split, out, lse,
                      workspace, ws_bytes);
  if (rc) return rc;
  if (n_q > 0 && (!pos || !prompt_len)) return fail(DA_EINVAL, "pos and prompt_len must be non-NULL");
  if ((count == nullptr) != (idx == nullptr))
    return fail(DA_EINVAL, "count and idx must both be given or both be NULL");
  if ((k_new == nullptr) != (v_new == nullptr))
    return fail(DA_EINVAL, "k_new and v_new must both be given or both be NULL");
  if (head_wb && count)
    return fail(DA_EINVAL, "per-head masks give per-head keep-sets: no per-query lists");
  if (head_wb && !use_mfma(dtype, hq / (hkv > 0 ? hkv : 1)) && hq != hkv)
    return fail(DA_ENOTSUP, "per-query-head masks with groups of query heads need bf16");
  if (((uintptr_t)k_new | (uintptr_t)v_new) % 16) return fail(DA_EINVAL, "k_new and v_new must be 16-byte aligned");
  clear_error();
  if (n_q == 0) return DA_OK;
  a.k_new = k_new;
  a.v_new = v_new;
  a.pos = pos;
  a.prompt = prompt_len;
  a.mode = m->mode;
  a.W = m->W;
  a.B = m->B;
  a.G = m->G;
  a.count_out = count;
  a.idx_out = idx;
  a.mcount = a.ws_cnt;                  // written by the decode kernel when there is a merge
  a.mcount_per_head = 1;
  a.head_wb = head_wb;
  return head_wb ? launch_decode<2>(a, dtype, head_dim, stream)
                 : launch_decode<1>(a, dtype, head_dim, stream);
}

extern "C" int da_sparse_decode_attn_masked_noalloc(const da_mask* m, const void* q, da_dtype dtype,
                                                    int32_t n_q, int32_t hq, int32_t hkv,
                                                    int32_t head_dim, float scale,
                                                    const da_kv_cache* kv, const int32_t* seq,
                                                    const int32_t* pos, const int32_t* prompt_len,
                                                    const int32_t* head_wb, const void* k_new,
                                                    const void* v_new, int32_t cap, int32_t split,
                                                    int32_t* count, int32_t* idx, void* out,
                                                    float* lse, void* stream) {
  if (n_q < 0 || hq < 1 || head_dim < 1 || cap < 1 || split < 1)
    return fail(DA_EINVAL, "n_q=%d hq=%d head_dim=%d cap=%d split=%d", n_q, hq, head_dim, cap, split);
  const int64_t need = ws_layout(n_q, hq, head_dim, n_splits(cap, split)).bytes;
  if (need > kScratchBytes)
    return fail(DA_ECAPACITY, "these sizes need %lld bytes of scratch; the allocation-free call has %lld",
                (long long)need, (long long)kScratchBytes);
  void* ws = nullptr;
  if (need > 0 && n_q > 0) {
    ws = scratch_ptr();
    if (!ws) return DA_EHIP;
  }
  return da_sparse_decode_attn_masked(m, q, dtype, n_q, hq, hkv, head_dim, scale, kv, seq, pos,
                                      prompt_len, head_wb, k_new, v_new, cap, split, count, idx, out,
                                      lse, ws, ws ? kScratchBytes : 0, stream);
}
