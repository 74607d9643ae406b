// keepset_build: per-query (or per (query, head)) ascending KV index lists
// and maximal runs.
//
// One wave per list.  The prompt part [0, min(P, L)) is written directly;
// the window part [max(P, i - W), i] (plus future keys within B in the matrix
// form) is scanned 64 positions at a time: each lane tests one position with
// window_keep(), a ballot gives the kept lanes and a popcount of the lanes
// below gives each kept position its slot, so the list comes out ascending
// with no sort and no atomics.  Run ends are found the same way; each end
// lane walks back to its run's first position (runs inside the window are
// at most a band wide, 2B + 1 positions, unless bands overlap).
#include "common.h"

namespace da {

struct KeepsetArgs {
  int mode, W, B, G, causal;
  int n_q, n_keys, cap, max_runs;
  int n_heads;              // lists per query: list q * n_heads + h
  const int32_t* head_wb;   // (W, B) of head h at [2h], [2h + 1], or null
  const int32_t* pos;
  const int32_t* prompt;
  int32_t* count;
  int32_t* idx;
  int32_t* n_runs;
  int32_t* runs;
};

// The position and prompt-length arrays and the query count also come as
// leading arguments, which the hardware preloads into SGPRs (the library is
// built with kernel-argument preloading): a wave reads its query's position
// and prompt length without first waiting for the argument block.
__global__ void __launch_bounds__(256) keepset_kernel(const int32_t* pos, const int32_t* prompt, int n_q,
                                                      KeepsetArgs a) {
  const int lane = threadIdx.x & 63;
  // list q * n_heads + h: query q under head h's window and band
  const int64_t q = blockIdx.x * (int64_t)4 + (threadIdx.x >> 6);
  if (q >= (int64_t)n_q * a.n_heads) return;
  const int qq = (int)(q / a.n_heads);
  const int hh = (int)(q % a.n_heads);
  int Wh = a.W, Bh = a.B;
  if (a.head_wb) {
    Wh = a.head_wb[2 * hh] > 0 ? a.head_wb[2 * hh] : 0;
    Bh = a.head_wb[2 * hh + 1] > 0 ? a.head_wb[2 * hh + 1] : 0;
  }
  const int i = pos[qq];
  const int P = prompt[qq];
  const bool bad = i < 0 || P < 0 || (!a.causal && i >= a.n_keys);
  if (bad) {
    if (lane == 0) {
      a.count[q] = 0;
      if (a.n_runs) a.n_runs[q] = 0;
    }
    return;
  }
  // positions and window ends in 64 bits: i + 1 and i + B may pass INT32_MAX
  const int64_t L = a.causal ? (int64_t)i + 1 : (int64_t)a.n_keys;
  int32_t* my_idx = a.idx + q * a.cap;
  int32_t* my_runs = a.runs ? a.runs + q * a.max_runs * 2 : nullptr;

  int64_t Pc, wlo, whi;
  if (a.mode == DA_MODE_DENSE) {
    Pc = L;           // everything up to L is one run
    wlo = 1;
    whi = 0;          // empty window
  } else {
    Pc = P < L ? (int64_t)P : L;
    wlo = (int64_t)i - Wh > Pc ? (int64_t)i - Wh : Pc;
    whi = a.causal ? (int64_t)i : (L - 1 < (int64_t)i + Bh ? L - 1 : (int64_t)i + Bh);
  }

  const int64_t pw = Pc < a.cap ? Pc : (int64_t)a.cap;
  for (int64_t r = lane; r < pw; r += 64) my_idx[r] = (int32_t)r;

  // The prompt run is run 0 unless the first window position continues it.
  const bool joins = Pc > 0 && wlo == Pc && wlo <= whi &&
                     window_keep(a.mode, i - wlo, Bh, a.G);
  int nr = 0;
  if (Pc > 0 && !joins) {
    if (lane == 0 && my_runs && a.max_runs > 0) {
      my_runs[0] = 0;
      my_runs[1] = (int32_t)Pc;
    }
    nr = 1;
  }

  int64_t n = Pc;
  const uint64_t below = (uint64_t(1) << lane) - 1;
  for (int64_t base = wlo; base <= whi; base += 64) {
    const int64_t j = base + lane;
    const bool kp = j <= whi && window_keep(a.mode, i - j, Bh, a.G);
    const uint64_t kb = __ballot(kp);
    if (kp) {
      const int64_t slot = n + __popcll(kb & below);
      if (slot < a.cap) my_idx[slot] = (int32_t)j;
    }
    n += __popcll(kb);

    const bool next = j + 1 <= whi && window_keep(a.mode, i - j - 1, Bh, a.G);
    const bool end = kp && !next;
    const uint64_t eb = __ballot(end);
    if (end && my_runs) {
      const int k = nr + __popcll(eb & below);
      int64_t s = j;
      while (s - 1 >= wlo && window_keep(a.mode, i - (s - 1), Bh, a.G)) --s;
      if (s == wlo && joins) s = 0;
      if (k < a.max_runs) {
        my_runs[2 * k] = (int32_t)s;
        my_runs[2 * k + 1] = (int32_t)(j - s + 1);
      }
    }
    nr += __popcll(eb);
  }
  if (lane == 0) {
    a.count[q] = (int32_t)(n < INT32_MAX ? n : INT32_MAX);   // 2^31 keys: saturated
    if (a.n_runs) a.n_runs[q] = nr;
  }
}


// Tile list of the keep-sets: each list's first min(count, cap) entries
// cut into consecutive chunks of `tile` entries, in list order, as
// (list, first entry) pairs -- the split-KV work list.  One workgroup:
// lists are taken 1024 at a time, each thread counts its list's chunks,
// a workgroup-wide exclusive scan gives each list its first slot, and the
// running total carries over to the next 1024 lists.  Entries past
// cap_tiles are not written; n_tiles receives the true total.
__global__ void __launch_bounds__(1024) keepset_tiles_kernel(const int32_t* count, int n_q, int cap,
                                                             int tile, int32_t* tiles,
                                                             int64_t cap_tiles, int64_t* n_tiles) {
  __shared__ int64_t wsum[16];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  int64_t total = 0;
  for (int base = 0; base < n_q; base += 1024) {
    const int q = base + t;
    int c = q < n_q ? count[q] : 0;
    c = c < 0 ? 0 : (c < cap ? c : cap);
    const int64_t nt = (c + (int64_t)tile - 1) / tile;
    // inclusive scan within the wave, then across the 16 waves
    int64_t x = nt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int64_t y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int64_t before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      before += w < wave ? wsum[w] : 0;
      all += wsum[w];
    }
    const int64_t first = total + before + x - nt;
    for (int64_t k = 0; k < nt; ++k) {
      const int64_t e = first + k;
      if (e < cap_tiles) {
        tiles[2 * e] = q;
        tiles[2 * e + 1] = (int32_t)(k * tile);
      }
    }
    total += all;
    __syncthreads();                   // wsum is rewritten by the next round
  }
  if (t == 0) *n_tiles = total;
}

}  // namespace da

using namespace da;

extern "C" int da_keepset_build(const da_mask* m, int32_t n_q, const int32_t* pos,
                                const int32_t* prompt_len, int32_t n_keys, int32_t n_heads,
                                const int32_t* head_wb, int32_t cap,
                                int32_t* count, int32_t* idx, int32_t max_runs,
                                int32_t* n_runs, int32_t* runs, int32_t tile, int32_t* tiles,
                                int64_t cap_tiles, int64_t* n_tiles, void* stream) {
  int rc = check_mask(m);
  if (rc) return rc;
  if (n_q < 0) return fail(DA_EINVAL, "n_q=%d < 0", n_q);
  if (n_heads < 1) return fail(DA_EINVAL, "n_heads=%d < 1", n_heads);
  const int64_t n_lists = (int64_t)n_q * n_heads;
  if (n_lists > INT32_MAX) return fail(DA_EINVAL, "n_q * n_heads = %lld lists > INT32_MAX", (long long)n_lists);
  if ((uintptr_t)head_wb % 4) return fail(DA_EINVAL, "head_wb not 4-byte aligned");
  if (n_q > 0 && (!pos || !prompt_len || !count || !idx))
    return fail(DA_EINVAL, "pos, prompt_len, count and idx must be non-NULL");
  if (cap < 1) return fail(DA_EINVAL, "cap=%d < 1", cap);
  if (!m->causal && n_keys < 1) return fail(DA_EINVAL, "matrix form needs n_keys >= 1");
  if ((runs == nullptr) != (n_runs == nullptr))
    return fail(DA_EINVAL, "runs and n_runs must both be given or both be NULL");
  if (runs && max_runs < 1) return fail(DA_EINVAL, "max_runs=%d < 1", max_runs);
  if ((tiles == nullptr) != (n_tiles == nullptr))
    return fail(DA_EINVAL, "tiles and n_tiles must both be given or both be NULL");
  if (n_tiles && (tile < 1 || cap_tiles < 0))
    return fail(DA_EINVAL, "tile=%d must be >= 1 and cap_tiles=%lld >= 0", tile, (long long)cap_tiles);
  clear_error();
  if (n_q == 0 && n_tiles) {
    // an empty tile list still has its size written
    hipLaunchKernelGGL(keepset_tiles_kernel, dim3(1), dim3(1024), 0, (hipStream_t)stream, count, 0, cap,
                       tile, tiles, cap_tiles, n_tiles);
    return check_launch("keepset_tiles_kernel");
  }
  if (n_q == 0) return DA_OK;
  KeepsetArgs a;
  a.mode = m->mode;
  a.W = m->W;
  a.B = m->B;
  a.G = m->G;
  a.causal = m->causal;
  a.n_q = n_q;
  a.n_heads = n_heads;
  a.head_wb = head_wb;
  a.n_keys = n_keys;
  a.cap = cap;
  a.max_runs = runs ? max_runs : 0;
  a.pos = pos;
  a.prompt = prompt_len;
  a.count = count;
  a.idx = idx;
  a.n_runs = n_runs;
  a.runs = runs;
  const int64_t blocks = (n_lists + 3) / 4;
  hipLaunchKernelGGL(keepset_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, a.pos, a.prompt,
                     a.n_q, a);
  rc = check_launch("keepset_kernel");
  if (rc || !n_tiles) return rc;
  hipLaunchKernelGGL(keepset_tiles_kernel, dim3(1), dim3(1024), 0, (hipStream_t)stream, count, (int)n_lists,
                     cap, tile, tiles, cap_tiles, n_tiles);
  return check_launch("keepset_tiles_kernel");
}
