/*
 * diagattn.h -- C ABI of libdiagattn.so: diagonal-aware sparse attention for
 * autoregressive image generation on MI355X (gfx950).
 *
 * The operation.  "Understanding and Exploiting Diagonal Attention Sparsity in
 * Autoregressive Image Generation" (arXiv 2609.19702) computes, per query,
 * softmax(Q K^T / sqrt(d) (.) M) V where M keeps key j for query i when
 * |i - j| <= B and j >= i - W (paper-daily summary page, section
 * "核心公式与算法", core formulas).  Masked keys are skipped: they are never
 * read and get no weight (same summary, section "具体技术细节示例", the
 * worked example, which normalises over the kept keys and counts only their
 * KV reads).  The arXiv abstract names the two other facts used here:
 * attention concentrates on the prompt tokens, and the diagonal pattern comes
 * from the spatial locality of visual tokens in raster order.  Hence the
 * keep-set of a decode query at position i with a prompt of P tokens is
 *
 *   DENSE   : every j <= i                                  (the baseline)
 *   BAND    : j < P, or |i - j| <= B and j >= i - W          (the printed M)
 *   ROWDIAG : j < P, or j >= i - W and |(i - j) - k*G| <= B for some k >= 0
 *             (the main band plus one band per raster row above, G = grid
 *             width; distances are plain sequence distances)
 *
 * with j <= i (causal) in decode.  Masked logits are -inf; the scale is
 * 1/sqrt(head_dim) unless the caller passes another; query head h reads kv
 * head h / (hq / hkv).
 *
 * Conventions.
 *   - Every pointer is a DEVICE pointer owned by the caller unless marked
 *     [host].  The library allocates no memory and keeps no state besides a
 *     thread-local error string and, on each GPU, the fixed scratch array
 *     of da_sparse_decode_attn_masked_noalloc (part of the loaded code
 *     object).
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream).  No call synchronises the device or copies host<->device.
 *   - Host-checkable argument errors return a negative da_status before any
 *     launch; da_last_error() then describes the problem.  A failed kernel
 *     launch returns DA_EHIP with the HIP error text.  Values that live in
 *     device memory (positions, counts, indices, block tables) cannot be
 *     checked on the host: their preconditions are stated per call.
 *   - Floating point: inputs and outputs share one dtype (fp32 or bf16);
 *     accumulation and softmax state are fp32; bf16 outputs are rounded to
 *     nearest even.
 */
#ifndef DIAGATTN_H
#define DIAGATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DA_OK = 0,
  DA_EINVAL = -1,     /* bad argument (null pointer, negative size, ...) */
  DA_ENOTSUP = -2,    /* valid but unsupported (head_dim, dtype, group) */
  DA_ECAPACITY = -3,  /* a caller-provided buffer is too small */
  DA_EHIP = -4        /* a HIP runtime call or kernel launch failed */
} da_status;

typedef enum { DA_MODE_DENSE = 0, DA_MODE_BAND = 1, DA_MODE_ROWDIAG = 2 } da_mode;

typedef enum { DA_F32 = 0, DA_BF16 = 1 } da_dtype;

/* Mask parameters.  W and B are in tokens (a window of r raster rows is
 * W = r * G).  causal = 1: a query at position i sees keys 0..i (decode and
 * prefill); causal = 0: it sees keys 0..n_keys-1 (the N x N matrix form of
 * the summary's mask, where future keys within B are kept too). */
typedef struct {
  int32_t mode;    /* da_mode */
  int32_t W;       /* recent window, >= 0 */
  int32_t B;       /* diagonal half-width, >= 0 */
  int32_t G;       /* raster grid width, >= 1 (used by ROWDIAG) */
  int32_t causal;  /* 0 or 1 */
} da_mask;

/* Library version, major * 10000 + minor * 100 + patch. */
int32_t da_version(void);

/* Text of the last non-OK status returned on the calling thread ("" if none). */
const char* da_last_error(void);

/* [host] Exact keep-set size of one query at `pos` with `prompt_len` prompt
 * tokens (n_keys is read only when m->causal == 0).  Returns a negative
 * da_status for invalid arguments. */
int64_t da_keep_count(const da_mask* m, int32_t pos, int32_t prompt_len, int32_t n_keys);

/* [host] Upper bound on the keep-set size of any query with pos <= max_pos
 * and prompt_len <= max_prompt (n_keys as above); use it to size `cap`. */
int64_t da_keep_cap(const da_mask* m, int32_t max_pos, int32_t max_prompt, int32_t n_keys);

/* keepset_build -- KV index lists per query (or per query and head), their
 * maximal runs and the split-KV tile list.
 *
 * For each query q < n_q at position pos[q] with prompt_len[q] tokens of
 * prompt and each head h < n_heads, list l = q*n_heads + h is the keep-set
 * (rule above) of that query under head h's window and band -- head_wb[2h]
 * and head_wb[2h+1] (device, int32; negative values read as 0), or m->W
 * and m->B for every head when head_wb is NULL -- written as ascending
 * positions:
 *   count[l]              number of kept keys (the true size, even if > cap;
 *                         saturated at INT32_MAX)
 *   idx[l*cap + r]        r-th kept position, for r < min(count[l], cap)
 *   n_runs[l]             number of maximal runs of consecutive positions
 *   runs[(l*max_runs + k)*2 + {0,1}] = (first position, length) of run k,
 *                         for k < min(n_runs[l], max_runs)
 *   tiles[e*2 + {0,1}]    = (list, first entry) of tile e: each list's
 *                         first min(count[l], cap) entries cut into
 *                         consecutive chunks of `tile` entries, lists in
 *                         order (the work list of a split-KV decode with
 *                         split = tile), for e < min(*n_tiles, cap_tiles)
 *   *n_tiles              total number of tiles (int64, the true total)
 * runs/n_runs may both be NULL (then max_runs is ignored), and so may
 * tiles/n_tiles (then tile and cap_tiles are ignored).  Entries of idx,
 * runs and tiles past count / n_runs / n_tiles are left untouched.  The
 * summary page's custom kernels work on tiles of the kept entries (section
 * "技术方法详解", item 4); the tile list is that decomposition.  Per-head
 * windows and bands follow the summary page's future-directions section
 * ("未来研究方向": adapting B and W) and the per-head budgets of the HeadKV
 * abstract (thelatestinai.com page); n_heads = 1 with head_wb = NULL is the
 * one list per query that da_sparse_decode_attn reads.
 *
 * Preconditions on device data: 0 <= pos[q]; 0 <= prompt_len[q]; for
 * causal = 0 also pos[q] < n_keys.  Queries that break them get count 0.
 * Overflow is reported, never written: if count[q] > cap (or n_runs[q] >
 * max_runs, or *n_tiles > cap_tiles) the caller's list is truncated and
 * must be treated as an error (da_keep_cap gives a safe cap).
 * Errors: DA_EINVAL for null required pointers, n_q < 0, n_heads < 1,
 * n_q * n_heads > INT32_MAX, cap < 1, W/B < 0, G < 1, mode or causal out of
 * range, causal = 0 with n_keys < 1, runs/n_runs given with max_runs < 1 or
 * only one of them given, tiles/n_tiles given with tile < 1 or
 * cap_tiles < 0 or only one given, head_wb misaligned. */
int da_keepset_build(const da_mask* m /* [host] */, int32_t n_q,
                     const int32_t* pos, const int32_t* prompt_len, int32_t n_keys,
                     int32_t n_heads, const int32_t* head_wb,
                     int32_t cap, int32_t* count, int32_t* idx,
                     int32_t max_runs, int32_t* n_runs, int32_t* runs,
                     int32_t tile, int32_t* tiles, int64_t cap_tiles, int64_t* n_tiles,
                     void* stream);

/* KV cache descriptor: one form for contiguous and paged caches.
 * Element (kv head g, logical position j) of request s starts at
 *   base + page * page_stride + g * head_stride + slot * slot_stride
 * with page = block_table[s * bt_stride + j / page_size] and
 * slot = j % page_size; when block_table is NULL, page = s and slot = j
 * (a contiguous [n_seq][hkv][Lmax][head_dim] cache has
 * page_stride = hkv*Lmax*hd, head_stride = Lmax*hd, slot_stride = hd).
 * Strides are in elements; head_dim elements of one row are contiguous and
 * 16-byte aligned.  page_size must be a power of two when block_table is set.
 * Extents: n_seq requests (rows of the block table; with no table, requests
 * in the cache), n_pages pages in k/v (with no table: = n_seq), max_len
 * logical positions per request (<= bt_stride * page_size with a table).
 * The kernels clamp every request, position and page index they read from
 * device memory into these extents, so inconsistent device-side lists give
 * wrong numbers, never an out-of-bounds access. */
typedef struct {
  const void* k;
  const void* v;
  int64_t page_stride;
  int64_t head_stride;
  int64_t slot_stride;
  int32_t page_size;
  int32_t bt_stride;
  const int32_t* block_table;   /* [n_seq][bt_stride] or NULL */
  int32_t n_seq;
  int32_t n_pages;
  int32_t max_len;
} da_kv_cache;

/* [host] Workspace bytes da_sparse_decode_attn and da_sparse_decode_attn_masked
 * need for these sizes (0 when every keep-set fits one chunk, i.e. cap <=
 * split): the per-chunk partial results (max, sum, unnormalised output) that
 * the merge kernel combines, and (mask form) the keep-set size of each
 * (query, kv head). */
int64_t da_decode_workspace_bytes(int32_t n_q, int32_t hq, int32_t head_dim,
                                  int32_t cap, int32_t split);

/* sparse_decode_attn -- one decode step of masked attention over kept keys.
 *
 * out[q][h][:] = sum_r w_r V[g, idx[q*cap + r]] with
 * w = softmax_r(scale * q[q][h] . K[g, idx[q*cap + r]]), r < count[q],
 * g = h / (hq/hkv), K/V rows of request seq[q] read through `kv`.
 * This is the summary's masked softmax with the exclusion reading: only the
 * count[q] listed keys are loaded and weighted (worked example).  A DENSE
 * keep-set (every j <= pos) makes this the dense baseline at the same shape.
 *
 * Work split: each query's list is cut into chunks of `split` keys; each
 * (query, kv head, chunk) is one workgroup that serves all hq/hkv query heads
 * of the kv head, so each kept K/V row is read from HBM once.  When a list
 * spans several chunks (cap > split), a second kernel combines the chunk
 * partials by a log-sum-exp merge.
 *
 *   q     [n_q][hq][head_dim] in `dtype`
 *   out   [n_q][hq][head_dim] in `dtype`
 *   lse   [n_q][hq] fp32 natural-log sum of exp of the scaled logits, or NULL
 *   seq   [n_q] request (block-table row) of each query
 *   count [n_q], idx [n_q][cap] as written by da_keepset_build; or, with
 *         list_heads = hkv, one list per kv head: count [n_q][hkv],
 *         idx [n_q][hkv][cap] (da_keepset_build with n_heads = hkv and a
 *         (W, B) per kv head), kv head g of query q attending list q*hkv + g
 *         -- per-kv-head budgets; list_heads must be 1 or hkv
 *   workspace: da_decode_workspace_bytes(...) bytes, 256-byte aligned, or
 *         NULL when that is 0; no initialisation needed.  Calls that share a
 *         workspace must not overlap in time (one workspace per stream).
 * Device data: counts above cap are read as cap; a query with count 0 gets
 * no output written.  Listed positions, seq[] and block-table entries are
 * clamped into the descriptor's extents (see da_kv_cache).
 * Errors: DA_EINVAL (null pointers, n_q < 0, hq or hkv < 1, hq % hkv != 0,
 * cap < 1, split < 1, non-power-of-two page_size with a block table,
 * bt_stride < 1, extents < 1, max_len > bt_stride * page_size, list_heads
 * not 1 or hkv), DA_ENOTSUP (head_dim not 64/128, dtype, hq/hkv not in
 * {1,2,4,8}, split > 4096), DA_ECAPACITY (workspace too small). */
int da_sparse_decode_attn(const void* q, da_dtype dtype, int32_t n_q,
                          int32_t hq, int32_t hkv, int32_t head_dim, float scale,
                          const da_kv_cache* kv /* [host] */, const int32_t* seq,
                          const int32_t* count, const int32_t* idx, int32_t cap,
                          int32_t list_heads, int32_t split, void* out, float* lse,
                          void* workspace, int64_t ws_bytes, void* stream);

/* sparse_decode_attn_masked -- the same decode step with the keep-set taken
 * from the mask instead of lists: keep-set build and attention in one launch.
 *
 * For query q the kept keys are the keep-set of position pos[q] with
 * prompt_len[q] prompt tokens under `m` (causal form), in the order and with
 * the truncation of da_keepset_build: entries r < min(count, cap).  The
 * output is then exactly that of da_sparse_decode_attn on the lists
 * da_keepset_build would write (the same rows in the same order through the
 * same kernel).  Rule and example as for da_keepset_build (the summary's M,
 * prompt columns, row-offset diagonals; worked example).
 *
 *   m      [host] mask; m->causal must be 1
 *   pos, prompt_len [n_q] int32 position and prompt length of each query
 *   count, idx  optional outputs (both or neither): the lists exactly as
 *          da_keepset_build writes them (count[q] the true size; idx[q*cap+r]
 *          for r < min(count[q], cap)), for callers that reuse them
 *   head_wb optional [hq][2] int32: a window and band (W, B) per query
 *          head, replacing m->W, m->B for that head (per-head budgets and
 *          windows adapted to the content, as the summary page's future
 *          directions and the HeadKV abstract propose; negative values read
 *          as 0).  The query heads of one kv head read the keep-set of the
 *          group's widest (max W, max B) once -- it contains every head's,
 *          both rules growing with W and B -- and each head masks the rows
 *          outside its own keep-set, so a kept row is still read once per kv
 *          head; `cap` must bound that widest keep-set.  Groups of 2, 4 or 8
 *          query heads need bf16 (DA_ENOTSUP otherwise); with hq == hkv any
 *          dtype.  Not allowed with count/idx (those lists are per query).
 *   k_new, v_new optional inputs (both or neither) [n_q][hkv][head_dim] in
 *          `dtype`, 16-byte aligned: KV append.  The row of each query's own
 *          position pos[q] is written into the cache (kv->k, kv->v, which must
 *          then be writable), and the step attends to these new key and value
 *          rows at that position (not to what the cache held).  Precondition: no query of the call reads a
 *          row another query of the call appends (e.g. one query per request);
 *          positions outside [0, kv->max_len) are not written.
 *   other arguments as for da_sparse_decode_attn (cap bounds the entries a
 *          query attends to and sizes the chunk grid with `split`).
 * Device data: pos[q] < 0 or prompt_len[q] < 0 gives count 0 and no output
 * written for that query; positions and requests are clamped into the
 * descriptor's extents.
 * Errors: as da_sparse_decode_attn, plus DA_EINVAL for an invalid mask, null
 * pos/prompt_len, only one of count/idx or of k_new/v_new given, head_wb
 * together with count/idx, or misaligned k_new/v_new; DA_ENOTSUP for
 * causal = 0 or head_wb with fp32 groups of query heads. */
int da_sparse_decode_attn_masked(const da_mask* m /* [host] */, const void* q,
                                 da_dtype dtype, int32_t n_q, int32_t hq, int32_t hkv,
                                 int32_t head_dim, float scale,
                                 const da_kv_cache* kv /* [host] */, const int32_t* seq,
                                 const int32_t* pos, const int32_t* prompt_len,
                                 const int32_t* head_wb,
                                 const void* k_new, const void* v_new,
                                 int32_t cap, int32_t split, int32_t* count, int32_t* idx,
                                 void* out, float* lse, void* workspace, int64_t ws_bytes,
                                 void* stream);

/* [host] Size in bytes of the scratch memory behind
 * da_sparse_decode_attn_masked_noalloc (a fixed maximum, 32 MiB). */
int64_t da_decode_scratch_bytes(void);

/* sparse_decode_attn_masked_noalloc -- da_sparse_decode_attn_masked without
 * a caller workspace and without any allocation, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).
 *
 * Arguments, outputs and results are those of da_sparse_decode_attn_masked
 * (the same kernels run).  The workspace it needs when a keep-set spans
 * several chunks (cap > split) comes from a device array inside the library,
 * da_decode_scratch_bytes() long, one per GPU, held until the process ends;
 * its device address is looked up (not allocated) on the first call on each
 * device.  No hipMalloc, hipFree or allocating library routine is called.
 * The array keeps the last call's contents; nothing in it needs clearing
 * between calls.  Every call on one GPU shares that GPU's array, so calls
 * that overlap in time on one GPU (concurrent streams, or host threads
 * sharing a device) race: order them on one stream.
 * Errors: as da_sparse_decode_attn_masked, plus DA_ECAPACITY when the
 * sizes need more than da_decode_scratch_bytes() of workspace
 * (da_decode_workspace_bytes(n_q, hq, head_dim, cap, split) > that), and
 * DA_EHIP if the device address of the array cannot be obtained. */
int da_sparse_decode_attn_masked_noalloc(const da_mask* m /* [host] */, const void* q,
                                         da_dtype dtype, int32_t n_q, int32_t hq, int32_t hkv,
                                         int32_t head_dim, float scale,
                                         const da_kv_cache* kv /* [host] */, const int32_t* seq,
                                         const int32_t* pos, const int32_t* prompt_len,
                                         const int32_t* head_wb,
                                         const void* k_new, const void* v_new,
                                         int32_t cap, int32_t split, int32_t* count, int32_t* idx,
                                         void* out, float* lse, void* stream);

/* KV residency.  Under the keep-set rule a decode query at position i reads
 * prompt keys and keys j >= i - W (the summary's M, core formulas; BAND also
 * needs |i - j| <= B, so only j >= i - min(B, W)), and later queries only
 * move that window forward.  Rows older than the window are therefore dead
 * once a request has passed them, and a request needs its prompt pages plus
 * a ring of R = ceil((Wlive + 1) / page_size) + 1 window pages (Wlive = W,
 * or min(B, W) for BAND) instead of one page per position.  DENSE keeps
 * every page.
 *
 * [host] da_ring_pages: pages one request needs, for prompt_len prompt
 * tokens and up to max_len positions: ceil(prompt_len / page_size) + R,
 * capped at ceil(max_len / page_size).  Negative da_status on bad arguments
 * (DA_ENOTSUP for causal = 0). */
int64_t da_ring_pages(const da_mask* m /* [host] */, int32_t prompt_len, int32_t max_len,
                      int32_t page_size);

/* [host] ring_block_table -- a static block table that recycles dead rows.
 *
 * Request s gets the next da_ring_pages(...) physical pages from first_page
 * on (requests in order); its logical page lp maps to its own page lp while
 * lp < ceil(prompt_len[s] / page_size), and past that to ring slot
 * (lp - that count) mod R.  Writing each new token's K/V row at
 * (block_table[s][j / page_size], j % page_size) then overwrites only rows
 * no later query of s reads, and the decode entry points, given this table,
 * return exactly what they return on a full cache.  Entries past
 * ceil(max_len / page_size) are set to the request's first page.
 *   prompt_len  [host] [n_seq]
 *   block_table [host] [n_seq][bt_stride] out, bt_stride >= ceil(max_len / page_size)
 *   n_pages     [host] out (may be NULL): pages used by all requests
 * Errors: DA_EINVAL (mask, sizes, null pointers, negative prompt_len, page
 * ids past INT32_MAX), DA_ENOTSUP (causal = 0). */
int da_ring_block_table(const da_mask* m /* [host] */, int32_t n_seq, const int32_t* prompt_len,
                        int32_t max_len, int32_t page_size, int32_t first_page,
                        int32_t bt_stride, int32_t* block_table, int64_t* n_pages);

/* [host] Bytes of the prefill tile lists for `batch` sequences of n tokens. */
int64_t da_prefill_tiles_bytes(int32_t batch, int32_t n);

/* prefill_tiles_build -- the tile lists of the keep-set for prefill.
 *
 * Queries are cut into tiles of 128 rows (4 waves x 2 blocks of 16) and keys
 * into tiles of 64 (4 blocks of 16) on two grids: prompt tiles at multiples
 * of 64 for keys below prompt_len[b] (DENSE: every key), and window tiles
 * for keys at or past it, starting on keys congruent to (first row - B)
 * mod 16, so that the kept keys of a 16-row block on one diagonal of the
 * row-diagonal rule (summary page, core formulas) start on a 16-key block.
 * For each batch b and query tile qt this writes the key tiles that hold at
 * least one kept (row, key) pair of the causal keep rule -- prompt tiles
 * counting keys below the prompt end only, window tiles keys at or past it
 * -- and for each two 64-bit masks over (wave w, row block rb, key block kq),
 * bit w*8 + rb*4 + kq: the block holds a kept pair / every pair of the block
 * is kept (bits 32..63, waves 4..7, are zero with 4 waves a tile); row block
 * rb of wave w is rows 128 qt + 16 w + 64 rb .. + 15.  Tiles in which some
 * wave needs three or four of the key blocks come first ("whole" tiles),
 * then the tiles in which every wave's two row blocks together need at most
 * two ("half" tiles: only those two are computed, shared by both row
 * blocks).  Layout of `tiles` (16-byte aligned, da_prefill_tiles_bytes
 * long):
 *   int32 count[batch][n_qt] = list length | number of whole tiles << 16,
 *         padded to 16 bytes, then
 *   int32 entry[batch][n_qt][max_tiles][8] = {first key, need lo, need hi,
 *         window tile (0/1), full lo, full hi, 0, 0}
 * with n_qt = ceil(n / 128), max_tiles = ceil(n / 64) + 3; a window tile's
 * first key may be up to 15 below 0.  The lists depend only on the mask, n
 * and prompt_len: build them once and reuse them for every head and layer.
 * Errors: DA_EINVAL (mask, sizes, null pointers, alignment), DA_ENOTSUP
 * (causal = 0), DA_ECAPACITY (tiles_bytes too small). */
int da_prefill_tiles_build(const da_mask* m /* [host] */, int32_t batch, int32_t n,
                           const int32_t* prompt_len, void* tiles, int64_t tiles_bytes,
                           void* stream);

/* band_prefill_attn -- keep-set-masked causal attention over whole sequences
 * (prefill), on the matrix cores.
 *
 * For every batch b, query head h and row i < n:
 *   out[b][h][i][:] = sum_j w_ij v[b][hk][j][:],
 *   w_i = softmax over kept keys j <= i of scale * q[b][h][i] . k[b][hk][j],
 * with the keep rule above for a query at position i and prompt_len[b]
 * prompt tokens, hk = h / (heads / kv_heads).  This is the summary's masked
 * softmax (core formulas) applied to every row of the sequence; the pages
 * apply the sparsity to decode, and this call serves the same mask where a
 * whole sequence is attended at once.  Only the key tiles listed in `tiles`
 * (da_prefill_tiles_build with the same mask, n and prompt_len) are
 * computed; element masks (a 64-bit keep word per row and key tile) are
 * applied where a wave's blocks are not all entirely kept.
 *
 *   q, out [batch][heads][n][head_dim], k, v [batch][kv_heads][n][head_dim],
 *          bf16, head_dim elements contiguous and 16-byte aligned;
 *   strides[12] [host]: element strides (batch, head, position) of q, k, v,
 *          out, in that order, each a multiple of 8;
 *   prompt_len [batch] (device; read clamped to [0, n]);
 *   tiles, tiles_bytes: the lists of da_prefill_tiles_build for this mask, n
 *          and prompt_len, and the size of that buffer (at least
 *          da_prefill_tiles_bytes(batch, n));
 *   lse [batch][heads][n] fp32 natural-log sums, or NULL.
 * W and B of n or more are read as n (no row/key distance reaches n).
 * Scores accumulate in fp32 from bf16 products; probabilities are rounded to
 * bf16 for the second product; outputs round to nearest even.  Tile entries
 * and counts are clamped into range, so an inconsistent list gives wrong
 * numbers, never an out-of-bounds access.
 * Limits (LDS copies of the tile list and of the row-diagonal band pattern):
 * n <= 65536 tokens; in ROWDIAG mode G <= 1016; the k and v position strides
 * such that 63 positions plus one row span under 4 GiB (32-bit offsets
 * within a 64-key tile).
 * Errors: DA_EINVAL (mask, null pointers, sizes, strides, alignment, a
 * scale that is not positive and finite),
 * DA_ENOTSUP (causal = 0, dtype other than bf16, head_dim not 64/128,
 * n > 65536, ROWDIAG with G > 1016, k/v position stride too large),
 * DA_ECAPACITY (tiles_bytes below da_prefill_tiles_bytes(batch, n)). */
int da_band_prefill_attn(const da_mask* m /* [host] */, da_dtype dtype, int32_t batch,
                         int32_t heads, int32_t kv_heads, int32_t n, int32_t head_dim,
                         const void* q, const void* k, const void* v, void* out,
                         const int64_t* strides /* [host] 12 */, const int32_t* prompt_len,
                         const void* tiles, int64_t tiles_bytes, float scale, float* lse,
                         void* stream);

/* [host] decode_schedule -- a batch order that balances the decode step's
 * kept rows over the compute units.
 *
 * cost[q] (host, >= 0) is query q's work, e.g. da_keep_count of its position
 * and prompt length; wg_per_query is the number of workgroups the decode
 * launches per query (hkv for one chunk a list); n_cu the compute units (0:
 * those of the current device).  Writes order[p] (host), a permutation of
 * 0..n-1: the query to place in batch slot p.  Workgroups are dealt to the
 * compute units in turn, so the slots p, p + R, p + 2R, ... (R = n_cu /
 * wg_per_query, at least 1) share compute units; queries are taken largest
 * first, R a round, each into the round's slot group with the least cost so
 * far.  The decode step of a batch laid out in this order computes the same
 * outputs for every query (only their slots move) and ends sooner when
 * costs differ: the last compute unit to finish has less work.  This is a
 * scheduling aid for the serving layer around the step, which knows each
 * request's prompt length and position (the summary page's serving system,
 * "技术方法详解" item 4, schedules requests around its sparse kernels).
 * Errors: DA_EINVAL (n < 0, wg_per_query < 1, n_cu < 0, a negative cost,
 * null pointers), DA_EHIP (n_cu = 0 and no device). */
int da_decode_schedule(const int64_t* cost /* [host] */, int32_t n, int32_t wg_per_query, int32_t n_cu,
                       int32_t* order /* [host] */);

/* Measurement: streaming read of `bytes` bytes at `buf` (16-byte aligned, a
 * multiple of 16) by `grid` workgroups of 256 threads, 16-byte nontemporal
 * loads, `loads_in_flight` (1, 2, 4, 8 or 16) independent loads per thread
 * per iteration; writes one word per workgroup to sink[grid].  Its bytes /
 * duration, best over grids and depths, is the attainable HBM read
 * bandwidth that decode's kept-byte bandwidth is compared with.  Errors:
 * DA_EINVAL for NULL pointers, a bad size or alignment, grid < 1, or
 * another loads_in_flight. */
int da_hbm_read_probe(const void* buf, int64_t bytes, uint32_t* sink, int32_t grid,
                      int32_t loads_in_flight, void* stream);

/* Measurement: a gather of rows of two buffers, K and V, at n_rows byte
 * offsets (offsets[n_rows] int64, device) -- given the byte offsets of the
 * kept K/V rows of a decode step, resolved through its lists and block table
 * beforehand, it reads exactly what the step must read and nothing else: the
 * attainable rate of decode's own access pattern (the summary page finds
 * decode bound by KV-cache reads), without its arithmetic or its address
 * chain.  Rows of row_bytes (128, 256 or 512) bytes; offsets are clamped
 * into [0, span_bytes - row_bytes] and rounded down to 16, so no offset
 * reads outside the buffers (span_bytes: the bytes of K, and of V, from the
 * base pointers).  `grid` workgroups of 256 threads, `loads_in_flight` (1, 2
 * or 4) rows of K and of V in flight per lane group; one XOR of the words
 * read per workgroup to sink[grid] (the XOR over sink is the XOR of every
 * word of the rows read).  Errors: DA_EINVAL (NULL pointers, sizes,
 * alignment, grid, loads_in_flight), DA_ENOTSUP (row size). */
int da_gather_read_probe(const void* k, const void* v, const int64_t* offsets, int64_t n_rows,
                         int32_t row_bytes, int64_t span_bytes, uint32_t* sink, int32_t grid,
                         int32_t loads_in_flight, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DIAGATTN_H */
