// KV residency under the keep-set rule (host side).
//
// A decode query at position i keeps only prompt keys and keys inside its
// window (the summary's M: j >= i - W; the band half-width B bounds BAND
// further), and later queries only move the window forward.  So once a
// request has reached position i, a key j >= P with j < i - Wlive is never
// read again: its cache row can be recycled.  Pages of the prompt stay put;
// the window's pages form a ring of R slots, R = ceil((Wlive + 1) / page) + 1,
// enough that the pages of any live window never share a slot.
//
// The mapping is static -- logical page lp of a request sits in a fixed
// physical page -- so it is an ordinary block table: the decode kernels read
// through it unchanged, and a writer that stores each new token's K/V row at
// (block_table[lp], slot) overwrites exactly the rows that have died.
#include "common.h"

namespace da {

// Positions before i - live_window(m) are dead for queries at i or later
// (prompt excepted).  DENSE keeps everything: no ring.
static int64_t live_window(const da_mask* m) {
  if (m->mode == DA_MODE_BAND) return m->B < m->W ? m->B : m->W;
  return m->W;
}

static int64_t ring_slots(const da_mask* m, int32_t page_size) {
  return (live_window(m) + 1 + page_size - 1) / page_size + 1;
}

}  // namespace da

using namespace da;

extern "C" int64_t da_ring_pages(const da_mask* m, int32_t prompt_len, int32_t max_len,
                                 int32_t page_size) {
  int rc = check_mask(m);
  if (rc) return rc;
  if (!m->causal) return fail(DA_ENOTSUP, "residency is defined for causal decode");
  if (prompt_len < 0 || max_len < 1 || page_size < 1)
    return fail(DA_EINVAL, "prompt_len=%d max_len=%d page_size=%d", prompt_len, max_len, page_size);
  clear_error();
  const int64_t all = ((int64_t)max_len + page_size - 1) / page_size;
  if (m->mode == DA_MODE_DENSE) return all;
  const int64_t fixed = ((int64_t)(prompt_len < max_len ? prompt_len : max_len) + page_size - 1) / page_size;
  const int64_t ring = ring_slots(m, page_size);
  return fixed + ring < all ? fixed + ring : all;
}

extern "C" int da_ring_block_table(const da_mask* m, int32_t n_seq, const int32_t* prompt_len,
                                   int32_t max_len, int32_t page_size, int32_t first_page,
                                   int32_t bt_stride, int32_t* block_table, int64_t* n_pages) {
  int rc = check_mask(m);
  if (rc) return rc;
  if (!m->causal) return fail(DA_ENOTSUP, "residency is defined for causal decode");
  if (n_seq < 0 || max_len < 1 || page_size < 1 || first_page < 0)
    return fail(DA_EINVAL, "n_seq=%d max_len=%d page_size=%d first_page=%d", n_seq, max_len,
                page_size, first_page);
  const int64_t lpages = ((int64_t)max_len + page_size - 1) / page_size;
  if (bt_stride < lpages) return fail(DA_EINVAL, "bt_stride=%d < %lld logical pages", bt_stride, (long long)lpages);
  if (n_seq > 0 && (!prompt_len || !block_table))
    return fail(DA_EINVAL, "prompt_len and block_table must be non-NULL");
  for (int32_t s = 0; s < n_seq; ++s)
    if (prompt_len[s] < 0) return fail(DA_EINVAL, "prompt_len[%d]=%d < 0", s, prompt_len[s]);
  int64_t next = first_page;
  for (int32_t s = 0; s < n_seq; ++s) {
    const int64_t need = da_ring_pages(m, prompt_len[s], max_len, page_size);
    if (need < 0) return (int)need;
    const int32_t P = prompt_len[s] < max_len ? prompt_len[s] : max_len;
    const int64_t fixed = (P + (int64_t)page_size - 1) / page_size;
    const int64_t ring = need - fixed;       // ring slots (== lpages - fixed when no saving)
    if (next + need > INT32_MAX) return fail(DA_EINVAL, "page ids overflow int32");
    int32_t* row = block_table + (int64_t)s * bt_stride;
    for (int64_t lp = 0; lp < bt_stride; ++lp) {
      int64_t pg;
      if (lp < fixed) pg = lp;
      else if (lp < lpages) pg = fixed + (lp - fixed) % ring;
      else pg = 0;                          // past max_len: never addressed
      row[lp] = (int32_t)(next + pg);
    }
    next += need;
  }
  if (n_pages) *n_pages = next - first_page;
  clear_error();
  return DA_OK;
}
