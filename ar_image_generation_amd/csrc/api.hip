// Host-side pieces of the C ABI: version, error text, keep-set sizing.
#include <stdarg.h>
#include <stdio.h>

#include "common.h"

namespace da {

static thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() { g_err[0] = '\0'; }

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(DA_EHIP, "%s: %s", what, hipGetErrorString(e));
  return DA_OK;
}

// Number of distances d in [0, D] within B of a multiple of G.
static int64_t rowdiag_window_count(int64_t D, int64_t B, int64_t G) {
  if (D < 0) return 0;
  if (2 * B + 1 >= G) return D + 1;
  const int64_t n = D + 1, full = n / G, rem = n % G;
  int64_t c = full * (2 * B + 1);
  c += rem < B + 1 ? rem : B + 1;
  if (rem > G - B) c += rem - (G - B);
  return c;
}

int check_mask(const da_mask* m) {
  if (!m) return fail(DA_EINVAL, "mask is NULL");
  if (m->mode < DA_MODE_DENSE || m->mode > DA_MODE_ROWDIAG)
    return fail(DA_EINVAL, "mask mode %d out of range", m->mode);
  if (m->W < 0 || m->B < 0) return fail(DA_EINVAL, "mask W=%d B=%d must be >= 0", m->W, m->B);
  if (m->G < 1) return fail(DA_EINVAL, "mask G=%d must be >= 1", m->G);
  if (m->causal != 0 && m->causal != 1) return fail(DA_EINVAL, "mask causal=%d not 0/1", m->causal);
  return DA_OK;
}

}  // namespace da

using namespace da;

extern "C" int32_t da_version(void) { return 300; }

extern "C" const char* da_last_error(void) { return g_err; }

extern "C" int64_t da_keep_count(const da_mask* m, int32_t pos, int32_t prompt_len,
                                 int32_t n_keys) {
  int rc = check_mask(m);
  if (rc) return rc;
  if (pos < 0 || prompt_len < 0) return fail(DA_EINVAL, "pos/prompt_len must be >= 0");
  if (!m->causal && (n_keys < 1 || pos >= n_keys))
    return fail(DA_EINVAL, "matrix form needs 0 <= pos < n_keys");
  clear_error();
  const int64_t i = pos, P = prompt_len;
  const int64_t L = m->causal ? i + 1 : n_keys;
  if (m->mode == DA_MODE_DENSE) return L;
  const int64_t Pc = P < L ? P : L;
  int64_t c = Pc;
  // past part of the window: j in [max(Pc, i - W), i]
  const int64_t lo = Pc > i - m->W ? Pc : i - m->W;
  if (lo <= i) {
    const int64_t D = i - lo;  // largest distance inside the window
    if (m->mode == DA_MODE_BAND) c += (D < m->B ? D : m->B) + 1;
    else c += rowdiag_window_count(D, m->B, m->G);
  }
  // future part (matrix form): j in [max(Pc, i + 1), min(L - 1, i + B)]
  if (!m->causal) {
    const int64_t flo = Pc > i + 1 ? Pc : i + 1;
    const int64_t fhi = L - 1 < i + m->B ? L - 1 : i + m->B;
    if (fhi >= flo) c += fhi - flo + 1;
  }
  return c;
}

extern "C" int64_t da_keep_cap(const da_mask* m, int32_t max_pos, int32_t max_prompt,
                               int32_t n_keys) {
  int rc = check_mask(m);
  if (rc) return rc;
  if (max_pos < 0 || max_prompt < 0) return fail(DA_EINVAL, "max_pos/max_prompt must be >= 0");
  if (!m->causal && n_keys < 1) return fail(DA_EINVAL, "matrix form needs n_keys >= 1");
  clear_error();
  const int64_t L = m->causal ? int64_t(max_pos) + 1 : n_keys;
  if (m->mode == DA_MODE_DENSE) return L;
  const int64_t bound = int64_t(max_prompt) + m->W + 1 + (m->causal ? 0 : m->B);
  return bound < L ? bound : L;
}
