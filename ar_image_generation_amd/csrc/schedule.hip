// Batch order for the decode step (host side).
//
// The decode grid has one workgroup per (query, kv head) -- wg_per_query
// consecutive workgroups per query -- and the hardware deals workgroups to
// its compute units in turn, so the workgroups of batch slots p and
// p + R (R = n_cu / wg_per_query) land on the same compute units.  When
// every workgroup of a step is resident at once, the step ends when the
// compute unit with the most kept rows does, and the rows a query keeps
// differ with its prompt length and position.  A scheduler that knows each
// query's keep-set size (da_keep_count on host-side positions and prompt
// lengths) can lay the batch out so that every group of slots {j, j + R,
// j + 2R, ...} -- one compute unit's share -- sums to about the same:
// queries are taken largest first, R at a time (one round of slots), and
// each goes to the slot group with the least work so far.  Earlier rounds
// are dispatched first, so the largest queries also get the oldest, fastest
// workgroups of each compute unit.  The order changes only which slot a
// query sits in, never what is computed.
#include "common.h"

#include <algorithm>
#include <numeric>
#include <vector>

using namespace da;

extern "C" int da_decode_schedule(const int64_t* cost, int32_t n, int32_t wg_per_query, int32_t n_cu,
                                  int32_t* order) {
  if (n < 0) return fail(DA_EINVAL, "n=%d < 0", n);
  if (wg_per_query < 1) return fail(DA_EINVAL, "wg_per_query=%d < 1", wg_per_query);
  if (n > 0 && (!cost || !order)) return fail(DA_EINVAL, "cost and order must be non-NULL");
  if (n_cu == 0) {
    int dev = 0;
    hipDeviceProp_t prop;
    if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess)
      return fail(DA_EHIP, "no device to take the compute-unit count from");
    n_cu = prop.multiProcessorCount;
  }
  if (n_cu < 1) return fail(DA_EINVAL, "n_cu=%d < 1", n_cu);
  for (int32_t i = 0; i < n; ++i)
    if (cost[i] < 0) return fail(DA_EINVAL, "cost[%d] = %lld < 0", i, (long long)cost[i]);
  clear_error();
  if (n == 0) return DA_OK;
  const int64_t R = std::max<int64_t>(1, n_cu / wg_per_query);   // slots a round
  std::vector<int32_t> by_cost(n);
  std::iota(by_cost.begin(), by_cost.end(), 0);
  std::stable_sort(by_cost.begin(), by_cost.end(),
                   [&](int32_t a, int32_t b) { return cost[a] > cost[b]; });
  std::vector<int64_t> load(R, 0);
  std::vector<int64_t> groups(R);
  for (int64_t first = 0; first < n; first += R) {
    const int64_t m = std::min<int64_t>(R, n - first);   // the last round may be short
    // slot groups 0..m-1 of this round, least loaded first (ties: lower
    // group first), take this round's queries largest first
    std::iota(groups.begin(), groups.begin() + m, 0);
    std::stable_sort(groups.begin(), groups.begin() + m,
                     [&](int64_t a, int64_t b) { return load[a] < load[b]; });
    for (int64_t k = 0; k < m; ++k) {
      const int32_t q = by_cost[first + k];
      const int64_t grp = groups[k];
      order[first + grp] = q;
      load[grp] += cost[q];
    }
  }
  return DA_OK;
}
