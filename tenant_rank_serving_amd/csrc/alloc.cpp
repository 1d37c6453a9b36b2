// Bit allocation of the singular pairs (host): the 0/1 integer program of
// "Enhancing Delta Compression in LLMs via SVD-based Quantization Error
// Minimization" (§2.2: minimize the summed quantization error subject to a
// bit budget, one width per row, widths from a candidate set), solved
// exactly as a multiple-choice knapsack by dynamic programming over the
// budget used.
#include <cmath>
#include <cstdint>
#include <limits>
#include <vector>

#include "dc_internal.h"

extern "C" dc_status dc_allocate_bits(int32_t r, int32_t nb, const int32_t* cost, const double* err, int64_t budget,
                                      int32_t* choice, double* total) {
  if (r < 0 || nb <= 0 || nb > 127 || budget < 0 || !cost || (r > 0 && (!err || !choice)))
    return DC_ERR_INVALID_ARG;
  for (int k = 0; k < nb; ++k)
    if (cost[k] < 0) return DC_ERR_INVALID_ARG;
  for (size_t i = 0; i < (size_t)r * nb; ++i)
    if (!std::isfinite(err[i])) return DC_ERR_INVALID_ARG;
  if ((uint64_t)budget >= (uint64_t)INT32_MAX) return DC_ERR_UNSUPPORTED;
  const size_t cap = (size_t)budget + 1;   // states: budget used, 0..budget
  if ((size_t)r * cap > (size_t)INT32_MAX) return DC_ERR_UNSUPPORTED;   // one choice byte per (row, state)
  const double inf = std::numeric_limits<double>::infinity();
  // best[c]: least error of the rows so far using exactly c units
  std::vector<double> best(cap, inf), next(cap);
  std::vector<int8_t> arg((size_t)r * cap);
  best[0] = 0.0;
  for (int i = 0; i < r; ++i) {
    std::fill(next.begin(), next.end(), inf);
    int8_t* a = &arg[(size_t)i * cap];
    std::fill(a, a + cap, (int8_t)0);
    for (int k = 0; k < nb; ++k) {   // candidates in index order; a later one wins only if strictly better
      const size_t ck = (size_t)cost[k];
      if (ck >= cap) continue;
      const double e = err[(size_t)i * nb + k];
      for (size_t c = ck; c < cap; ++c) {
        const double v = best[c - ck] + e;
        if (v < next[c]) {
          next[c] = v;
          a[c] = (int8_t)k;
        }
      }
    }
    best.swap(next);
  }
  size_t c = 0;   // least error; the smallest budget used on ties
  for (size_t j = 1; j < cap; ++j)
    if (best[j] < best[c]) c = j;
  if (!(best[c] < inf)) return DC_ERR_RANGE;
  if (total) *total = best[c];
  for (int i = r - 1; i >= 0; --i) {
    const int k = arg[(size_t)i * cap + c];
    choice[i] = k;
    c -= (size_t)cost[k];
  }
  return DC_OK;
}
