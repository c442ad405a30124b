// Pairing of two strands' operator segments (host only, no HIP calls): the forward segments of one
// micro-batch and the backward segments of another, run in order within each strand, each step
// running one forward segment alone, one backward segment alone, or one of each side by side. The
// makespan of a pairing is the sum of its steps' measured times, and the best pairing follows the
// dynamic program over segment prefixes that the micro-batch co-execution review gives under "What
// carries the argument":
//   T(i, j) = min{ T(i-1, j) + P(i, none), T(i, j-1) + P(none, j), T(i-1, j-1) + P(i, j) },
// with T(0, 0) = 0 and P the offline pairwise profile.
#include <cmath>
#include <vector>

#include "plan.hpp"

namespace {
constexpr int32_t kMaxSegments = 4096;
}

extern "C" tpslice_status_t tpslice_strand_schedule(const double* P, int32_t nf, int32_t nb, int32_t* steps,
                                                    int32_t* n_steps, double* makespan) {
  tps::clear_error();
  if (!P || !steps || !n_steps || !makespan) return tps::fail(TPSLICE_ERR_INVALID, "a pointer argument is NULL");
  if (nf < 0 || nb < 0 || nf > kMaxSegments || nb > kMaxSegments)
    return tps::fail(TPSLICE_ERR_SHAPE, "segment counts %d and %d must lie in [0, %d]", nf, nb, kMaxSegments);
  const int64_t W = int64_t(nb) + 1;
  for (int64_t i = 0; i <= nf; ++i)
    for (int64_t j = 0; j <= nb; ++j) {
      if (i == 0 && j == 0) continue;
      const double v = P[i * W + j];
      if (!std::isfinite(v) || v < 0.0)
        return tps::fail(TPSLICE_ERR_INVALID, "P(%lld, %lld) = %g is not a finite time >= 0", (long long)i,
                         (long long)j, v);
    }
  // T[i][j]: the best makespan of the first i forward and j backward segments; `from` the step that
  // reached it (0 forward alone, 1 backward alone, 2 a pair). Ties go to the pair, then the forward.
  std::vector<double> T(size_t(nf + 1) * size_t(W), 0.0);
  std::vector<uint8_t> from(T.size(), 0);
  for (int64_t i = 0; i <= nf; ++i)
    for (int64_t j = 0; j <= nb; ++j) {
      if (i == 0 && j == 0) continue;
      double best = INFINITY;
      uint8_t how = 0;
      if (i > 0 && j > 0) {
        best = T[(i - 1) * W + (j - 1)] + P[i * W + j];
        how = 2;
      }
      if (i > 0) {
        const double c = T[(i - 1) * W + j] + P[i * W];
        if (c < best) { best = c; how = 0; }
      }
      if (j > 0) {
        const double c = T[i * W + (j - 1)] + P[j];
        if (c < best) { best = c; how = 1; }
      }
      T[i * W + j] = best;
      from[i * W + j] = how;
    }
  // the steps, traced back from (nf, nb) and written in execution order as (forward, backward)
  // pairs of 1-based segment numbers, 0 for none
  std::vector<int32_t> rev;
  for (int64_t i = nf, j = nb; i > 0 || j > 0;) {
    const uint8_t how = from[i * W + j];
    const int32_t fi = how != 1 ? int32_t(i) : 0, bj = how != 0 ? int32_t(j) : 0;
    rev.push_back(bj);
    rev.push_back(fi);
    if (how != 1) --i;
    if (how != 0) --j;
  }
  const int32_t n = int32_t(rev.size() / 2);
  for (int32_t k = 0; k < n; ++k) {
    steps[2 * k] = rev[rev.size() - 1 - 2 * k];
    steps[2 * k + 1] = rev[rev.size() - 2 - 2 * k];
  }
  *n_steps = n;
  *makespan = T[size_t(nf) * size_t(W) + size_t(nb)];
  return TPSLICE_OK;
}
