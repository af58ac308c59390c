// accept.h -- row statistics and token probabilities for the tree accept
// kernel (device code): p(x) = 2^{(l_x - m) c} / Z, with Z merged in fp64 from
// the per-chunk partials of the row-statistics kernel [Primer 考点2].
#pragma once

#include "sv_internal.h"

namespace sv {

struct RowStat {
  float m;   // row max
  double Z;  // sum 2^{(x-m)c32}
  int idx;   // greedy argmax
  bool ok;
};

// Merge the chunk partials of one row (chunks in ascending token order, so a
// strict comparison keeps the lowest index of a tied maximum). Partials are
// read four at a time so their loads overlap.
__device__ __forceinline__ RowStat merge_row(const Partial* __restrict__ p, int nchunk, float c32, bool greedy) {
  float M = -INFINITY;
  int idx = -1;
  bool bad = false;
  double Z = 0.0;
  const double c = (double)c32;
  for (int k0 = 0; k0 < nchunk; k0 += 4) {
    Partial q[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) q[u] = k0 + u < nchunk ? read_partial(p + k0 + u) : Partial{-INFINITY, 1u};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      bad |= partial_bad(q[u], greedy);
      const float s = partial_s(q[u]);
      if (q[u].m > M) {
        // new running maximum: rescale what was summed so far
        if (!greedy && M > -INFINITY) Z *= exp2_f64(((double)M - (double)q[u].m) * c);
        M = q[u].m;
        idx = partial_idx(q[u]);
        if (!greedy) Z += (double)s;
      } else if (!greedy && q[u].m > -INFINITY) {
        Z += (double)s * exp2_f64(((double)q[u].m - (double)M) * c);
      }
    }
  }
  RowStat r{M, 0.0, idx, !bad && M > -INFINITY && M < INFINITY};
  if (greedy || !r.ok) return r;
  r.Z = Z;
  r.ok = Z > 0.0 && Z < 1e308;
  return r;
}

// probability of token x in a row with statistics st
template <int DT>
__device__ __forceinline__ double prob_at(const void* base, long long row, int V, int x, const RowStat& st, float c32) {
  float l = Elem<DT>::at(base, row * (long long)V + x);
  return exp2_f64(((double)l - (double)st.m) * (double)c32) / st.Z;
}

}  // namespace sv
