// accept.h -- row statistics for the tree kernels (device code): the row max m
// and Z = sum 2^{(l - m) c}, merged in fp64 from the per-chunk partials of the
// row-statistics kernel, so that p(x) = 2^{(l_x - m) c} / Z [Primer 考点2].
#pragma once

#include "sv_internal.h"

namespace sv {

struct RowStat {
  float m;   // row max
  double Z;  // sum 2^{(x-m)c32}
  int idx;   // greedy argmax
  bool ok;
};

// Running merge of a row's chunk partials, fed in ascending token order (so a
// strict comparison keeps the lowest index of a tied maximum).
struct RowMerge {
  float M = -INFINITY;
  int idx = -1;
  bool bad = false;
  double Z = 0.0;

  __device__ __forceinline__ void add(const Partial& q, double c, bool greedy) {
    bad |= partial_bad(q, greedy);
    const float s = partial_s(q);
    if (q.m > M) {
      // new running maximum: rescale what was summed so far
      if (!greedy && M > -INFINITY) Z *= exp2_f64(((double)M - (double)q.m) * c);
      M = q.m;
      idx = partial_idx(q);
      if (!greedy) Z += (double)s;
    } else if (!greedy && q.m > -INFINITY) {
      Z += (double)s * exp2_f64(((double)q.m - (double)M) * c);
    }
  }

  __device__ __forceinline__ RowStat finish(bool greedy) const {
    RowStat r{M, 0.0, idx, !bad && M > -INFINITY && M < INFINITY};
    if (greedy || !r.ok) return r;
    r.Z = Z;
    r.ok = Z > 0.0 && Z < 1e308;
    return r;
  }
};

// Partials are read K at a time, all in flight together (one round of loads
// for rows of up to K chunks).
constexpr int kMergeLoads = 16;

template <int K>
__device__ __forceinline__ void load_partials(const Partial* __restrict__ p, int nchunk, int k0, bool use,
                                              Partial (&q)[K]) {
#pragma unroll
  for (int u = 0; u < K; ++u) q[u] = use && k0 + u < nchunk ? read_partial(p + k0 + u) : Partial{-INFINITY, 1u};
}

// Merge the chunk partials of one row.
template <int K = kMergeLoads>
__device__ __forceinline__ RowStat merge_row(const Partial* __restrict__ p, int nchunk, float c32, bool greedy) {
  RowMerge r;
  const double c = (double)c32;
  for (int k0 = 0; k0 < nchunk; k0 += K) {
    Partial q[K];
    load_partials<K>(p, nchunk, k0, true, q);
#pragma unroll
    for (int u = 0; u < K; ++u) r.add(q[u], c, greedy);  // past the row: {-inf, 1}, a no-op
  }
  return r.finish(greedy);
}

// Merge two rows at once (the second only when `two`), with the loads of both
// in flight together.
__device__ __forceinline__ void merge_rows2(const Partial* __restrict__ p0, bool greedy0, const Partial* __restrict__ p1,
                                            bool two, int nchunk, float c32, RowStat& r0, RowStat& r1) {
  RowMerge a, b;
  const double c = (double)c32;
  for (int k0 = 0; k0 < nchunk; k0 += kMergeLoads) {
    Partial q0[kMergeLoads], q1[kMergeLoads];
    load_partials<kMergeLoads>(p0, nchunk, k0, true, q0);
    load_partials<kMergeLoads>(p1, nchunk, k0, two, q1);
#pragma unroll
    for (int u = 0; u < kMergeLoads; ++u) {  // past the row (or no second row): {-inf, 1}, a no-op
      a.add(q0[u], c, greedy0);
      b.add(q1[u], c, false);
    }
  }
  r0 = a.finish(greedy0);
  r1 = b.finish(false);
}

}  // namespace sv
