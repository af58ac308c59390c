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

// Running merge of a row's chunk partials, fed in blocks in ascending token
// order.
struct RowMerge {
  float M = -INFINITY;
  int idx = -1;
  bool bad = false;
  double Z = 0.0;

  // K partials at once, in ascending token order: their maximum first (a
  // strict comparison keeps the lowest index of a tied maximum), then their
  // sum rescaled to it term by term (independent exponentials), merged into
  // the running statistic with at most one rescale.
  template <int K>
  __device__ __forceinline__ void add_block(const Partial (&q)[K], double c, bool greedy) {
    float bm = -INFINITY;
    int bi = -1;
#pragma unroll
    for (int u = 0; u < K; ++u) {
      bad |= partial_bad(q[u], greedy);
      if (q[u].m > bm) {
        bm = q[u].m;
        bi = partial_idx(q[u]);
      }
    }
    if (bm == -INFINITY) return;  // nothing but empty chunks (or past the row)
    double bz = 0.0;
    if (!greedy) {
#pragma unroll
      for (int u = 0; u < K; ++u)
        if (q[u].m > -INFINITY)
          bz += (double)partial_s(q[u]) * (q[u].m == bm ? 1.0 : exp2_f64(((double)q[u].m - (double)bm) * c));
    }
    if (bm > M) {
      if (!greedy && M > -INFINITY) Z *= exp2_f64(((double)M - (double)bm) * c);
      M = bm;
      idx = bi;
      if (!greedy) Z += bz;
    } else if (!greedy) {
      Z += bz * exp2_f64(((double)bm - (double)M) * c);
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
    r.add_block(q, c, greedy);  // past the row: {-inf, 1}, left out
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
    a.add_block(q0, c, greedy0);  // past the row (or no second row): {-inf, 1}, left out
    b.add_block(q1, c, false);
  }
  r0 = a.finish(greedy0);
  r1 = b.finish(false);
}

}  // namespace sv
