// row_stats.hip -- the streaming row-statistics kernel (the first launch of
// every verify call and of the statistics entry point), and the per-row
// finalisation of the statistics entry point.
#include "stream.h"

#include <stdlib.h>

namespace sv {

__device__ __forceinline__ long long request_of_row(const Layout& L, long long r, bool draft) {
  switch (L.mode) {
    case LAYOUT_DENSE:
      return draft ? r / L.gamma : r / (L.gamma + 1);
    case LAYOUT_TREE:
      return draft ? r / (L.gamma - 1) : r / L.gamma;
    case LAYOUT_RAGGED: {
      // largest b in [0, B) with key(b) <= r; key(b) = cu[b] (+ b for target rows)
      int lo = 0, hi = L.B - 1;
      while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        long long key = (long long)L.cu[mid] + (draft ? 0 : mid);
        if (key <= r) lo = mid; else hi = mid - 1;
      }
      return lo;
    }
    default:
      return r;
  }
}

// One workgroup per (row, chunk); rows are the target rows, then the draft rows.
// NB: groups of 16-byte loads a thread has in flight at once (1 or 2).
// The first B workgroups also zero `zero_counts` (when given, B + 1 ints), the
// per-request counters of the chain tail kernel, and workgroup 0 stores the
// ragged layout's validity in zero_counts[B].
template <int DT, int NB>
__global__ __launch_bounds__(kTPB) void k_row_stats(const void* __restrict__ tgt, const void* __restrict__ dft,
                                                    int V, Layout L, const float* __restrict__ temperature,
                                                    int chunk_vecs, int nchunk, Partial* __restrict__ part,
                                                    int* __restrict__ zero_counts) {
  using E = Elem<DT>;
  const long long item = blockIdx.x;
  // (workgroups past the last item exist for the counters only)
  if (item < (L.RT + L.RD) * (long long)nchunk) {
    const long long row = item / nchunk;
    const int chunk = (int)(item - row * nchunk);
    const bool draft = row >= L.RT;
    const long long r = draft ? row - L.RT : row;
    long long b = request_of_row(L, r, draft);
    if (b < 0) b = 0;
    if (b >= L.B) b = L.B - 1;
    const float T = temperature[b];
    if (temperature_ok(T) && !(draft && T == 0.0f)) {
      const void* rowp =
          reinterpret_cast<const char*>(draft ? dft : tgt) + (size_t)r * (size_t)V * sizeof(typename E::T);
      row_chunk_stats<DT, NB>(rowp, V, chunk, chunk_vecs, T, part + item);
    }
  }
  // The stores for the kernel that follows come last: a store before the
  // cu_gamma reads of request_of_row could alias them, and the compiler would
  // then read cu_gamma through vector loads instead of the scalar cache.
  // Per-request counters start from zero.
  if (zero_counts && item < L.B && threadIdx.x == 0) zero_counts[item] = 0;
  // A ragged layout is checked once, here: it is usable when cu_gamma[0] == 0,
  // it never decreases, every step is at most gamma_max and cu_gamma[B] ==
  // total_draft (zero_counts[B] = 1 if so).
  if (zero_counts && item == 0 && L.mode == LAYOUT_RAGGED) {
    bool ok = threadIdx.x != 0 || (L.cu[0] == 0 && L.cu[L.B] == L.total_draft);
    for (int k = threadIdx.x; k < L.B; k += kTPB) {
      const int lo = L.cu[k], hi = L.cu[k + 1];
      ok = ok && hi >= lo && hi - lo <= L.gamma;
    }
    ok = __syncthreads_and(ok) != 0;
    if (threadIdx.x == 0) zero_counts[L.B] = ok ? 1 : 0;
  }
}

hipError_t launch_row_stats(int dt, const void* tgt, const void* dft, int V, const Layout& L,
                            const float* temperature, int chunk_vecs, int nchunk, Partial* part, int* zero_counts,
                            hipStream_t st) {
  long long grid = (L.RT + L.RD) * (long long)nchunk;
  if (zero_counts && grid < L.B) grid = L.B;  // every counter gets a workgroup
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  // Groups of loads in flight per thread: two (a whole 2048-vector chunk at
  // once; 78 VGPRs, six workgroups per CU for bf16) for the dense, tree and
  // row layouts; one (57 VGPRs, eight per CU) for chunks of a single group and
  // for the ragged layout, where two measured slower. Two instead of one,
  // measured on one box: large -1.4%, trees -1.0%, sampled rows -0.7%,
  // ragged +1.3%. SPECVERIFY_STREAM_GROUPS (1 or 2) overrides.
  static const int nb_env = [] {
    const char* e = getenv("SPECVERIFY_STREAM_GROUPS");
    const int v = e ? atoi(e) : 0;
    return v == 1 || v == 2 ? v : 0;
  }();
  const int nb = nb_env ? nb_env : (L.mode == LAYOUT_RAGGED || chunk_vecs < 2 * kTPB * kU ? 1 : 2);
  if (dt == 1) {
    if (nb == 2)
      hipLaunchKernelGGL((k_row_stats<1, 2>), dim3((unsigned)grid), dim3(kTPB), 0, st, tgt, dft, V, L, temperature,
                         chunk_vecs, nchunk, part, zero_counts);
    else
      hipLaunchKernelGGL((k_row_stats<1, 1>), dim3((unsigned)grid), dim3(kTPB), 0, st, tgt, dft, V, L, temperature,
                         chunk_vecs, nchunk, part, zero_counts);
  } else {
    if (nb == 2)
      hipLaunchKernelGGL((k_row_stats<0, 2>), dim3((unsigned)grid), dim3(kTPB), 0, st, tgt, dft, V, L, temperature,
                         chunk_vecs, nchunk, part, zero_counts);
    else
      hipLaunchKernelGGL((k_row_stats<0, 1>), dim3((unsigned)grid), dim3(kTPB), 0, st, tgt, dft, V, L, temperature,
                         chunk_vecs, nchunk, part, zero_counts);
  }
  return hipGetLastError();
}

// Per-row finalisation for the statistics entry point.
__global__ __launch_bounds__(64) void k_stats_finalize(const Partial* __restrict__ part, int nchunk, int rows,
                                                       const float* __restrict__ temperature,
                                                       float* __restrict__ out_max, float* __restrict__ out_logz,
                                                       int32_t* __restrict__ out_argmax) {
  int r = blockIdx.x * 64 + threadIdx.x;
  if (r >= rows) return;
  float T = temperature[r];
  const float qnan = __uint_as_float(0x7fc00000u);
  if (!temperature_ok(T)) {
    out_max[r] = qnan; out_logz[r] = qnan; out_argmax[r] = -1;
    return;
  }
  const bool greedy = T == 0.0f;
  const Partial* p = part + (long long)r * nchunk;
  float M = -INFINITY;
  int idx = -1;
  bool bad = false;
  for (int k = 0; k < nchunk; ++k) {
    const Partial q = read_partial(p + k);
    bad |= partial_bad(q, greedy);
    if (q.m > M) { M = q.m; idx = partial_idx(q); }
  }
  bool ok = !bad && M > -INFINITY && M < INFINITY;
  if (greedy) {
    out_max[r] = ok ? M : qnan;
    out_logz[r] = qnan;
    out_argmax[r] = ok ? idx : -1;
    return;
  }
  double c = (double)c32_of(T), Z = 0.0;
  for (int k = 0; k < nchunk; ++k) {
    const Partial q = read_partial(p + k);
    if (q.m > -INFINITY) Z += (double)partial_s(q) * exp2_f64(((double)q.m - (double)M) * c);
  }
  ok = ok && Z > 0.0 && Z < 1e308;
  out_max[r] = ok ? M : qnan;
  out_logz[r] = ok ? (float)log(Z) : qnan;
  out_argmax[r] = -1;
}

hipError_t launch_stats_finalize(const Partial* part, int nchunk, int rows, const float* temperature,
                                 float* out_max, float* out_logz, int32_t* out_argmax, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(k_stats_finalize, dim3((rows + 63) / 64), dim3(64), 0, st, part, nchunk, rows, temperature,
                     out_max, out_logz, out_argmax);
  return hipGetLastError();
}

}  // namespace sv
