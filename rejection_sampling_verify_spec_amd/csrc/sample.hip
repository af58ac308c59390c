// sample.hip -- draft-token sampling: one token per logit row from
// softmax(l/T), drawn with the inverse CDF of the verify draw, the way the
// draft model proposes the tokens that verification then tests [Primer 考点1;
// Edge page, scheduler section: temperature softmax exp((l - max)/T) / sum].
//
// A call runs the streaming statistics kernel over the rows, then
// k_sample_jobs (one wave per row: the row maximum from the chunk partials,
// the greedy token for T == 0, or a bonus-type sampling job with the row
// chunks it need not read), then the tile pass and pick of the verify draw
// over each row (finish.hip).
#include "sv_internal.h"

namespace sv {

constexpr int kJobRowsPerBlock = 4;  // one wave per row

template <int DT>
__global__ __launch_bounds__(kJobRowsPerBlock * 64) void k_sample_jobs(const void* __restrict__ logits, int V,
                                                                      const Partial* __restrict__ part, int nchunk,
                                                                      int chunk_vecs, int rows,
                                                                      const float* __restrict__ temperature,
                                                                      const float* __restrict__ u,
                                                                      SampleJob* __restrict__ jobs,
                                                                      int32_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const long long r = (long long)blockIdx.x * kJobRowsPerBlock + (threadIdx.x >> 6);
  if (r >= rows) return;
  const float T = temperature[r];
  const float ur = u[r];
  const bool t_ok = temperature_ok(T);
  const bool greedy = T == 0.0f;
  // merge of the row's chunk partials: largest maximum, lowest index on ties
  float M = -INFINITY;
  int idx = -1;
  bool bad = false;
  if (t_ok) {
    const Partial* p = part + r * nchunk;
    for (int k = lane; k < nchunk; k += 64) {
      const Partial q = read_partial(p + k);
      bad |= partial_bad(q, greedy);
      if (q.m > M) {
        M = q.m;
        idx = partial_idx(q);
      }
    }
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float M2 = __shfl_xor(M, off, 64);
    const int i2 = __shfl_xor(idx, off, 64);
    bad |= __shfl_xor((int)bad, off, 64) != 0;
    if (M2 > M || (M2 == M && (unsigned)i2 < (unsigned)idx)) {
      M = M2;
      idx = i2;
    }
  }
  const bool ok = t_ok && !bad && M > -INFINITY && M < INFINITY;
  // Row chunks whose maximum lies more than -kTinyExp below the row maximum
  // hold only masses below 2^-50 of it (at most 2^-36 in all): their tiles are
  // not read again, their mass comes from the partial (16-byte aligned rows,
  // so that chunks start on tile boundaries).
  constexpr int es = sizeof(typename Elem<DT>::T), epv = Elem<DT>::kPerVec;
  const long long ctok = (long long)chunk_vecs * epv;
  const int tok = tile_tokens(DT);
  const bool row_aligned =
      ((reinterpret_cast<uintptr_t>(logits) + (uintptr_t)r * (uintptr_t)V * es) & 15u) == 0;
  unsigned long long skip = 0ull;
  if (ok && !greedy && row_aligned && nchunk > 1 && nchunk <= 64 && ctok % tok == 0) {
    bool tiny = false;
    if (lane < nchunk) {
      const Partial q = read_partial(part + r * nchunk + lane);
      tiny = q.m == -INFINITY || (q.m - M) * c32_of(T) < kTinyExp;
    }
    skip = __ballot(tiny);
  }
  if (lane != 0) return;
  SampleJob J{};
  J.kind = JOB_NONE;
  if (ok && greedy) {
    out[r] = idx;
  } else if (ok && uniform_ok(ur)) {
    J.kind = JOB_BONUS;
    J.pos = 0;
    J.trow = r;
    J.drow = r;
    J.c64 = c64_of(T);
    J.c32 = c32_of(T);
    J.rho = 0.0;
    J.mt = M;
    J.md = 0.0f;
    J.u = ur;
    J.skip = skip;
    J.chunk_tiles = skip ? (int)(ctok / tok) : 0;
    J.slow = 0.0;
  } else {
    out[r] = -1;
  }
  jobs[r] = J;
}

hipError_t launch_sample_jobs(int dt, const void* logits, int V, const Partial* part, int nchunk, int chunk_vecs,
                              int rows, const float* temperature, const float* u, SampleJob* jobs, int32_t* out,
                              hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const long long grid = ((long long)rows + kJobRowsPerBlock - 1) / kJobRowsPerBlock;
  const dim3 g((unsigned)grid), b(kJobRowsPerBlock * 64);
  if (dt == 1)
    hipLaunchKernelGGL(k_sample_jobs<1>, g, b, 0, st, logits, V, part, nchunk, chunk_vecs, rows, temperature, u,
                       jobs, out);
  else
    hipLaunchKernelGGL(k_sample_jobs<0>, g, b, 0, st, logits, V, part, nchunk, chunk_vecs, rows, temperature, u,
                       jobs, out);
  return hipGetLastError();
}

}  // namespace sv
