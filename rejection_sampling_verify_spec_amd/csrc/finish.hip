// finish.hip -- the draw as a kernel of its own: k_draw_jobs, G workgroups
// per job, runs the tile pass over the drawn row(s) and, in the last
// workgroup to finish, the inverse-CDF pick over the tile records. A job is
// either written by an earlier kernel (one per request of a token tree) or,
// for draft-token sampling, built by the kernel from the row's chunk
// partials (one per logit row).
// The draw itself (tail.h) is the one the chain kernel runs [Primer 考点2
// residual; 考点4 bonus].
#include "tail.h"

#include <stdlib.h>

namespace sv {

constexpr int kNW = 4;  // waves per workgroup

// A job written by an earlier kernel, read by the whole wave into scalar
// registers (lane i loads 64-bit word i).
__device__ __forceinline__ SampleJob load_job(const SampleJob* src, int lane) {
  static_assert(sizeof(SampleJob) % 8 == 0, "job of 64-bit words");
  constexpr int nw = (int)(sizeof(SampleJob) / 8);
  uint64_t mine = 0;
  if (lane < nw) mine = reinterpret_cast<const uint64_t*>(src)[lane];
  uint64_t w[nw];
#pragma unroll
  for (int i = 0; i < nw; ++i) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)mine, i);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(mine >> 32), i);
    w[i] = ((uint64_t)hi << 32) | lo;
  }
  SampleJob J;
  __builtin_memcpy(&J, w, sizeof(J));
  return J;
}

struct DrawArgs {
  const void* tgt;
  const void* dft;
  int V;
  int G;                 // workgroups per job
  int B;                 // jobs
  const SampleJob* jobs; // [B]
  TileRec* recs;         // [B, ntile]
  const Partial* part;   // chunk partials (masses of skipped chunks)
  int nchunk;
  long long RT;          // target rows: draft row d has partials at row RT + d
  int* done;             // [B] workgroups finished with their tiles (zeroed by the streaming kernel)
  int32_t* out;
  int out_width;
  int force_exact;
  // draft-token sampling (jobs == nullptr): job b is row b of `tgt`, built here
  int chunk_vecs;
  const float* temperature;  // [B]
  const float* u;            // [B]
};

// The sampling job of logit row r, by one whole wave (draft-token sampling
// [Primer 考点1; Edge page, scheduler section: temperature softmax
// exp((l - max)/T) / sum]): the row maximum merged from the chunk partials
// (largest maximum, lowest index on ties), the greedy token for T == 0, or a
// bonus-type job over the row; chunks whose maximum lies more than -kTinyExp
// below the row maximum hold only masses below 2^-50 of it (at most 2^-36 in
// all): their tiles are not read again, their mass (into mass_t, lane k for
// chunk k) comes from the partial (16-byte aligned rows, so that chunks start
// on tile boundaries). One round of loads: lane k holds partial k throughout
// (rows of up to 64 chunks; longer rows skip nothing). With `write`, lane 0
// stores the token of a row without a draw (the greedy token, or -1 for an
// unusable temperature, uniform or row).
template <int DT>
__device__ __forceinline__ SampleJob row_job(const void* logits, int V, const Partial* part, int nchunk,
                                             int chunk_vecs, long long r, float T, float ur, int lane,
                                             int32_t* out_r, bool write, double* mass_t) {
  const bool t_ok = temperature_ok(T);
  const bool greedy = T == 0.0f;
  float M = -INFINITY;
  int idx = -1;
  bool bad = false;
  Partial q0{};
  bool have0 = false;
  if (t_ok) {
    const Partial* p = part + r * nchunk;
    for (int k = lane; k < nchunk; k += 64) {
      const Partial q = read_partial(p + k);
      if (k == lane) {
        q0 = q;
        have0 = true;
      }
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
  constexpr int es = sizeof(typename Elem<DT>::T), epv = Elem<DT>::kPerVec;
  const long long ctok = (long long)chunk_vecs * epv;
  const int tok = tile_tokens(DT);
  const bool row_aligned =
      ((reinterpret_cast<uintptr_t>(logits) + (uintptr_t)r * (uintptr_t)V * es) & 15u) == 0;
  unsigned long long skip = 0ull;
  if (ok && !greedy && row_aligned && nchunk > 1 && nchunk <= 64 && ctok % tok == 0) {
    const bool tiny = have0 && (q0.m == -INFINITY || (q0.m - M) * c32_of(T) < kTinyExp);
    skip = __ballot(tiny);
    if (have0 && tiny)
      mass_t[lane] = q0.m == -INFINITY
                         ? 0.0
                         : (double)partial_s(q0) * exp2_f64(((double)q0.m - (double)M) * (double)c32_of(T));
  }
  SampleJob J{};
  J.kind = JOB_NONE;
  if (ok && greedy) {
    if (write && lane == 0) *out_r = idx;
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
  } else if (write && lane == 0) {
    *out_r = -1;
  }
  return J;
}

// Workgroups (b, g), g < G, of job b: wave w of workgroup g takes the tiles
// g*kNW + w, + G*kNW, ... that are read (tiles of skipped chunks get their
// record from the chunk's partial); the last workgroup to finish runs the pick.
template <int DT, bool STAGED>
__global__ __launch_bounds__(kNW * 64) __attribute__((amdgpu_waves_per_eu(4))) void k_draw_jobs(DrawArgs A) {
  __shared__ union {
    TileSpace<kNW> ts;
    PickSpace<kNW> pick;
  } u;
  __shared__ double tab[64];                 // 2^{j/64}
  __shared__ double mass_t[64], mass_d[64];  // masses of the skipped chunks
  __shared__ SampleJob s_job;
  __shared__ int s_last;
  const JobPart jp = xcd_job_part(blockIdx.x, A.G);
  if (jp.job >= A.B) return;  // padding of the grid to whole XCD rounds
  const int b = jp.job, g = jp.part;
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  if (tid < 64) tab[tid] = exp2_f64((double)tid * 0.015625);
  SampleJob J;
  if (A.jobs) {
    J = load_job(A.jobs + b, lane);
  } else {  // a row of draft-token sampling: its job (and the masses of the chunks it skips) from its
            // partials; workgroup 0 writes a greedy token
    if (wv == 0) {
      const SampleJob Jw = row_job<DT>(A.tgt, A.V, A.part, A.nchunk, A.chunk_vecs, b, A.temperature[b], A.u[b],
                                       lane, A.out + (long long)b * A.out_width, g == 0, mass_t);
      if (lane == 0) s_job = Jw;
    }
    __syncthreads();
    J = uniform_job(s_job);
  }
  if (J.kind == JOB_NONE) return;
  const bool res = J.kind == JOB_RESIDUAL;
  if (A.jobs && J.skip && tid < 64 && tid < A.nchunk) {
    auto mass = [&](long long prow, float m_row) -> double {
      const Partial q = read_partial(A.part + prow * A.nchunk + tid);
      return q.m == -INFINITY ? 0.0
                              : (double)partial_s(q) * exp2_f64(((double)q.m - (double)m_row) * (double)J.c32);
    };
    mass_t[tid] = mass(J.trow, J.mt);
    if (res) mass_d[tid] = mass(A.RT + J.drow, J.md);
  }
  __syncthreads();
  constexpr int es = sizeof(typename Elem<DT>::T);
  const char* trow = reinterpret_cast<const char*>(A.tgt) + (size_t)J.trow * (size_t)A.V * es;
  const char* drow = reinterpret_cast<const char*>(A.dft) + (size_t)J.drow * (size_t)A.V * es;
  const int ntile = tiles_per_row(A.V, DT);
  TileRec* recs = A.recs + (long long)b * ntile;
  if (res)
    wave_tiles<DT, true, kNW>(trow, drow, A.V, ntile, g * kNW + wv, A.G * kNW, J, recs, mass_t, mass_d, u.ts, tab,
                              wv, lane);
  else
    wave_tiles<DT, false, kNW>(trow, drow, A.V, ntile, g * kNW + wv, A.G * kNW, J, recs, mass_t, mass_d, u.ts, tab,
                               wv, lane);
  // the records are complete before the count; the last workgroup picks
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) s_last = atomicAdd(A.done + b, 1) == A.G - 1;
  __syncthreads();
  if (!s_last) return;
  pick<DT, kNW, STAGED>(trow, drow, A.V, ntile, J, recs, A.out + (long long)b * A.out_width + J.pos, A.force_exact,
                        u.pick, tab);
}

namespace {
int device_cus_finish() {
  static int cus = 0;
  if (!cus) {
    int dev = 0, c = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c < 1)
      c = 1;
    cus = c;
  }
  return cus;
}
}  // namespace

hipError_t launch_finish_jobs(int dt, const void* tgt, const void* dft, int V, int B, SampleJob* jobs,
                              TileRec* recs, const Partial* part, int nchunk, long long RT, int* done, int32_t* out,
                              int out_width, int force_exact, hipStream_t st, int chunk_vecs,
                              const float* temperature, const float* u) {
  if (B == 0) return hipSuccess;
  // workgroups per job: enough for about four per CU, and 2 to 16 (two per job
  // balance 1280 sampled rows better than one; 16 per job draw the 32 rows of
  // the tree workload 2 us faster than 8; SPECVERIFY_JOB_GROUPS overrides)
  const long long want = (4ll * device_cus_finish() + B - 1) / B;
  int G = (int)(want < 2 ? 2 : (want > 16 ? 16 : want));
  if (const char* e = getenv("SPECVERIFY_JOB_GROUPS")) {
    const int g = atoi(e);
    if (g >= 1 && g <= 64) G = g;
  }
  if (xcd_grid(B, G) > 0x7fffffffLL) G = 1;
  const DrawArgs A{tgt, dft, V, G, B, jobs, recs, part, nchunk, RT, done, out, out_width, force_exact,
                   chunk_vecs, temperature, u};
  const dim3 grid((unsigned)xcd_grid(B, G)), blk(kNW * 64);
  const bool staged = tiles_per_row(V, dt) <= kPickStage;
  if (dt == 1) {
    if (staged) hipLaunchKernelGGL((k_draw_jobs<1, true>), grid, blk, 0, st, A);
    else hipLaunchKernelGGL((k_draw_jobs<1, false>), grid, blk, 0, st, A);
  } else {
    if (staged) hipLaunchKernelGGL((k_draw_jobs<0, true>), grid, blk, 0, st, A);
    else hipLaunchKernelGGL((k_draw_jobs<0, false>), grid, blk, 0, st, A);
  }
  return hipGetLastError();
}

}  // namespace sv
