// sv_internal.h -- shared types and device helpers of libspecverify (gfx950).
//
// A verify call runs three stages over the caller's batch:
//   1. streaming statistics (row_stats.hip, stream.h): one read of every logit
//      row the method reads -> per (row, chunk) max and sum of 2^{(x-max)c}
//      (T > 0) or max and lowest argmax (T == 0), in fp32 from 16-byte loads;
//   2. acceptance: per request, the chunk partials merged in fp64, the test
//      at every drafted position (or tree node), the first rejection, greedy
//      outputs and one sampling job;
//   3. draw: a tile pass over the drawn row(s) (fp32 triage, fp64 where
//      masses matter) and an inverse-CDF pick in fp64.
// Chain layouts run stages 2 and 3 in one kernel with a few workgroups per
// request (verify.hip); token trees run them as separate kernels (accept.hip,
// finish.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int kTPB = 256;        // threads per workgroup (4 waves of 64)
constexpr int kU = 4;            // 16-byte vectors per thread per step
constexpr int kGrp = 5;          // groups of undecided residual tokens kept per tile
constexpr double kLog2e = 1.4426950408889634073599246810019;
constexpr double kRhoBand = 1e-5;  // relative half-width of the undecided band around rho

// Layout of requests over rows.
enum LayoutMode : int { LAYOUT_DENSE = 0, LAYOUT_RAGGED = 1, LAYOUT_TREE = 2, LAYOUT_ROWS = 3 };

struct Layout {
  int mode;
  int B;
  int gamma;            // dense gamma, ragged gamma_max, tree N (nodes)
  const int32_t* cu;    // ragged: cu_gamma [B+1]
  int total_draft;      // ragged: rows of the draft array
  long long RT, RD;     // rows of the target and draft arrays
};

// Partial statistics of one (row, chunk), published as one 64-bit word.
//   m : chunk maximum (exact value of a logit), -inf if none;
//   w : T > 0 : bits of s = sum over the chunk of 2^{(x - m) c} (s >= 1 when
//               m is finite, 0 when m = -inf, NaN when the chunk holds a NaN
//               or a +inf);
//       T == 0: lowest index of the maximum + 2 (>= 1), or kGreedyBad when the
//               chunk holds a NaN or a +inf.
struct Partial {
  float m;
  uint32_t w;
};
constexpr uint32_t kGreedyBad = 0xffffffffu;

__device__ __forceinline__ Partial sampling_partial(float m, float s) { return Partial{m, __float_as_uint(s)}; }
__device__ __forceinline__ Partial greedy_partial(float m, int idx, bool bad) {
  return Partial{m, bad ? kGreedyBad : (uint32_t)(idx + 2)};
}
__device__ __forceinline__ float partial_s(const Partial& p) { return __uint_as_float(p.w); }
__device__ __forceinline__ int partial_idx(const Partial& p) { return p.w == kGreedyBad ? -1 : (int)p.w - 2; }
// bad for either kind: NaN sum or the greedy flag
__device__ __forceinline__ bool partial_bad(const Partial& p, bool greedy) {
  return greedy ? p.w == kGreedyBad : !(partial_s(p) == partial_s(p));
}

// Partials as 64-bit words (m in the low half, w in the high half: the
// in-memory order of the struct), written and read as single device-scope
// accesses.
__device__ __forceinline__ void publish_partial(Partial* p, Partial v) {
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), ((uint64_t)v.w << 32) | (uint64_t)__float_as_uint(v.m),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ Partial read_partial(const Partial* p) {
  const uint64_t x = __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<Partial*>(p)), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return Partial{__uint_as_float((uint32_t)x), (uint32_t)(x >> 32)};
}

enum JobKind : int { JOB_NONE = 0, JOB_BONUS = 1, JOB_RESIDUAL = 2 };

// One sampling job per request, written by the accept kernels.
struct SampleJob {
  int kind;
  int pos;            // output column of the drawn token
  long long trow;     // target row (global)
  long long drow;     // draft row (global, residual only)
  double c64;         // log2(e) / T
  double rho;         // estimate of Z_t / Z_d (residual only)
  float mt, md;       // row maxima (exact)
  float u;            // sampling uniform
  float c32;          // fl32(c64): argument of the fp32 exponential for negligible masses
  unsigned long long skip;  // row chunks whose tiles are not read (bit k = chunk k)
  int chunk_tiles;    // tiles per chunk when skip != 0
  int pad;
  double slow;        // residual: a lower bound of the residual total S (units of the target row maximum)
};

// Per (job, tile) record of the sampling pass (fp64 sums in a fixed order).
// Undecided tokens (likelihood ratio inside the band around rho~) are kept
// as groups of equal logit difference l_t - l_d: a group shares one ratio,
// hence one residual sign, and contributes max(0, sum e_t - rho sum e_d).
struct TileRec {
  double zt;          // sum of e_t
  double zd;          // sum of e_d (residual); the exact tile mass once the pick has run
  double dpos;        // sum over decided-positive tokens of (e_t - rho~ e_d)
  double bpos;        // sum over decided-positive tokens of e_d
  int ngrp;           // number of groups (>= 0), or one of the Rec* codes below
  int pad;
  double get[kGrp];   // per group: sum of e_t
  double ged[kGrp];   // per group: sum of e_d
  double pad2;
};


// Tokens per sampling tile: 4 16-byte vectors per lane when one wave owns a
// tile (2048 bf16 or 1024 fp32 tokens).
template <int DT> struct TileTok { static constexpr int value = DT == 1 ? 2048 : 1024; };
__host__ __device__ inline int tile_tokens(int dt) { return dt == 1 ? 2048 : 1024; }
__host__ __device__ inline int tiles_per_row(int V, int dt) { return (V + tile_tokens(dt) - 1) / tile_tokens(dt); }

// TileRec::ngrp codes.
constexpr int kRecOverflow = -1;    // undecided tokens did not fit: the pick recomputes the tile
constexpr int kRecRecomputed = -2;  // recomputed by the pick: exact residual mass in zd
constexpr int kRecChunkHead = -4;   // first tile of a skipped chunk: zt holds the whole chunk's mass
constexpr int kRecChunkBody = -5;   // other tiles of a skipped chunk: mass 0 here

// ---------------------------------------------------------------------------
// Temperature handling shared by every kernel: identical expressions give
// identical values in every kernel.

__device__ __forceinline__ bool temperature_ok(float T) {
  // usable: 0 (greedy) or a normal positive finite float
  return T == 0.0f || (T >= 1.17549435e-38f && T <= 3.40282347e+38f);
}
__device__ __forceinline__ float c32_of(float T) { return (float)(kLog2e / (double)T); }
__device__ __forceinline__ double c64_of(float T) { return kLog2e / (double)T; }
__device__ __forceinline__ bool uniform_ok(float u) { return u >= 0.0f && u < 1.0f; }  // false for NaN

// ---------------------------------------------------------------------------
// Element access.

template <int DT> struct Elem;
template <> struct Elem<0> {  // float32
  using T = float;
  static constexpr int kPerVec = 4;
  __device__ __forceinline__ static float at(const void* p, long long i) {
    return reinterpret_cast<const float*>(p)[i];
  }
};
template <> struct Elem<1> {  // bfloat16 bit patterns
  using T = uint16_t;
  static constexpr int kPerVec = 8;
  __device__ __forceinline__ static float at(const void* p, long long i) {
    uint32_t b = (uint32_t)reinterpret_cast<const uint16_t*>(p)[i] << 16;
    return __uint_as_float(b);
  }
};

// Unpack a 16-byte vector into floats.
template <int DT> __device__ __forceinline__ void unpack(const uint4& w, float* x);
template <> __device__ __forceinline__ void unpack<0>(const uint4& w, float* x) {
  x[0] = __uint_as_float(w.x); x[1] = __uint_as_float(w.y);
  x[2] = __uint_as_float(w.z); x[3] = __uint_as_float(w.w);
}
template <> __device__ __forceinline__ void unpack<1>(const uint4& w, float* x) {
  x[0] = __uint_as_float(w.x << 16); x[1] = __uint_as_float(w.x & 0xffff0000u);
  x[2] = __uint_as_float(w.y << 16); x[3] = __uint_as_float(w.y & 0xffff0000u);
  x[4] = __uint_as_float(w.z << 16); x[5] = __uint_as_float(w.z & 0xffff0000u);
  x[6] = __uint_as_float(w.w << 16); x[7] = __uint_as_float(w.w & 0xffff0000u);
}

// Vector split of one row: `head` scalar elements until a 16-byte boundary,
// `nvec` full vectors, then `tail` scalar elements.
struct RowSplit {
  int head, nvec, tail;
};
template <int DT>
__device__ __forceinline__ RowSplit split_row(const void* row, int V) {
  constexpr int es = sizeof(typename Elem<DT>::T);
  constexpr int epv = Elem<DT>::kPerVec;
  uintptr_t a = reinterpret_cast<uintptr_t>(row);
  int head = (int)(((16u - (unsigned)(a & 15u)) & 15u) / es);
  if (head > V) head = V;
  int nvec = (V - head) / epv;
  return RowSplit{head, nvec, V - head - nvec * epv};
}

// ---------------------------------------------------------------------------
// 2^a in double precision for a <= 0 (NaN propagates): a = n + f with
// n = rint(a), |f| <= 1/2, and 2^f = exp(f ln 2) by its Taylor series to
// degree 13 (coefficients ln2^k / k!, truncation below 5e-18 relative).
__device__ __forceinline__ double exp2_f64(double a) {
  if (!(a >= -1100.0)) return (a != a) ? a : 0.0;
  double n = __builtin_rint(a);
  double f = a - n;
  double p = 0x1.816193166d0f9p-40;
  p = __builtin_fma(p, f, 0x1.c3bd650fc2986p-36);
  p = __builtin_fma(p, f, 0x1.e8cac7351bb25p-32);
  p = __builtin_fma(p, f, 0x1.e4cf5158b8ecap-28);
  p = __builtin_fma(p, f, 0x1.b5253d395e7c4p-24);
  p = __builtin_fma(p, f, 0x1.62c0223a5c824p-20);
  p = __builtin_fma(p, f, 0x1.ffcbfc588b0c7p-17);
  p = __builtin_fma(p, f, 0x1.430912f86c787p-13);
  p = __builtin_fma(p, f, 0x1.5d87fe78a6731p-10);
  p = __builtin_fma(p, f, 0x1.3b2ab6fba4e77p-7);
  p = __builtin_fma(p, f, 0x1.c6b08d704a0c0p-5);
  p = __builtin_fma(p, f, 0x1.ebfbdff82c58fp-3);
  p = __builtin_fma(p, f, 0x1.62e42fefa39efp-1);
  p = __builtin_fma(p, f, 1.0);
  return __builtin_ldexp(p, (int)n);
}

// fp32 2^x on the hardware transcendental unit (v_exp_f32).
__device__ __forceinline__ float exp2_f32(float x) { return __builtin_amdgcn_exp2f(x); }

// Masses below 2^-50 of their row maximum (fp32 exponent argument below this)
// are evaluated on the fp32 exponential unit.
constexpr float kTinyExp = -50.0f;
// Masses below 2^-100 of their row maximum are left out of the draw's tile
// sums when a whole 16-byte vector of them, in every lane of a wave, lies
// there: at most V 2^-100 of the row maximum in all, below the double-precision
// resolution of any CDF position.
constexpr float kDropExp = -100.0f;

// ---------------------------------------------------------------------------
// Wave64 / workgroup reductions.

template <typename T, typename F>
__device__ __forceinline__ T wave_reduce(T v, F op) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = op(v, __shfl_xor(v, off, 64));
  return v;
}

// Workgroups of one job on one XCD. The dispatcher hands consecutive
// workgroup indices to the 8 XCDs of the part in turn, and each XCD has its
// own L2; a job whose G workgroups exchange records and re-read tiles keeps
// that traffic in one L2 when all its workgroups sit on the same XCD. Index i
// of a grid of jobs_padded * G workgroups (jobs_padded a multiple of kXcds)
// maps to job x + kXcds * (s / G) and part s % G, with x = i % kXcds and
// s = i / kXcds. Only placement depends on it: any dispatch order gives the
// same results.
constexpr int kXcds = 8;
struct JobPart {
  int job, part;
};
__device__ __forceinline__ JobPart xcd_job_part(int i, int G) {
  const int x = i % kXcds, s = i / kXcds;
  return JobPart{x + kXcds * (s / G), s % G};
}
__host__ __device__ inline long long xcd_grid(long long jobs, int G) {
  return (jobs + kXcds - 1) / kXcds * kXcds * G;
}

// Lossless tree walk: at most this many teams run at once (the workspace holds
// two residual buffers of one row per team).
constexpr int kLLMaxTeams = 256;

// Host-side launchers (defined next to their kernels).
hipError_t launch_row_stats(int dt, const void* tgt, const void* dft, int V, const Layout& L,
                            const float* temperature, int chunk_vecs, int nchunk, Partial* part, int* zero_counts,
                            hipStream_t st);
hipError_t launch_accept_tree(int dt, const void* tgt, const void* dft, int V, const Layout& L, int max_depth,
                              const int32_t* tokens, const int32_t* parents, const float* ua, const float* us,
                              const float* temperature, const Partial* part, int nchunk, int32_t* out,
                              int32_t* out_nodes, int32_t* num_acc, SampleJob* jobs, hipStream_t st);
hipError_t launch_verify_chain(int dt, const void* tgt, const void* dft, int V, const Layout& L,
                               const int32_t* tokens, const float* ua, const float* us, const float* temperature,
                               const Partial* part, int nchunk, int chunk_vecs, TileRec* recs, int* done,
                               int32_t* out, int out_width, int32_t* num_acc, float* diag, int force_exact,
                               hipStream_t st);
// The draw of each job (jobs != nullptr: written by an earlier kernel), or of
// each of B logit rows of draft-token sampling (jobs == nullptr: the kernel
// builds a row's job from its partials, chunk_vecs, temperature[b] and u[b]).
hipError_t launch_finish_jobs(int dt, const void* tgt, const void* dft, int V, int B, SampleJob* jobs,
                              TileRec* recs, const Partial* part, int nchunk, long long RT, int* done, int32_t* out,
                              int out_width, int force_exact, hipStream_t st, int chunk_vecs = 0,
                              const float* temperature = nullptr, const float* u = nullptr);
hipError_t launch_stats_finalize(const Partial* part, int nchunk, int rows, const float* temperature,
                                 float* out_max, float* out_logz, int32_t* out_argmax, hipStream_t st);

}  // namespace sv
