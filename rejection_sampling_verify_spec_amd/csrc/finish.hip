// finish.hip -- the draw of token-tree requests as kernels of their own, after
// the tree acceptance kernel has written one sampling job per request:
//   k_tiles (G workgroups per request): the tile pass over the drawn row(s);
//   k_pick (one workgroup per request): the inverse-CDF search over the tile
//   records.
// The draw itself (tail.h) is the one the chain kernel runs [Primer 考点2
// residual; 考点4 bonus].
#include "tail.h"

namespace sv {

constexpr int kNW = 4;  // waves per workgroup

// Workgroup (b, g), g < G: tiles g*kNW + i*G*kNW + [0, kNW) of request b's
// drawn row(s), one per wave.
template <int DT>
__global__ __launch_bounds__(kNW * 64) void k_tiles(const void* __restrict__ tgt, const void* __restrict__ dft, int V,
                                               int G, const SampleJob* __restrict__ jobs,
                                               TileRec* __restrict__ recs) {
  __shared__ TileSpace<kNW> ts;
  __shared__ double exp2tab[64];
  __shared__ SampleJob sj;
  const int b = blockIdx.x / G, g = blockIdx.x - b * G;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (threadIdx.x < 64) exp2tab[threadIdx.x] = exp2_f64((double)threadIdx.x * 0.015625);
  if (threadIdx.x == 0) sj = jobs[b];
  __syncthreads();
  const SampleJob J = uniform_job(sj);
  if (J.kind == JOB_NONE) return;
  constexpr int es = sizeof(typename Elem<DT>::T);
  const char* trow = reinterpret_cast<const char*>(tgt) + (size_t)J.trow * (size_t)V * es;
  const char* drow = reinterpret_cast<const char*>(dft) + (size_t)J.drow * (size_t)V * es;
  const int ntile = tiles_per_row(V, DT);
  TileRec* R = recs + (long long)b * ntile;
  for (int base = g * kNW; base < ntile; base += G * kNW)
    wave_tile<DT, kNW>(trow, drow, V, ntile, base + wv, J, R, ts, exp2tab, wv, lane);
}

template <int DT, bool STAGED>
__global__ __launch_bounds__(kNW * 64) void k_pick(const void* __restrict__ tgt, const void* __restrict__ dft, int V,
                                              const SampleJob* __restrict__ jobs, TileRec* __restrict__ recs,
                                              int32_t* __restrict__ out, int out_width, int force_exact) {
  __shared__ PickSpace<kNW> ps;
  __shared__ double exp2tab[64];
  __shared__ SampleJob sj;
  if (threadIdx.x < 64) exp2tab[threadIdx.x] = exp2_f64((double)threadIdx.x * 0.015625);
  if (threadIdx.x == 0) sj = jobs[blockIdx.x];
  __syncthreads();
  const SampleJob J = uniform_job(sj);
  if (J.kind == JOB_NONE) return;
  const int b = blockIdx.x;
  constexpr int es = sizeof(typename Elem<DT>::T);
  const char* trow = reinterpret_cast<const char*>(tgt) + (size_t)J.trow * (size_t)V * es;
  const char* drow = reinterpret_cast<const char*>(dft) + (size_t)J.drow * (size_t)V * es;
  const int ntile = tiles_per_row(V, DT);
  pick<DT, kNW, STAGED>(trow, drow, V, ntile, J, recs + (long long)b * ntile,
                        out + (long long)b * out_width + J.pos, force_exact, ps, exp2tab);
}

// Workgroups per request of k_tiles: one per kNW tiles, capped so that the
// grid stays within 2^20 workgroups.
static int tiles_groups(int B, int V, int dt) {
  const int ntile = tiles_per_row(V, dt);
  int G = (ntile + kNW - 1) / kNW;
  const long long cap = (1ll << 20) / (B > 0 ? B : 1);
  if (G > cap) G = (int)cap;
  return G < 1 ? 1 : G;
}

hipError_t launch_finish_jobs(int dt, const void* tgt, const void* dft, int V, int B, SampleJob* jobs,
                              TileRec* recs, int32_t* out, int out_width, int force_exact, hipStream_t st) {
  if (B == 0) return hipSuccess;
  const int G = tiles_groups(B, V, dt);
  const bool staged = tiles_per_row(V, dt) <= kPickStage;
  const dim3 blk(kNW * 64);
  if (dt == 1) {
    hipLaunchKernelGGL(k_tiles<1>, dim3((unsigned)(B * G)), blk, 0, st, tgt, dft, V, G, jobs, recs);
    if (staged)
      hipLaunchKernelGGL((k_pick<1, true>), dim3((unsigned)B), blk, 0, st, tgt, dft, V, jobs, recs, out, out_width,
                         force_exact);
    else
      hipLaunchKernelGGL((k_pick<1, false>), dim3((unsigned)B), blk, 0, st, tgt, dft, V, jobs, recs, out, out_width,
                         force_exact);
  } else {
    hipLaunchKernelGGL(k_tiles<0>, dim3((unsigned)(B * G)), blk, 0, st, tgt, dft, V, G, jobs, recs);
    if (staged)
      hipLaunchKernelGGL((k_pick<0, true>), dim3((unsigned)B), blk, 0, st, tgt, dft, V, jobs, recs, out, out_width,
                         force_exact);
    else
      hipLaunchKernelGGL((k_pick<0, false>), dim3((unsigned)B), blk, 0, st, tgt, dft, V, jobs, recs, out, out_width,
                         force_exact);
  }
  return hipGetLastError();
}

}  // namespace sv
