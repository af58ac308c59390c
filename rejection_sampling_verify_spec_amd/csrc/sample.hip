// sample.hip -- the drawn token of each request [Primer 考点2 residual
// P' = max(0, p_t - p_d) / sum; 考点4 bonus token from p_t when every draft
// passes], by inverse CDF y = min{ j : C_j > u S } in ascending token order.
//
// All masses are computed in double precision from the stored logits with
// e_t(j) = 2^{(l_t,j - m_t) c}, e_d(j) = 2^{(l_d,j - m_d) c}, c = log2(e)/T, so
// that the chosen token agrees with a double-precision sequential evaluation
// except when u S lies within ~1e-13 S of a CDF boundary. The residual in
// these units is q_j = max(0, e_t(j) - rho e_d(j)) with rho = Z_t / Z_d.
//
// Pass 1 (k_sample_tiles, one workgroup per job and tile of kTile tokens):
// Z_t and Z_d of the tile, and -- using the estimate rho~ from the fp32 row
// statistics -- the sums over tokens with e_t > rho~(1+band) e_d of
// (e_t - rho~ e_d) and of e_d; tokens inside the band are listed (they are
// the only ones whose residual sign the estimate cannot decide).
// Pass 2 (k_sample_pick, one workgroup per job): exact rho = Z_t / Z_d, the
// exact tile masses sum q = dpos + (rho~ - rho) bpos + listed tokens, the
// tile holding u S, and a fp64 prefix scan of that tile.
#include "sv_internal.h"

namespace sv {

template <int DT>
__device__ __forceinline__ double emass(const void* base, long long row, int V, int j, float m, double c) {
  return exp2_f64(((double)Elem<DT>::at(base, row * (long long)V + j) - (double)m) * c);
}

__device__ __forceinline__ double block_sum(double v, double* red) {
  v = wave_reduce(v, [](double a, double b) { return a + b; });
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double t = red[0];
  for (int w = 1; w < kTPB / 64; ++w) t += red[w];
  return t;
}

template <int DT>
__global__ __launch_bounds__(kTPB) void k_sample_tiles(const void* __restrict__ tgt, const void* __restrict__ dft,
                                                       int V, int ntile, const SampleJob* __restrict__ jobs,
                                                       TileRec* __restrict__ recs) {
  const int b = blockIdx.x / ntile, k = blockIdx.x - b * ntile;
  const SampleJob J = jobs[b];
  if (J.kind == JOB_NONE) return;
  const int tid = threadIdx.x;
  const int j0 = k * kTile, j1 = min(V, j0 + kTile);
  const bool res = J.kind == JOB_RESIDUAL;
  const double hi = J.rho * (1.0 + kRhoBand), lo = J.rho * (1.0 - kRhoBand);
  __shared__ int s_n;
  __shared__ int s_amb[64];
  __shared__ double red[kTPB / 64];
  if (tid == 0) s_n = 0;
  __syncthreads();
  double zt = 0.0, zd = 0.0, dp = 0.0, bp = 0.0;
  for (int j = j0 + tid; j < j1; j += kTPB) {
    double et = emass<DT>(tgt, J.trow, V, j, J.mt, J.c64);
    zt += et;
    if (res) {
      double ed = emass<DT>(dft, J.drow, V, j, J.md, J.c64);
      zd += ed;
      if (et > hi * ed) {
        dp += et - J.rho * ed;
        bp += ed;
      } else if (et > 0.0 && et >= lo * ed) {
        int slot = atomicAdd(&s_n, 1);
        if (slot < 64) s_amb[slot] = j;
      }
    }
  }
  zt = block_sum(zt, red);
  if (res) {
    zd = block_sum(zd, red);
    dp = block_sum(dp, red);
    bp = block_sum(bp, red);
  }
  __syncthreads();
  if (tid == 0) {
    TileRec R;
    R.zt = zt; R.zd = zd; R.dpos = dp; R.bpos = bp;
    int n = s_n, kept = min(n, 64);
    // ascending order of the listed indices (insertion sort, at most 64)
    for (int a = 1; a < kept; ++a) {
      int x = s_amb[a], c = a - 1;
      while (c >= 0 && s_amb[c] > x) { s_amb[c + 1] = s_amb[c]; --c; }
      s_amb[c + 1] = x;
    }
    R.namb = n;
    for (int a = 0; a < kAmbMax; ++a) R.amb[a] = a < kept ? s_amb[a] : -1;
    recs[(long long)b * ntile + k] = R;
  }
}

// Residual (or bonus) mass of one token with exact rho.
template <int DT>
__device__ __forceinline__ double qmass(const void* tgt, const void* dft, const SampleJob& J, bool res, double rho,
                                        int V, int j) {
  double et = emass<DT>(tgt, J.trow, V, j, J.mt, J.c64);
  if (!res) return et;
  double ed = emass<DT>(dft, J.drow, V, j, J.md, J.c64);
  double q = et - rho * ed;
  return q > 0.0 ? q : 0.0;
}

template <int DT>
__global__ __launch_bounds__(kTPB) void k_sample_pick(const void* __restrict__ tgt, const void* __restrict__ dft,
                                                      int V, int ntile, const SampleJob* __restrict__ jobs,
                                                      TileRec* __restrict__ recs, int32_t* __restrict__ out,
                                                      int out_width) {
  const int b = blockIdx.x, tid = threadIdx.x;
  const SampleJob J = jobs[b];
  if (J.kind == JOB_NONE) return;
  TileRec* R = recs + (long long)b * ntile;
  __shared__ double red[kTPB / 64];
  __shared__ double s_rho, s_W, s_thr;
  __shared__ int s_exact_all, s_tile, s_last, s_res;
  __shared__ double s_scan[kTPB];
  __shared__ int s_pick;

  if (tid == 0) {
    double Zt = 0.0, Zd = 0.0;
    for (int k = 0; k < ntile; ++k) { Zt += R[k].zt; Zd += R[k].zd; }
    bool res = J.kind == JOB_RESIDUAL;
    double rho = res ? Zt / Zd : 0.0;
    s_rho = rho;
    s_res = res;
    // the band test: every token outside the band has the same residual sign under rho and rho~
    s_exact_all = res && !(fabs(rho - J.rho) <= 0.5 * kRhoBand * J.rho);
  }
  __syncthreads();
  bool res = s_res != 0;
  const double rho = s_rho;
  __syncthreads();  // every thread has read s_res before thread 0 may rewrite it

  // tiles whose mass must be recomputed exactly (band failure or too many listed tokens)
  if (res) {
    for (int k = 0; k < ntile; ++k) {
      if (!(s_exact_all || R[k].namb > kAmbMax)) continue;
      const int j0 = k * kTile, j1 = min(V, j0 + kTile);
      double acc = 0.0;
      for (int j = j0 + tid; j < j1; j += kTPB) acc += qmass<DT>(tgt, dft, J, true, rho, V, j);
      acc = block_sum(acc, red);
      if (tid == 0) {
        R[k].dpos = acc; R[k].bpos = 0.0; R[k].namb = 0;
        for (int a = 0; a < kAmbMax; ++a) R[k].amb[a] = -1;
      }
      __syncthreads();
    }
  }

  if (tid == 0) {
    // tile masses, total, and the tile holding u S
    auto tile_mass = [&](int k, bool r) -> double {
      if (!r) return R[k].zt;
      double t = R[k].dpos + (J.rho - rho) * R[k].bpos;
      for (int a = 0; a < R[k].namb && a < kAmbMax; ++a) t += qmass<DT>(tgt, dft, J, true, rho, V, R[k].amb[a]);
      return t > 0.0 ? t : 0.0;
    };
    double S = 0.0;
    for (int k = 0; k < ntile; ++k) S += tile_mass(k, res);
    if (!(S > 0.0) && res) {  // residual underflow: draw from p_t of the same row
      res = false;
      S = 0.0;
      for (int k = 0; k < ntile; ++k) S += tile_mass(k, false);
    }
    const double thr = (double)J.u * S;
    double W = 0.0;
    int tile = -1, last_pos = -1;
    for (int k = 0; k < ntile; ++k) {
      double t = tile_mass(k, res);
      if (t > 0.0) last_pos = k;
      if (tile < 0 && W + t > thr) { tile = k; break; }
      W += t;
    }
    s_last = tile < 0;
    if (tile < 0) {  // rounding left no tile above u S: take the last token with positive mass
      tile = last_pos;
      W = 0.0;
    }
    s_tile = tile;
    s_W = W;
    s_thr = thr;
    s_res = res;
    s_pick = 0x7fffffff;
  }
  __syncthreads();
  res = s_res != 0;
  const int tile = s_tile;
  if (tile < 0) {  // no positive mass anywhere (cannot happen for usable rows)
    if (tid == 0) out[(long long)b * out_width + J.pos] = -1;
    return;
  }
  // fp64 inclusive scan of the tile, kTile / kTPB contiguous tokens per thread
  constexpr int PER = kTile / kTPB;
  const int j0 = tile * kTile + tid * PER;
  const int jend = min(V, tile * kTile + kTile);
  double q[PER];
  double local = 0.0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    int j = j0 + i;
    q[i] = j < jend ? qmass<DT>(tgt, dft, J, res, rho, V, j) : 0.0;
    local += q[i];
  }
  // exclusive scan of thread totals
  s_scan[tid] = local;
  __syncthreads();
  for (int off = 1; off < kTPB; off <<= 1) {
    double add = tid >= off ? s_scan[tid - off] : 0.0;
    __syncthreads();
    s_scan[tid] += add;
    __syncthreads();
  }
  const double excl = s_scan[tid] - local;
  const double thr = s_thr;
  const bool last_mode = s_last != 0;
  int pick = 0x7fffffff, lastpos = -1;
  double run = s_W + excl;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    run += q[i];
    if (q[i] > 0.0) {
      lastpos = j0 + i;
      if (!last_mode && run > thr && pick == 0x7fffffff) pick = j0 + i;
    }
  }
  if (pick != 0x7fffffff) atomicMin(&s_pick, pick);
  __syncthreads();
  int y = s_pick;
  if (y == 0x7fffffff) {  // no token passed u S in this tile (rounding): last positive token
    __shared__ int s_lastpos;
    if (tid == 0) s_lastpos = -1;
    __syncthreads();
    if (lastpos >= 0) atomicMax(&s_lastpos, lastpos);
    __syncthreads();
    y = s_lastpos;
  }
  if (tid == 0) out[(long long)b * out_width + J.pos] = y;
}

hipError_t launch_sample(int dt, const void* tgt, const void* dft, int V, int B, const SampleJob* jobs,
                         TileRec* recs, int32_t* out, int out_width, hipStream_t st) {
  if (B == 0) return hipSuccess;
  const int ntile = (V + kTile - 1) / kTile;
  const long long grid = (long long)B * ntile;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  if (dt == 1) {
    hipLaunchKernelGGL(k_sample_tiles<1>, dim3((unsigned)grid), dim3(kTPB), 0, st, tgt, dft, V, ntile, jobs, recs);
    hipLaunchKernelGGL(k_sample_pick<1>, dim3(B), dim3(kTPB), 0, st, tgt, dft, V, ntile, jobs, recs, out, out_width);
  } else {
    hipLaunchKernelGGL(k_sample_tiles<0>, dim3((unsigned)grid), dim3(kTPB), 0, st, tgt, dft, V, ntile, jobs, recs);
    hipLaunchKernelGGL(k_sample_pick<0>, dim3(B), dim3(kTPB), 0, st, tgt, dft, V, ntile, jobs, recs, out, out_width);
  }
  return hipGetLastError();
}

}  // namespace sv
