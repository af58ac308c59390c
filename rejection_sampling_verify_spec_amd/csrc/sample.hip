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
// Two kernels (a kernel boundary is the cheapest cross-workgroup hand-off on
// this multi-die part; device-scope fences cost an L2 write-back each):
//   k_sample_tiles (one wave per tile of kSTile tokens): Z_t and Z_d of the
//   tile and -- with the estimate rho~ of the fp32 row statistics -- the sums
//   over tokens with e_t > rho~(1+band) e_d of (e_t - rho~ e_d) and of e_d;
//   tokens inside the band (the only ones whose residual sign the estimate
//   cannot decide) are summed in groups of equal logit difference l_t - l_d,
//   which share one likelihood ratio.
//   k_sample_pick (one workgroup per job): exact rho = Z_t / Z_d, exact tile
//   masses dpos + (rho~ - rho) bpos + sum over groups of
//   max(0, sum e_t - rho sum e_d) (tiles whose groups did not fit, or every
//   tile when rho leaves the band, are recomputed token by token), a prefix
//   scan over tiles for the one holding u S, and a fp64 prefix scan of that
//   tile.
#include "sv_internal.h"

namespace sv {

constexpr int kSE = kSTile / kTPB;    // tokens per thread when a workgroup scans one tile
constexpr int kWE = kSTile / 64;      // tokens per lane when a wave owns a tile
constexpr int kTilesPerWG = kTPB / 64;
constexpr int kList = 64;             // undecided tokens collected per tile

// Fixed-order workgroup sum of doubles (same result in every thread).
__device__ __forceinline__ double block_sum(double v, double* red) {
  v = wave_reduce(v, [](double a, double b) { return a + b; });
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double t = red[0];
  for (int w = 1; w < kTPB / 64; ++w) t += red[w];
  __syncthreads();
  return t;
}

// A workgroup's view of one tile: tokens j = j0 + u*kTPB + tid (u < kSE); out of range -> -inf.
template <int DT>
__device__ __forceinline__ void load_tile(const void* base, long long row, int V, int j0, float* x) {
  const int tid = threadIdx.x;
  const long long off = row * (long long)V;
#pragma unroll
  for (int u = 0; u < kSE; ++u) {
    int j = j0 + u * kTPB + tid;
    x[u] = j < V ? Elem<DT>::at(base, off + j) : -INFINITY;
  }
}

// Per-wave list of undecided tokens of the tile pass (in a fixed order).
struct TileLists {
  double dl[kTilesPerWG][kList], et[kTilesPerWG][kList], ed[kTilesPerWG][kList];
};

// A wave's view of one tile: lane l holds tokens j0 + (u*64 + l)*epv + e (u < kWE/epv, e < epv),
// read with 16-byte loads when the row is 16-byte aligned, token by token otherwise.
template <int DT>
__device__ __forceinline__ void load_tile_wave(const void* rowp, bool vec_ok, int j0, int V, int lane, float* x) {
  using E = Elem<DT>;
  constexpr int epv = E::kPerVec;
  constexpr int nv = kWE / epv;
  if (vec_ok) {
    const uint4* vp = reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(rowp) +
                                                     (size_t)j0 * sizeof(typename E::T));
#pragma unroll
    for (int u = 0; u < nv; ++u) {
      const int v = u * 64 + lane;
      const int jv = j0 + v * epv;
      if (jv + epv <= V) {
        unpack<DT>(vp[v], x + u * epv);
      } else {
#pragma unroll
        for (int e = 0; e < epv; ++e) x[u * epv + e] = jv + e < V ? E::at(rowp, jv + e) : -INFINITY;
      }
    }
  } else {
#pragma unroll
    for (int u = 0; u < nv; ++u)
#pragma unroll
      for (int e = 0; e < epv; ++e) {
        const int j = j0 + (u * 64 + lane) * epv + e;
        x[u * epv + e] = j < V ? E::at(rowp, j) : -INFINITY;
      }
  }
}

// One wave owns tile k; writes the tile record. Undecided tokens are appended in a fixed
// order (element slot, then lane) through wave ballots.
template <int DT>
__device__ void tile_pass(const void* tgt, const void* dft, int V, const SampleJob& J, int k, TileRec* rec,
                          TileLists& L, int wv, int lane) {
  using E = Elem<DT>;
  const bool res = J.kind == JOB_RESIDUAL;
  const int j0 = k * kSTile;
  const double hi = J.rho * (1.0 + kRhoBand), lo = J.rho * (1.0 - kRhoBand);
  const void* trow = reinterpret_cast<const char*>(tgt) + (size_t)J.trow * (size_t)V * sizeof(typename E::T);
  const void* drow = reinterpret_cast<const char*>(dft) + (size_t)J.drow * (size_t)V * sizeof(typename E::T);
  const bool t_al = (reinterpret_cast<uintptr_t>(trow) & 15u) == 0;
  const bool d_al = (reinterpret_cast<uintptr_t>(drow) & 15u) == 0;
  const unsigned long long below = (1ull << lane) - 1ull;
  float xt[kWE], xd[kWE];
  load_tile_wave<DT>(trow, t_al, j0, V, lane, xt);
  if (res) load_tile_wave<DT>(drow, d_al, j0, V, lane, xd);
  double zt = 0.0, zd = 0.0, dp = 0.0, bp = 0.0;
  int n = 0;  // undecided tokens seen (wave-uniform)
#pragma unroll
  for (int i = 0; i < kWE; ++i) {
    const double et = emass(xt[i], J.mt, J.c64);
    zt += et;
    if (res) {
      const double ed = emass(xd[i], J.md, J.c64);
      zd += ed;
      bool und = false;
      if (et > hi * ed) {
        dp += et - J.rho * ed;
        bp += ed;
      } else {
        und = et > 0.0 && et >= lo * ed;
      }
      const unsigned long long m = __ballot(und);
      if (m) {
        const int slot = n + __builtin_popcountll(m & below);
        if (und && slot < kList) {
          L.dl[wv][slot] = (double)xt[i] - (double)xd[i];
          L.et[wv][slot] = et;
          L.ed[wv][slot] = ed;
        }
        n += __builtin_popcountll(m);
      }
    }
  }
  auto add = [](double a, double b) { return a + b; };
  zt = wave_reduce(zt, add);
  int ng = 0;
  double gt = 0.0, gd = 0.0;  // lane g < ng holds group g's sums
  if (res) {
    zd = wave_reduce(zd, add);
    dp = wave_reduce(dp, add);
    bp = wave_reduce(bp, add);
    if (n > kList) {
      ng = -1;
    } else if (n > 0) {
      // the wave's list entries are complete before lanes read them
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
      __builtin_amdgcn_wave_barrier();
      const bool have = lane < n;
      const double key = have ? L.dl[wv][lane] : 0.0;
      const double my_et = have ? L.et[wv][lane] : 0.0, my_ed = have ? L.ed[wv][lane] : 0.0;
      // first list entry with the same logit difference
      int first = lane;
      for (int e = 0; e < n; ++e) {
        const double ke = __shfl(key, e, 64);
        if (e < first && ke == key) first = e;
      }
      const unsigned long long leaders = __ballot(have && first == lane);
      ng = __builtin_popcountll(leaders);
      const int grp = __builtin_popcountll(leaders & ((1ull << first) - 1ull));
      if (ng > kGrp) {
        ng = -1;
      } else {
        // group sums in list order: lane g accumulates the entries of group g
        for (int e = 0; e < n; ++e) {
          const int ge = __shfl(grp, e, 64);
          const double te = __shfl(my_et, e, 64), de = __shfl(my_ed, e, 64);
          if (lane == ge) { gt += te; gd += de; }
        }
      }
    }
  }
  // lanes 0..kGrp-1 hold the group sums; lane 0 writes the scalar fields
  if (lane < kGrp) {
    rec->get[lane] = ng > lane ? gt : 0.0;
    rec->ged[lane] = ng > lane ? gd : 0.0;
  }
  if (lane == 0) {
    rec->zt = zt;
    rec->zd = zd;
    rec->dpos = dp;
    rec->bpos = bp;
    rec->ngrp = ng;
    rec->pad = 0;
    rec->pad2 = 0.0;
  }
}

template <int DT>
__global__ __launch_bounds__(kTPB) void k_sample_tiles(const void* __restrict__ tgt, const void* __restrict__ dft,
                                                       int V, int ntile, int wg_per_job,
                                                       const SampleJob* __restrict__ jobs,
                                                       TileRec* __restrict__ recs) {
  const int b = blockIdx.x / wg_per_job, g = blockIdx.x - b * wg_per_job;
  const SampleJob J = jobs[b];
  if (J.kind == JOB_NONE) return;
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  __shared__ TileLists lists;
  const int k = g * kTilesPerWG + wv;
  if (k < ntile) tile_pass<DT>(tgt, dft, V, J, k, recs + (long long)b * ntile + k, lists, wv, lane);
}

struct PickSpace {
  double red[kTPB / 64];
  double sq[kSTile];
  double Zt, Zd, W, thr, S;
  int tile, last_mode, any_exact, res;
  int smin[kTPB / 64], smax[kTPB / 64];
};

// Inclusive prefix sum over the 64 lanes of a wave (fixed order).
__device__ __forceinline__ double wave_incl_scan(double v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double o = __shfl_up(v, off, 64);
    if (lane >= off) v += o;
  }
  return v;
}

template <int DT>
__device__ void pick(const void* tgt, const void* dft, int V, int ntile, const SampleJob& J, TileRec* R,
                     int32_t* dst, int force_exact, PickSpace& P) {
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  auto add = [](double a, double b) { return a + b; };
  // --- exact normalisers: wave 0, lanes over tiles, fixed-order sums
  if (wv == 0) {
    double zt = 0.0, zd = 0.0;
    int need = 0;
    for (int k = lane; k < ntile; k += 64) {
      zt += R[k].zt;
      zd += R[k].zd;
      need |= R[k].ngrp < 0;
    }
    zt = wave_reduce(zt, add);
    zd = wave_reduce(zd, add);
    need = __any(need);
    if (lane == 0) {
      const bool res = J.kind == JOB_RESIDUAL;
      const double rho = res ? zt / zd : 0.0;
      P.Zt = zt;
      P.Zd = zd;
      P.res = res;
      // every token outside the band has the same residual sign under rho and rho~
      const bool exact_all = res && (force_exact || !(fabs(rho - J.rho) <= 0.5 * kRhoBand * J.rho));
      P.any_exact = res && (exact_all || need) ? (exact_all ? 2 : 1) : 0;
    }
  }
  __syncthreads();
  bool res = P.res != 0;
  const double rho = res ? P.Zt / P.Zd : 0.0;

  // --- tiles whose residual mass is recomputed token by token (marked ngrp = -2, mass in zd)
  if (P.any_exact) {
    const bool all = P.any_exact == 2;
    for (int k = 0; k < ntile; ++k) {
      if (!(all || R[k].ngrp < 0)) continue;
      float xt[kSE], xd[kSE];
      load_tile<DT>(tgt, J.trow, V, k * kSTile, xt);
      load_tile<DT>(dft, J.drow, V, k * kSTile, xd);
      double acc = 0.0;
#pragma unroll
      for (int u = 0; u < kSE; ++u) {
        const double q = emass(xt[u], J.mt, J.c64) - rho * emass(xd[u], J.md, J.c64);
        acc += q > 0.0 ? q : 0.0;
      }
      acc = block_sum(acc, P.red);
      if (tid == 0) {
        R[k].zd = acc;
        R[k].ngrp = -2;
      }
      __syncthreads();
    }
  }

  // --- tile masses, total S, and the first tile whose inclusive prefix exceeds u S (wave 0)
  auto tile_mass = [&](int k, bool r) -> double {
    if (!r) return R[k].zt;
    const int ng = R[k].ngrp;
    if (ng == -2) return R[k].zd;
    double t = R[k].dpos + (J.rho - rho) * R[k].bpos;
    for (int g = 0; g < ng; ++g) {
      const double q = R[k].get[g] - rho * R[k].ged[g];
      t += q > 0.0 ? q : 0.0;
    }
    return t > 0.0 ? t : 0.0;
  };
  if (wv == 0) {
    double part = 0.0;
    for (int k = lane; k < ntile; k += 64) part += tile_mass(k, res);
    double S = wave_reduce(part, add);
    if (!(S > 0.0) && res) {  // residual underflow: draw from p_t of the same row
      res = false;
      part = 0.0;
      for (int k = lane; k < ntile; k += 64) part += tile_mass(k, false);
      S = wave_reduce(part, add);
    }
    const double thr = (double)J.u * S;
    double base = 0.0;
    int tile = -1, lastpos = -1;
    double W = 0.0;
    for (int k0 = 0; k0 < ntile; k0 += 64) {
      const int k = k0 + lane;
      const double t = k < ntile ? tile_mass(k, res) : 0.0;
      const double incl = wave_incl_scan(t, lane);
      const unsigned long long pos = __ballot(t > 0.0);
      if (pos) lastpos = k0 + 63 - __builtin_clzll(pos);
      const unsigned long long hit = __ballot(t > 0.0 && base + incl > thr);
      if (hit) {
        const int l = __builtin_ctzll(hit);
        tile = k0 + l;
        W = base + __shfl(incl - t, l, 64);
        break;
      }
      base += __shfl(incl, 63, 64);
    }
    if (lane == 0) {
      P.last_mode = tile < 0;  // rounding left no tile above u S: last token with positive mass
      P.tile = tile < 0 ? lastpos : tile;
      P.W = W;
      P.thr = thr;
      P.res = res;
    }
  }
  __syncthreads();
  res = P.res != 0;
  const int tile = P.tile;
  if (tile < 0) {  // no positive mass anywhere (cannot happen for usable rows)
    if (tid == 0) *dst = -1;
    return;
  }
  const bool last_mode = P.last_mode != 0;
  const double thr = P.thr, Wtile = P.W;

  // --- masses of the chosen tile into shared memory, then a contiguous scan per thread
  {
    float xt[kSE], xd[kSE];
    load_tile<DT>(tgt, J.trow, V, tile * kSTile, xt);
    if (res) load_tile<DT>(dft, J.drow, V, tile * kSTile, xd);
#pragma unroll
    for (int u = 0; u < kSE; ++u) {
      double q = emass(xt[u], J.mt, J.c64);
      if (res) {
        q -= rho * emass(xd[u], J.md, J.c64);
        q = q > 0.0 ? q : 0.0;
      }
      P.sq[u * kTPB + tid] = q;
    }
  }
  __syncthreads();
  double q[kSE];
  double local = 0.0;
#pragma unroll
  for (int i = 0; i < kSE; ++i) {
    q[i] = P.sq[tid * kSE + i];
    local += q[i];
  }
  const double wincl = wave_incl_scan(local, lane);
  if (lane == 63) P.red[wv] = wincl;
  __syncthreads();
  double run = Wtile;
  for (int w = 0; w < wv; ++w) run += P.red[w];
  run += wincl - local;
  const int jt = tile * kSTile + tid * kSE;
  int pk = 0x7fffffff, lastpos = -1;
#pragma unroll
  for (int i = 0; i < kSE; ++i) {
    run += q[i];
    if (q[i] > 0.0) {
      lastpos = jt + i;
      if (!last_mode && run > thr && pk == 0x7fffffff) pk = jt + i;
    }
  }
  pk = wave_reduce(pk, [](int a, int b) { return a < b ? a : b; });
  lastpos = wave_reduce(lastpos, [](int a, int b) { return a > b ? a : b; });
  if (lane == 0) { P.smin[wv] = pk; P.smax[wv] = lastpos; }
  __syncthreads();
  if (tid == 0) {
    int y = 0x7fffffff, yl = -1;
    for (int w = 0; w < kTPB / 64; ++w) {
      y = min(y, P.smin[w]);
      yl = max(yl, P.smax[w]);
    }
    // no token passed u S in this tile (rounding at its end): the last positive token
    *dst = y != 0x7fffffff ? y : yl;
  }
}

template <int DT>
__global__ __launch_bounds__(kTPB) void k_sample_pick(const void* __restrict__ tgt, const void* __restrict__ dft,
                                                      int V, int ntile, const SampleJob* __restrict__ jobs,
                                                      TileRec* __restrict__ recs, int32_t* __restrict__ out,
                                                      int out_width, int force_exact) {
  const int b = blockIdx.x;
  const SampleJob J = jobs[b];
  if (J.kind == JOB_NONE) return;
  __shared__ PickSpace P;
  pick<DT>(tgt, dft, V, ntile, J, recs + (long long)b * ntile, out + (long long)b * out_width + J.pos, force_exact,
           P);
}

hipError_t launch_sample(int dt, const void* tgt, const void* dft, int V, int B, const SampleJob* jobs,
                         TileRec* recs, int32_t* out, int out_width, int force_exact, hipStream_t st) {
  if (B == 0) return hipSuccess;
  const int ntile = (V + kSTile - 1) / kSTile;
  const int wg_per_job = (ntile + kTilesPerWG - 1) / kTilesPerWG;
  const long long grid = (long long)B * wg_per_job;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  if (dt == 1) {
    hipLaunchKernelGGL(k_sample_tiles<1>, dim3((unsigned)grid), dim3(kTPB), 0, st, tgt, dft, V, ntile, wg_per_job,
                       jobs, recs);
    hipLaunchKernelGGL(k_sample_pick<1>, dim3(B), dim3(kTPB), 0, st, tgt, dft, V, ntile, jobs, recs, out,
                       out_width, force_exact);
  } else {
    hipLaunchKernelGGL(k_sample_tiles<0>, dim3((unsigned)grid), dim3(kTPB), 0, st, tgt, dft, V, ntile, wg_per_job,
                       jobs, recs);
    hipLaunchKernelGGL(k_sample_pick<0>, dim3(B), dim3(kTPB), 0, st, tgt, dft, V, ntile, jobs, recs, out,
                       out_width, force_exact);
  }
  return hipGetLastError();
}

}  // namespace sv
