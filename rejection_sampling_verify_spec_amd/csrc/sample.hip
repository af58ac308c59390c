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
// Two kernels, after an accept kernel has written one job per request:
//   k_sample_tiles (one workgroup per slice of a request's tiles; each wave
//   owns one tile of kSTile tokens at a time): per tile Z_t and Z_d and, with the estimate
//   rho~ of the fp32 row statistics, the sums over tokens with
//   e_t > rho~(1+band) e_d of (e_t - rho~ e_d) and of e_d; tokens inside the
//   band (the only ones whose residual sign the estimate cannot decide) are
//   summed in groups of equal logit difference l_t - l_d, which share one
//   likelihood ratio.
//   k_sample_pick (one workgroup per job): exact rho = Z_t / Z_d, exact tile
//   masses dpos + (rho~ - rho) bpos + sum over groups of
//   max(0, sum e_t - rho sum e_d) (tiles whose groups did not fit, or every
//   tile when rho leaves the band, are recomputed token by token), a prefix
//   scan over tiles for the one holding u S, and a fp64 prefix scan of that
//   tile.
#include "sv_internal.h"

namespace sv {

constexpr int kEPL = kSTile / 64;     // tokens per lane when a wave owns a tile
constexpr int kEPT = kSTile / kTPB;   // tokens per thread when a workgroup owns a tile
constexpr int kWaves = kTPB / 64;
constexpr int kList = 64;             // undecided tokens collected per tile

static_assert(kEPT == 8, "a workgroup tile gives each thread 8 contiguous tokens");

// Raw bits of one logit and of -inf, per storage type.
template <int DT> __device__ __forceinline__ uint32_t raw_at(const void* rowp, int j);
template <> __device__ __forceinline__ uint32_t raw_at<0>(const void* rowp, int j) {
  return reinterpret_cast<const uint32_t*>(rowp)[j];
}
template <> __device__ __forceinline__ uint32_t raw_at<1>(const void* rowp, int j) {
  return reinterpret_cast<const uint16_t*>(rowp)[j];
}
template <int DT> struct NegInf;
template <> struct NegInf<0> { static constexpr uint32_t bits = 0xff800000u; };
template <> struct NegInf<1> { static constexpr uint32_t bits = 0xff80u; };

// n consecutive tokens starting at j as packed 16-byte vectors (element order of
// unpack<DT>); tokens at or beyond V read as -inf. Vector loads when the whole
// span is in range and 16-byte aligned, token by token otherwise.
template <int DT, int NV>
__device__ __forceinline__ void load_span(const void* rowp, int j, int V, uint4* w) {
  constexpr int epv = Elem<DT>::kPerVec;
  constexpr int es = sizeof(typename Elem<DT>::T);
  const char* p = reinterpret_cast<const char*>(rowp) + (size_t)j * es;
  if (j + NV * epv <= V && (reinterpret_cast<uintptr_t>(p) & 15u) == 0) {
#pragma unroll
    for (int u = 0; u < NV; ++u) w[u] = reinterpret_cast<const uint4*>(p)[u];
  } else {
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      uint32_t b[epv];
#pragma unroll
      for (int e = 0; e < epv; ++e) {
        const int jj = j + u * epv + e;
        b[e] = jj < V ? raw_at<DT>(rowp, jj) : NegInf<DT>::bits;
      }
      if constexpr (DT == 1) {
        w[u] = make_uint4(b[0] | (b[1] << 16), b[2] | (b[3] << 16), b[4] | (b[5] << 16), b[6] | (b[7] << 16));
      } else {
        w[u] = make_uint4(b[0], b[1], b[2], b[3]);
      }
    }
  }
}

// A wave's tile: lane l holds vectors u*64 + l (u < NV) of the tile, i.e. tokens
// j0 + (u*64 + l)*epv + e.
template <int DT>
__device__ __forceinline__ void load_tile_wave(const void* rowp, int j0, int V, int lane,
                                               uint4 (&w)[kEPL / Elem<DT>::kPerVec]) {
  constexpr int epv = Elem<DT>::kPerVec;
  constexpr int nv = kEPL / epv;
  constexpr int es = sizeof(typename Elem<DT>::T);
  const char* p = reinterpret_cast<const char*>(rowp) + (size_t)j0 * es;
  if (j0 + kSTile <= V && (reinterpret_cast<uintptr_t>(p) & 15u) == 0) {
#pragma unroll
    for (int u = 0; u < nv; ++u) w[u] = reinterpret_cast<const uint4*>(p)[u * 64 + lane];
  } else {
#pragma unroll
    for (int u = 0; u < nv; ++u) load_span<DT, 1>(rowp, j0 + (u * 64 + lane) * epv, V, &w[u]);
  }
}

// Per-wave list of undecided tokens of the tile pass (in a fixed order).
struct TileLists {
  double dl[kWaves][kList], et[kWaves][kList], ed[kWaves][kList];
};

// One wave's pass over one tile; writes the tile record. Undecided tokens are
// appended in a fixed order (element slot, then lane) through wave ballots.
template <int DT, bool RES>
__device__ __forceinline__ void tile_pass(const uint4* wt, const uint4* wd, const SampleJob& J, TileRec* rec,
                                          TileLists& L, int wv, int lane) {
  constexpr int epv = Elem<DT>::kPerVec;
  constexpr int nv = kEPL / epv;
  const double hi = J.rho * (1.0 + kRhoBand), lo = J.rho * (1.0 - kRhoBand);
  const unsigned long long below = (1ull << lane) - 1ull;
  double zt = 0.0, zd = 0.0, dp = 0.0, bp = 0.0;
  int n = 0;  // undecided tokens seen (wave-uniform)
#pragma unroll
  for (int u = 0; u < nv; ++u) {
    float xt[epv], xd[epv];
    unpack<DT>(wt[u], xt);
    if (RES) unpack<DT>(wd[u], xd);
#pragma unroll
    for (int e = 0; e < epv; ++e) {
      const double et = emass(xt[e], J.mt, J.c64, J.c32);
      zt += et;
      if (RES) {
        const double ed = emass(xd[e], J.md, J.c64, J.c32);
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
            L.dl[wv][slot] = (double)xt[e] - (double)xd[e];
            L.et[wv][slot] = et;
            L.ed[wv][slot] = ed;
          }
          n += __builtin_popcountll(m);
        }
      }
    }
  }
  auto add = [](double a, double b) { return a + b; };
  zt = wave_reduce(zt, add);
  int ng = 0;
  double gt = 0.0, gd = 0.0;  // lane g < ng holds group g's sums
  if (RES) {
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
      // the lists are reused by the wave's next tile
      __builtin_amdgcn_wave_barrier();
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

// Workgroup (b, g) of G per request: tiles g*kWaves + wv + i*G*kWaves of job b.
template <int DT>
__global__ __launch_bounds__(kTPB) void k_sample_tiles(const void* __restrict__ tgt, const void* __restrict__ dft,
                                                       int V, int ntile, int G, const SampleJob* __restrict__ jobs,
                                                       TileRec* __restrict__ recs) {
  const int b = blockIdx.x / G, g = blockIdx.x - b * G;
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  __shared__ TileLists lists;
  const SampleJob J = jobs[b];
  if (J.kind == JOB_NONE) return;
  constexpr int epv = Elem<DT>::kPerVec;
  constexpr int es = sizeof(typename Elem<DT>::T);
  const char* trow = reinterpret_cast<const char*>(tgt) + (size_t)J.trow * (size_t)V * es;
  const char* drow = reinterpret_cast<const char*>(dft) + (size_t)J.drow * (size_t)V * es;
  TileRec* R = recs + (long long)b * ntile;
  for (int k = g * kWaves + wv; k < ntile; k += G * kWaves) {
    uint4 wt[kEPL / epv];
    load_tile_wave<DT>(trow, k * kSTile, V, lane, wt);
    if (J.kind == JOB_RESIDUAL) {
      uint4 wd[kEPL / epv];
      load_tile_wave<DT>(drow, k * kSTile, V, lane, wd);
      tile_pass<DT, true>(wt, wd, J, R + k, lists, wv, lane);
    } else {
      tile_pass<DT, false>(wt, wt, J, R + k, lists, wv, lane);
    }
  }
}

// ---------------------------------------------------------------------------
// Pick.

struct PickSpace {
  double red[kWaves];
  double Zt, Zd, W, thr;
  int tile, last_mode, any_exact, res;
  int smin[kWaves], smax[kWaves];
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

// Fixed-order workgroup sum of doubles (same result in every thread).
__device__ __forceinline__ double block_sum(double v, double* red) {
  v = wave_reduce(v, [](double a, double b) { return a + b; });
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double t = red[0];
  for (int w = 1; w < kWaves; ++w) t += red[w];
  __syncthreads();
  return t;
}

// A workgroup's tile: thread tid holds the 8 contiguous tokens j0 + 8 tid + i.
template <int DT>
__device__ __forceinline__ void load_tile_block(const void* rowp, int j0, int V, int tid, float* x) {
  constexpr int epv = Elem<DT>::kPerVec;
  uint4 w[kEPT / epv];
  load_span<DT, kEPT / epv>(rowp, j0 + tid * kEPT, V, w);
#pragma unroll
  for (int u = 0; u < kEPT / epv; ++u) unpack<DT>(w[u], x + u * epv);
}

template <int DT>
__device__ void pick(const void* tgt, const void* dft, int V, int ntile, const SampleJob& J, TileRec* R,
                     int32_t* dst, int force_exact, PickSpace& P) {
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  constexpr int es = sizeof(typename Elem<DT>::T);
  const char* trow = reinterpret_cast<const char*>(tgt) + (size_t)J.trow * (size_t)V * es;
  const char* drow = reinterpret_cast<const char*>(dft) + (size_t)J.drow * (size_t)V * es;
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
      float xt[kEPT], xd[kEPT];
      load_tile_block<DT>(trow, k * kSTile, V, tid, xt);
      load_tile_block<DT>(drow, k * kSTile, V, tid, xd);
      double acc = 0.0;
#pragma unroll
      for (int i = 0; i < kEPT; ++i) {
        const double q = emass(xt[i], J.mt, J.c64, J.c32) - rho * emass(xd[i], J.md, J.c64, J.c32);
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

  // --- masses of the chosen tile (8 contiguous tokens per thread), then a fixed-order scan
  double q[kEPT];
  double local = 0.0;
  {
    float xt[kEPT], xd[kEPT];
    load_tile_block<DT>(trow, tile * kSTile, V, tid, xt);
    if (res) load_tile_block<DT>(drow, tile * kSTile, V, tid, xd);
#pragma unroll
    for (int i = 0; i < kEPT; ++i) {
      double v = emass(xt[i], J.mt, J.c64, J.c32);
      if (res) {
        v -= rho * emass(xd[i], J.md, J.c64, J.c32);
        v = v > 0.0 ? v : 0.0;
      }
      q[i] = v;
      local += v;
    }
  }
  const double wincl = wave_incl_scan(local, lane);
  if (lane == 63) P.red[wv] = wincl;
  __syncthreads();
  double run = Wtile;
  for (int w = 0; w < wv; ++w) run += P.red[w];
  run += wincl - local;
  const int jt = tile * kSTile + tid * kEPT;
  int pk = 0x7fffffff, lastpos = -1;
#pragma unroll
  for (int i = 0; i < kEPT; ++i) {
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
    for (int w = 0; w < kWaves; ++w) {
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

// ---------------------------------------------------------------------------
// Launchers.

int sample_tiles(int V) { return (V + kSTile - 1) / kSTile; }

// Workgroups per request in the tiles kernel: enough for about four resident
// workgroups per compute unit over the batch, at most one per kWaves tiles.
static int tiles_groups(int B, int ntile) {
  constexpr int kTargetWG = 4 * 256;
  const int maxg = (ntile + kWaves - 1) / kWaves;
  int G = (kTargetWG + B - 1) / B;
  return G < 1 ? 1 : (G > maxg ? maxg : G);
}

template <int DT>
static hipError_t launch_tail(const void* tgt, const void* dft, int V, int B, SampleJob* jobs, TileRec* recs,
                              int32_t* out, int out_width, int force_exact, hipStream_t st) {
  const int ntile = sample_tiles(V);
  const int G = tiles_groups(B, ntile);
  const long long grid = (long long)B * G;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_sample_tiles<DT>, dim3((unsigned)grid), dim3(kTPB), 0, st, tgt, dft, V, ntile, G, jobs, recs);
  hipLaunchKernelGGL(k_sample_pick<DT>, dim3(B), dim3(kTPB), 0, st, tgt, dft, V, ntile, jobs, recs, out, out_width,
                     force_exact);
  return hipGetLastError();
}

hipError_t launch_sample_jobs(int dt, const void* tgt, const void* dft, int V, int B, SampleJob* jobs,
                              TileRec* recs, int32_t* out, int out_width, int force_exact, hipStream_t st) {
  if (B == 0) return hipSuccess;
  return dt == 1 ? launch_tail<1>(tgt, dft, V, B, jobs, recs, out, out_width, force_exact, st)
                 : launch_tail<0>(tgt, dft, V, B, jobs, recs, out, out_width, force_exact, st);
}

}  // namespace sv
