// finish.hip -- the tail of a verify call after the streaming pass: the
// acceptance scan and the draw of each request's final token.
//
//   k_accept_chain (one workgroup per request): the acceptance scan of chain
//   layouts; writes the accepted tokens, num_accepted, the diagnostics and the
//   request's sampling job (token trees get theirs from the tree accept kernel).
//   k_tiles (G workgroups per request): the tile pass over the drawn row(s).
//   k_pick (one workgroup per request): the inverse-CDF search over the tile
//   records.
//
// Acceptance [Primer 考点2 / 第二章]: drafted token x_i is accepted when
// u_accept[i] * p_d,i(x_i) < p_t,i(x_i), i.e. with probability
// min(1, p_t/p_d); the first rejected position n ends the scan. Greedy
// requests (T == 0) accept while x_i equals the target argmax (lowest index on
// ties) and emit the argmax at n. p(x) = 2^{(l_x - m) c} / Z, with the row
// statistics merged here in fp64 from the chunk partials of the streaming pass.
//
// Draw [Primer 考点2 residual P' = max(0, p_t - p_d) / sum; 考点4 bonus token
// from p_t when every draft passes]: inverse CDF y = min{ j : C_j > u S } in
// ascending token order. Masses are double precision in units of each row's
// maximum: e_t(j) = 2^{(l_t,j - m_t) c}, e_d(j) = 2^{(l_d,j - m_d) c},
// c = log2(e)/T, and the residual in these units is
// q_j = max(0, e_t(j) - rho e_d(j)) with rho = Z_t / Z_d, so that the chosen
// token agrees with a double-precision sequential evaluation unless u S lies
// within ~1e-13 S of a CDF boundary.
//   tile pass (each wave owns tiles of kSTile tokens): an fp32 triage; tiles
//   whose masses are all negligible (below 2^-50 of the row maximum) and, for
//   a residual, whose likelihood ratios are all clear of the band around the
//   estimate rho~ (from the fp32 row statistics) are summed in fp32; the other
//   tiles take the exact pass on the same registers: fp64 masses, Z_t and Z_d,
//   the sums over tokens with e_t > rho~(1+band) e_d of (e_t - rho~ e_d) and of
//   e_d; tokens inside the band (the only ones whose residual sign the
//   estimate cannot decide) are summed in groups of equal logit difference
//   l_t - l_d, which share one likelihood ratio.
//   pick: exact rho = Z_t / Z_d, exact tile masses dpos + (rho~ - rho) bpos +
//   sum over groups of max(0, sum e_t - rho sum e_d) (tiles whose groups did
//   not fit, or every tile when rho leaves the band, are recomputed token by
//   token), a scan over tiles for the one holding u S, and a fixed-order fp64
//   scan of that tile.
#include "specverify.h"
#include "sv_internal.h"

namespace sv {

constexpr int kVT = 256;              // threads of a workgroup of either kernel
constexpr int kVW = kVT / 64;         // its waves
constexpr int kEPL = kSTile / 64;     // tokens per lane when a wave owns a tile
constexpr int kBT = kSTile / kVT;     // tokens per thread when a workgroup owns a tile
constexpr int kTPG = kVW;             // tiles per k_tiles workgroup (one per wave)
constexpr int kList = 64;             // undecided tokens collected per tile
constexpr int kMaxPos = SV_MAX_GAMMA + 1;
constexpr int kRowLanes = 8;          // lanes merging one row's chunk partials
constexpr int kRowGroups = kVT / kRowLanes;

static_assert(kBT * kVT == kSTile, "a workgroup tile splits evenly over the threads");

// ---------------------------------------------------------------------------
// Shared memory of a finishing workgroup.

struct TileLists {  // per-wave lists of undecided tokens of the exact pass
  double dl[kVW][kList], et[kVW][kList], ed[kVW][kList];
};

struct PickSpace {
  double red[kVW];
  double Zt, Zd, W, thr;
  int tile, last_mode, any_exact, res;
  int smin[kVW], smax[kVW];
};

struct AcceptSpace {
  // per position i <= g
  int x[kMaxPos];
  float ua[kMaxPos], us[kMaxPos], lt[kMaxPos], ld[kMaxPos], pt[kMaxPos], pd[kMaxPos];
  // per row: target rows 0..g, then draft rows 0..g-1
  double rz[2 * kMaxPos];
  float rm[2 * kMaxPos];
  int ridx[2 * kMaxPos];
  unsigned char rok[2 * kMaxPos];
};

struct VerifyShared {
  double exp2tab[64];  // 2^{j/64}
  AcceptSpace acc;
  TileLists lists;
  SampleJob job;
  int n, bad;
};

struct PickShared {
  double exp2tab[64];
  PickSpace pick;
  SampleJob job;
};

// ---------------------------------------------------------------------------
// Token masses of the draw.

// 2^a in double precision for a <= 0 (NaN propagates), with tab[j] = 2^{j/64}:
// a = n + j/64 + r with n an integer, 0 <= j < 64 and |r| <= 1/128 (r is exact:
// a and k/64 are within a factor of two of each other or r is the tiny rest),
// and 2^r = exp(r ln 2) by its Taylor series to degree 5 (truncation below
// 4e-17 relative). About 3 ulp in all.
__device__ __forceinline__ double exp2_tab(double a, const double* tab) {
  if (!(a >= -1100.0)) return (a != a) ? a : 0.0;
  const double k = __builtin_rint(a * 64.0);
  const double r = __builtin_fma(k, -0.015625, a);
  const int ki = (int)k;
  double p = 0x1.5d87fe78a6731p-10;  // ln2^5 / 5!
  p = __builtin_fma(p, r, 0x1.3b2ab6fba4e77p-7);  // ln2^4 / 4!
  p = __builtin_fma(p, r, 0x1.c6b08d704a0c0p-5);  // ln2^3 / 3!
  p = __builtin_fma(p, r, 0x1.ebfbdff82c58fp-3);  // ln2^2 / 2!
  p = __builtin_fma(p, r, 0x1.62e42fefa39efp-1);  // ln2
  p = __builtin_fma(p, r, 1.0);
  return __builtin_ldexp(tab[ki & 63] * p, ki >> 6);
}

// Mass 2^{(l - m) c} of one token in double precision (c64 = c, c32 = fl32(c)),
// in units of its row's maximum. Terms below 2^-50 of the row maximum (fp32
// argument a32 < kTinyExp) take the fp32 exponential unit: the argument's error
// (three fp32 roundings, about 2e-7 |a|) and the unit's ulp leave an absolute
// error below 2^-60 per token, under the rounding of the double-precision sums
// these terms enter.
__device__ __forceinline__ double emass_t(float l, float m, double c64, float c32, const double* tab) {
  const float a32 = (l - m) * c32;
  if (a32 < kTinyExp) return (double)exp2_f32(a32);
  return exp2_tab(((double)l - (double)m) * c64, tab);
}

// ---------------------------------------------------------------------------
// Acceptance scan of chain request b by the whole workgroup.

// Merge the chunk partials of one row by the kRowLanes lanes of a group (lane
// `sub` takes chunks sub, sub + kRowLanes, ...). The maximum keeps the lowest
// token index among equal values (chunks are in ascending token order); Z is
// the fixed-order sum of s_k 2^{(m_k - M) c}. Every lane of the group ends
// with the same values.
__device__ __forceinline__ void merge_row_group(const Partial* __restrict__ p, int nchunk, double c, bool greedy,
                                                int sub, float& M, int& idx, double& Z, bool& ok) {
  M = -INFINITY;
  idx = -1;
  bool nan = false;
  for (int k = sub; k < nchunk; k += kRowLanes) {
    const Partial q = p[k];
    nan |= q.s != q.s;
    if (q.m > M) { M = q.m; idx = q.idx; }
  }
#pragma unroll
  for (int off = 1; off < kRowLanes; off <<= 1) {
    const float M2 = __shfl_xor(M, off, 64);
    const int i2 = __shfl_xor(idx, off, 64);
    nan |= __shfl_xor((int)nan, off, 64) != 0;
    if (M2 > M || (M2 == M && (unsigned)i2 < (unsigned)idx)) { M = M2; idx = i2; }
  }
  ok = !nan && M > -INFINITY && M < INFINITY;
  Z = 0.0;
  if (greedy || !ok) return;
  for (int k = sub; k < nchunk; k += kRowLanes) {
    const Partial q = p[k];
    if (q.m > -INFINITY) Z += (double)q.s * exp2_f64(((double)q.m - (double)M) * c);
  }
#pragma unroll
  for (int off = 1; off < kRowLanes; off <<= 1) Z += __shfl_xor(Z, off, 64);
  ok = Z > 0.0 && Z < 1e308;
}

struct ChainArgs {
  Layout L;
  const int32_t* tokens;
  const float* ua;
  const float* us;
  const float* temperature;
  const Partial* part;
  int nchunk;
  int chunk_vecs;  // 16-byte vectors per chunk of the streaming pass
  int32_t* num_acc;
  float* diag;
};

// Writes the request's accepted tokens (and the greedy token), num_accepted and
// the diagnostics when `write` is set, and leaves the sampling job in S.job.
template <int DT>
__device__ void accept_chain(const void* __restrict__ tgt, const void* __restrict__ dft, int V, const ChainArgs& A,
                             int b, int32_t* __restrict__ orow, int out_width, bool write, VerifyShared& S) {
  const int tid = threadIdx.x;
  const Layout& L = A.L;
  AcceptSpace& P = S.acc;
  if (tid == 0) {
    S.n = 0x7fffffff;
    S.bad = 0;
  }
  // --- the request's rows
  bool layout_ok = true;
  int g;
  long long t0, d0;
  if (L.mode == LAYOUT_RAGGED) {
    const int32_t* cu = L.cu;
    bool ok = true;
    if (tid == 0) ok = cu[0] == 0 && cu[L.B] == L.total_draft;
    for (int k = tid; k < L.B; k += kVT) {
      const int lo = cu[k], hi = cu[k + 1];
      ok = ok && hi >= lo && hi - lo <= L.gamma;
    }
    layout_ok = __syncthreads_and(ok) != 0;
    g = layout_ok ? cu[b + 1] - cu[b] : 0;
    d0 = layout_ok ? cu[b] : 0;
    t0 = d0 + b;
  } else {
    __syncthreads();
    g = L.gamma;
    d0 = (long long)b * g;
    t0 = (long long)b * (g + 1);
  }
  const float T = A.temperature[b];
  const bool bad0 = !layout_ok || !temperature_ok(T);
  const bool greedy = T == 0.0f;
  const float c32 = bad0 || greedy ? 0.0f : c32_of(T);
  const double c = (double)c32;

  // --- per-position inputs: token, uniforms, and the two logits at the token
  if (!bad0) {
    bool lbad = false;
    for (int i = tid; i <= g; i += kVT) {
      int x = 0;
      float u_a = 0.f, u_s = 0.f, lt = 0.f, ld = 0.f;
      if (i < g) x = A.tokens[d0 + i];
      const bool xok = i == g || (x >= 0 && x < V);
      if (!greedy) {
        u_s = A.us[t0 + i];
        if (i < g) u_a = A.ua[d0 + i];
        if (i < g && xok) {
          lt = Elem<DT>::at(tgt, (t0 + i) * (long long)V + x);
          ld = Elem<DT>::at(dft, (d0 + i) * (long long)V + x);
        }
        lbad |= !uniform_ok(u_s) || (i < g && !uniform_ok(u_a));
      }
      lbad |= !xok;
      P.x[i] = x;
      P.ua[i] = u_a;
      P.us[i] = u_s;
      P.lt[i] = lt;
      P.ld[i] = ld;
    }
    if (lbad) S.bad = 1;

    // --- row statistics: target rows 0..g, then (T > 0) draft rows 0..g-1
    const int nrows = (g + 1) + (greedy ? 0 : g);
    const int grp = tid / kRowLanes, sub = tid % kRowLanes;
    for (int r = grp; r < nrows; r += kRowGroups) {
      const long long prow = r <= g ? t0 + r : L.RT + d0 + (r - g - 1);
      float M;
      int idx;
      double Z;
      bool ok;
      merge_row_group(A.part + prow * A.nchunk, A.nchunk, c, greedy, sub, M, idx, Z, ok);
      if (sub == 0) {
        P.rm[r] = M;
        P.rz[r] = Z;
        P.ridx[r] = idx;
        P.rok[r] = ok;
      }
    }
  }
  __syncthreads();

  // --- decisions per position; validation covers every position
  if (!bad0) {
    bool lbad = false;
    int rej = 0x7fffffff;
    for (int i = tid; i <= g; i += kVT) {
      bool pb = !P.rok[i];
      if (i < g && !greedy) pb |= !P.rok[g + 1 + i];
      lbad |= pb;
      if (i < g && !pb) {
        const int x = P.x[i];
        bool reject;
        if (greedy) {
          reject = x != P.ridx[i];
        } else {
          const double pt = exp2_f64(((double)P.lt[i] - (double)P.rm[i]) * c) / P.rz[i];
          const double pd = exp2_f64(((double)P.ld[i] - (double)P.rm[g + 1 + i]) * c) / P.rz[g + 1 + i];
          reject = !((double)P.ua[i] * pd < pt);
          P.pt[i] = (float)pt;
          P.pd[i] = (float)pd;
        }
        if (reject && i < rej) rej = i;
      }
    }
    if (lbad) S.bad = 1;
    if (rej != 0x7fffffff) atomicMin(&S.n, rej);
  }
  __syncthreads();

  // --- outputs and the sampling job
  const bool bad = bad0 || S.bad != 0;
  const int n = bad ? 0 : min(S.n, g);
  for (int k = tid; write && k < out_width; k += kVT) {
    int v = -1;
    if (!bad) {
      if (k < n) v = P.x[k];
      else if (k == n && greedy) v = P.ridx[n];
    }
    orow[k] = v;
  }
  if (write && tid == 0) A.num_acc[b] = bad ? -1 : n;
  if (write && A.diag)
    for (int i = tid; i < g; i += kVT) {
      const float qnan = __uint_as_float(0x7fc00000u);
      A.diag[2 * (d0 + i)] = bad || greedy ? qnan : P.pt[i];
      A.diag[2 * (d0 + i) + 1] = bad || greedy ? qnan : P.pd[i];
    }
  if (tid == 0) {
    SampleJob J;
    J.kind = (bad || greedy) ? JOB_NONE : (n < g ? JOB_RESIDUAL : JOB_BONUS);
    J.pos = n;
    J.trow = t0 + n;
    J.drow = d0 + n;
    J.c64 = bad || greedy ? 0.0 : c64_of(T);
    J.c32 = c32;
    J.skip = 0ull;
    J.chunk_tiles = 0;
    J.pad = 0;
    J.u = bad || greedy ? 0.0f : P.us[n];
    J.mt = bad ? 0.0f : P.rm[n];
    J.md = J.kind == JOB_RESIDUAL ? P.rm[g + 1 + n] : 0.0f;
    J.rho = J.kind == JOB_RESIDUAL ? P.rz[n] / P.rz[g + 1 + n] : 0.0;
    S.job = J;
  }
}

// ---------------------------------------------------------------------------
// Tile loads.

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

// One 16-byte vector of tokens j .. j+epv-1 (element order of unpack<DT>);
// tokens at or beyond V read as -inf. A vector load when the vector is in range
// and 16-byte aligned, token by token otherwise.
template <int DT>
__device__ __forceinline__ uint4 load_vec(const void* rowp, int j, int V) {
  constexpr int epv = Elem<DT>::kPerVec;
  constexpr int es = sizeof(typename Elem<DT>::T);
  const char* p = reinterpret_cast<const char*>(rowp) + (size_t)j * es;
  if (j + epv <= V && (reinterpret_cast<uintptr_t>(p) & 15u) == 0) return *reinterpret_cast<const uint4*>(p);
  uint32_t bits[epv];
#pragma unroll
  for (int e = 0; e < epv; ++e) bits[e] = j + e < V ? raw_at<DT>(rowp, j + e) : NegInf<DT>::bits;
  if constexpr (DT == 1)
    return make_uint4(bits[0] | (bits[1] << 16), bits[2] | (bits[3] << 16), bits[4] | (bits[5] << 16),
                      bits[6] | (bits[7] << 16));
  else
    return make_uint4(bits[0], bits[1], bits[2], bits[3]);
}

// A wave's tile: lane l holds vectors u*64 + l (u < nv) of the tile, i.e. tokens
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
    for (int u = 0; u < nv; ++u) w[u] = load_vec<DT>(rowp, j0 + (u * 64 + lane) * epv, V);
  }
}

// ---------------------------------------------------------------------------
// Tile pass.

// Record fields of a tile pass: lanes 0..kGrp-1 hold the group sums, lane 0
// writes the scalar fields.
__device__ __forceinline__ void write_rec(TileRec* rec, double zt, double zd, double dp, double bp, int ng, double gt,
                                          double gd, int lane) {
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

// LDS copy of the waves' tiles (raw 16-byte vectors [u][lane]) for the per-token
// double-precision fixup; residual draws also stage the draft row.
template <int DT>
struct TileStage {
  static constexpr int nv = kEPL / Elem<DT>::kPerVec;
  uint4 t[kVW][nv][64];
  uint4 d[kVW][nv][64];
};

// Double-precision treatment of one flagged token (has == false: this lane has
// none left this step, but still takes part in the wave ballot).
struct ExactAcc {
  double zt, zd, dp, bp;
  int n;  // undecided tokens seen (wave-uniform)
};

template <bool RES>
__device__ __forceinline__ void exact_token(bool has, float xt, float xd, const SampleJob& J, double hi, double lo,
                                            unsigned long long below, ExactAcc& A, TileLists& L, int wv,
                                            const double* tab) {
  double et = 0.0, ed = 0.0;
  bool und = false;
  if (has) {
    et = emass_t(xt, J.mt, J.c64, J.c32, tab);
    A.zt += et;
    if (RES) {
      ed = emass_t(xd, J.md, J.c64, J.c32, tab);
      A.zd += ed;
      if (et > hi * ed) {
        A.dp += et - J.rho * ed;
        A.bp += ed;
      } else {
        und = et > 0.0 && et >= lo * ed;
      }
    }
  }
  if (!RES) return;
  const unsigned long long m = __ballot(und);
  if (m) {
    const int slot = A.n + __builtin_popcountll(m & below);
    if (und && slot < kList) {
      L.dl[wv][slot] = (double)xt - (double)xd;
      L.et[wv][slot] = et;
      L.ed[wv][slot] = ed;
    }
    A.n += __builtin_popcountll(m);
  }
}

// Token e of a staged 16-byte vector, read from LDS.
template <int DT>
__device__ __forceinline__ float staged_at(const uint4& v, int e) {
  if constexpr (DT == 1) {
    const uint16_t bits = reinterpret_cast<const uint16_t*>(&v)[e];
    return __uint_as_float((uint32_t)bits << 16);
  } else {
    return reinterpret_cast<const float*>(&v)[e];
  }
}

// Pass over one tile by one wave; writes the tile record. The lane holds the
// tile's 16-byte vectors u*64 + lane (u < nv) in wt (and wd); its token (u, e)
// is token j0 + (u*64 + lane)*epv + e.
//
// Every token first goes through fp32. A token whose mass is below 2^-50 of its
// row maximum in both rows (fp32 argument a < kTinyExp) and, for a residual,
// whose likelihood ratio lies outside twice the band around rho~ contributes
// terms whose fp32 rounding is below 2^-70 of the row maximum: it is summed,
// and for a residual decided, in fp32. Every other token is flagged. The
// lane's flagged tokens are then taken one per step in double precision (fp64
// masses; the band decision in fp64; undecided tokens appended to a list in a
// fixed order (step, lane) through wave ballots), with their logits read back
// from an LDS copy of the tile. Near one-hot rows flag a handful of tokens per
// row; rows where every mass is significant flag every token.
template <int DT, bool RES>
__device__ __forceinline__ void tile_pass(const uint4 (&wt)[kEPL / Elem<DT>::kPerVec],
                                          const uint4 (&wd)[kEPL / Elem<DT>::kPerVec], const SampleJob& J,
                                          TileRec* rec, TileLists& L, TileStage<DT>& G, const double* tab, int wv,
                                          int lane) {
  constexpr int epv = Elem<DT>::kPerVec;
  constexpr int nv = kEPL / epv;
  static_assert(nv * epv <= 32, "one flag bit per token of the lane");
  const float mt = J.mt, md = J.md, c32 = J.c32;
  float st = 0.f, sd = 0.f, sdp = 0.f, sbp = 0.f;
  uint32_t flags = 0u;
  {
    const float rho32 = (float)J.rho;
    const float hi32 = (float)(J.rho * (1.0 + 2.0 * kRhoBand)), lo32 = (float)(J.rho * (1.0 - 2.0 * kRhoBand));
#pragma unroll
    for (int u = 0; u < nv; ++u) {
      float xt[epv], xd[epv];
      unpack<DT>(wt[u], xt);
      if (RES) unpack<DT>(wd[u], xd);
#pragma unroll
      for (int e = 0; e < epv; ++e) {
        const float at = (xt[e] - mt) * c32;
        const float et = exp2_f32(at);
        bool flag = at >= kTinyExp;
        if (RES) {
          const float ad = (xd[e] - md) * c32;
          const float ed = exp2_f32(ad);
          flag |= ad >= kTinyExp;
          const bool pos = et > hi32 * ed;
          flag |= !pos && et > 0.f && et >= lo32 * ed;
          if (!flag) {
            st += et;
            sd += ed;
            if (pos) {
              sdp += et - rho32 * ed;
              sbp += ed;
            }
          }
        } else if (!flag) {
          st += et;
        }
        flags |= (uint32_t)flag << (u * epv + e);
      }
    }
  }
  ExactAcc A{(double)st, (double)sd, (double)sdp, (double)sbp, 0};
  if (__any(flags != 0u)) {
#pragma unroll
    for (int u = 0; u < nv; ++u) {
      G.t[wv][u][lane] = wt[u];
      if (RES) G.d[wv][u][lane] = wd[u];
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    __builtin_amdgcn_wave_barrier();
    const double hi = J.rho * (1.0 + kRhoBand), lo = J.rho * (1.0 - kRhoBand);
    const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll 1
    while (__any(flags != 0u)) {
      const bool has = flags != 0u;
      const int i = has ? __builtin_ctz(flags) : 0;
      flags &= flags - 1u;
      float xt = 0.f, xd = 0.f;
      if (has) {
        xt = staged_at<DT>(G.t[wv][i / epv][lane], i % epv);
        if (RES) xd = staged_at<DT>(G.d[wv][i / epv][lane], i % epv);
      }
      exact_token<RES>(has, xt, xd, J, hi, lo, below, A, L, wv, tab);
    }
    // the stage and the lists are reused by the wave's next tile
    __builtin_amdgcn_wave_barrier();
  }
  auto add = [](double a, double b) { return a + b; };
  const double zt = wave_reduce(A.zt, add);
  double zd = 0.0, dp = 0.0, bp = 0.0, gt = 0.0, gd = 0.0;  // lane g < ng holds group g's sums
  int ng = 0;
  if (RES) {
    zd = wave_reduce(A.zd, add);
    dp = wave_reduce(A.dp, add);
    bp = wave_reduce(A.bp, add);
    const int n = A.n;
    if (n > kList) {
      ng = kRecOverflow;
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
        ng = kRecOverflow;
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
  write_rec(rec, zt, zd, dp, bp, ng, gt, gd, lane);
}

// One wave's tile k (if below ntile and not in a skipped chunk).
template <int DT, bool RES>
__device__ __forceinline__ void wave_tile(const char* trow, const char* drow, int V, int ntile, int k,
                                          const SampleJob& J, TileRec* R, TileLists& L, TileStage<DT>& G,
                                          const double* tab, int wv, int lane) {
  constexpr int nv = kEPL / Elem<DT>::kPerVec;
  if (k >= ntile) return;
  if (!RES && J.skip && ((J.skip >> (k / J.chunk_tiles)) & 1ull)) return;
  uint4 wt[nv], wd[nv];
  load_tile_wave<DT>(trow, k * kSTile, V, lane, wt);
  if (RES) load_tile_wave<DT>(drow, k * kSTile, V, lane, wd);
  tile_pass<DT, RES>(wt, RES ? wd : wt, J, R + k, L, G, tab, wv, lane);
}

// ---------------------------------------------------------------------------
// Pick.

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
  for (int w = 1; w < kVW; ++w) t += red[w];
  __syncthreads();
  return t;
}

// A workgroup's tile: thread tid holds the kBT contiguous tokens j0 + kBT tid + i
// (-inf beyond V).
template <int DT>
__device__ __forceinline__ void load_tile_block(const char* rowp, int j0, int V, float* x) {
#pragma unroll
  for (int i = 0; i < kBT; ++i) {
    const int j = j0 + kBT * (int)threadIdx.x + i;
    x[i] = j < V ? Elem<DT>::at(rowp, j) : -INFINITY;
  }
}

template <int DT>
__device__ void pick(const char* trow, const char* drow, int V, int ntile, const SampleJob& J, TileRec* R,
                     int32_t* dst, int force_exact, PickSpace& P, const double* tab) {
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  auto add = [](double a, double b) { return a + b; };
  // --- exact normalisers: wave 0, lanes over tiles, fixed-order sums
  if (wv == 0) {
    double zt = 0.0, zd = 0.0;
    int need = 0;
    for (int k = lane; k < ntile; k += 64) {
      zt += R[k].zt;
      zd += R[k].zd;
      need |= R[k].ngrp == kRecOverflow;
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

  // --- tiles whose residual mass is recomputed token by token (then marked kRecRecomputed, mass in zd)
  if (P.any_exact) {
    const bool all = P.any_exact == 2;
    for (int k = 0; k < ntile; ++k) {
      if (!(all || R[k].ngrp == kRecOverflow)) continue;
      float xt[kBT], xd[kBT];
      load_tile_block<DT>(trow, k * kSTile, V, xt);
      load_tile_block<DT>(drow, k * kSTile, V, xd);
      double acc = 0.0;
#pragma unroll
      for (int i = 0; i < kBT; ++i) {
        const double q = emass_t(xt[i], J.mt, J.c64, J.c32, tab) - rho * emass_t(xd[i], J.md, J.c64, J.c32, tab);
        acc += q > 0.0 ? q : 0.0;
      }
      acc = block_sum(acc, P.red);
      if (tid == 0) {
        R[k].zd = acc;
        R[k].ngrp = kRecRecomputed;
      }
      __syncthreads();
    }
  }

  // --- tile masses, total S, and the first tile whose inclusive prefix exceeds u S (wave 0)
  auto tile_mass = [&](int k, bool r) -> double {
    if (!r) return R[k].zt;
    const int ng = R[k].ngrp;
    if (ng == kRecRecomputed) return R[k].zd;
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

  // --- masses of the chosen unit (a tile, or every tile of a skipped chunk), kBT
  // contiguous tokens per thread, then a fixed-order scan from the unit's base
  int tile_end = tile + 1;
  if (!res && R[tile].ngrp == kRecChunkHead) tile_end = min(ntile, tile + J.chunk_tiles);
  double base = Wtile;
  int found = 0x7fffffff, lastpos = -1;
  for (int t = tile; t < tile_end; ++t) {
    double q[kBT];
    double local = 0.0;
    {
      float xt[kBT], xd[kBT];
      load_tile_block<DT>(trow, t * kSTile, V, xt);
      if (res) load_tile_block<DT>(drow, t * kSTile, V, xd);
#pragma unroll
      for (int i = 0; i < kBT; ++i) {
        double v = emass_t(xt[i], J.mt, J.c64, J.c32, tab);
        if (res) {
          v -= rho * emass_t(xd[i], J.md, J.c64, J.c32, tab);
          v = v > 0.0 ? v : 0.0;
        }
        q[i] = v;
        local += v;
      }
    }
    const double wincl = wave_incl_scan(local, lane);
    if (lane == 63) P.red[wv] = wincl;
    __syncthreads();
    double run = base;
    for (int w = 0; w < wv; ++w) run += P.red[w];
    run += wincl - local;
    double total = 0.0;  // the tile's sum, in the same order in every thread
    for (int w = 0; w < kVW; ++w) total += P.red[w];
    const int jt = t * kSTile + tid * kBT;
    int pk = 0x7fffffff, lp = -1;
#pragma unroll
    for (int i = 0; i < kBT; ++i) {
      run += q[i];
      if (q[i] > 0.0) {
        lp = jt + i;
        if (!last_mode && run > thr && pk == 0x7fffffff) pk = jt + i;
      }
    }
    pk = wave_reduce(pk, [](int a, int b) { return a < b ? a : b; });
    lp = wave_reduce(lp, [](int a, int b) { return a > b ? a : b; });
    if (lane == 0) { P.smin[wv] = pk; P.smax[wv] = lp; }
    __syncthreads();
    for (int w = 0; w < kVW; ++w) {
      found = min(found, P.smin[w]);
      lastpos = max(lastpos, P.smax[w]);
    }
    __syncthreads();  // P is reused by the next tile
    base = base + total;
    if (found != 0x7fffffff) break;
  }
  // no token passed u S in the unit (rounding at its end): the last positive token
  if (tid == 0) *dst = found != 0x7fffffff ? found : lastpos;
}

// ---------------------------------------------------------------------------
// Kernels.

// The job from shared memory into scalar registers (it is the same for every
// thread; a plain load would hold it in vector registers).
__device__ __forceinline__ SampleJob uniform_job(const SampleJob& src) {
  static_assert(sizeof(SampleJob) % 4 == 0, "job of 32-bit words");
  constexpr int nw = sizeof(SampleJob) / 4;
  int w[nw];
  const int* p = reinterpret_cast<const int*>(&src);
#pragma unroll
  for (int i = 0; i < nw; ++i) w[i] = __builtin_amdgcn_readfirstlane(p[i]);
  SampleJob J;
  __builtin_memcpy(&J, w, sizeof(J));
  return J;
}

// Chain acceptance scan, one workgroup per request: outputs and the job.
//
// For a bonus draw whose row is 16-byte aligned (so that the streaming pass's
// chunks start on tile boundaries), a chunk whose maximum lies more than
// -kTinyExp below the row maximum (in units of the exponent argument) holds
// only negligible masses: every token would take the fp32 sum of the triage.
// Its tiles are not read again; its mass comes from the chunk's partial,
// s 2^{(m_chunk - m_row) c}, accurate to the fp32 sum of the streaming pass
// (relative 1e-6 of a total below 2^-36 of the row maximum's mass), and is
// recorded in the chunk's first tile.
template <int DT>
__global__ __launch_bounds__(kVT) void k_accept_chain(const void* __restrict__ tgt, const void* __restrict__ dft,
                                                      int V, ChainArgs A, SampleJob* __restrict__ jobs,
                                                      TileRec* __restrict__ recs, int32_t* __restrict__ out,
                                                      int out_width) {
  __shared__ VerifyShared S;
  const int b = blockIdx.x;
  accept_chain<DT>(tgt, dft, V, A, b, out + (long long)b * out_width, out_width, true, S);
  __syncthreads();
  if (threadIdx.x >= 64) return;
  SampleJob J = S.job;
  constexpr int es = sizeof(typename Elem<DT>::T);
  constexpr int epv = Elem<DT>::kPerVec;
  const int lane = threadIdx.x;
  const long long ctok = (long long)A.chunk_vecs * epv;
  const bool aligned_row =
      (reinterpret_cast<uintptr_t>(reinterpret_cast<const char*>(tgt) + (size_t)J.trow * (size_t)V * es) & 15u) == 0;
  if (J.kind == JOB_BONUS && aligned_row && A.nchunk <= 64 && A.nchunk > 1 && ctok % kSTile == 0) {
    const int tpc = (int)(ctok / kSTile);
    const int ntile = (V + kSTile - 1) / kSTile;
    bool tiny = false;
    double mass = 0.0;
    if (lane < A.nchunk) {
      const Partial q = A.part[J.trow * A.nchunk + lane];
      const float a32 = (q.m - J.mt) * J.c32;  // the largest triage argument in the chunk
      tiny = q.m == -INFINITY || a32 < kTinyExp;
      if (tiny && q.m > -INFINITY) mass = (double)q.s * exp2_f64(((double)q.m - (double)J.mt) * (double)J.c32);
    }
    const unsigned long long mask = __ballot(tiny);
    if (tiny) {
      TileRec* R = recs + (long long)b * ntile + (long long)lane * tpc;
      for (int i = 0; i < tpc && lane * tpc + i < ntile; ++i) {
        R[i].zt = i == 0 ? mass : 0.0;
        R[i].zd = 0.0;
        R[i].dpos = 0.0;
        R[i].bpos = 0.0;
        R[i].ngrp = i == 0 ? kRecChunkHead : kRecChunkBody;
        R[i].pad = 0;
      }
    }
    J.skip = mask;
    J.chunk_tiles = tpc;
  }
  if (lane == 0) jobs[b] = J;
}

// Workgroup (b, g), g < G: tiles g*kTPG + i*G*kTPG + [0, kTPG) of request b's
// drawn row(s).
template <int DT>
__global__ __launch_bounds__(kVT) void k_tiles(const void* __restrict__ tgt, const void* __restrict__ dft, int V,
                                               int G, const SampleJob* __restrict__ jobs,
                                               TileRec* __restrict__ recs) {
  __shared__ TileLists lists;
  __shared__ TileStage<DT> stage;
  __shared__ double exp2tab[64];
  __shared__ SampleJob sj;
  if (threadIdx.x < 64) exp2tab[threadIdx.x] = exp2_f64((double)threadIdx.x * 0.015625);
  const int b = blockIdx.x / G, g = blockIdx.x - b * G;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (threadIdx.x == 0) sj = jobs[b];
  __syncthreads();
  const SampleJob J = uniform_job(sj);
  if (J.kind == JOB_NONE) return;
  constexpr int es = sizeof(typename Elem<DT>::T);
  const char* trow = reinterpret_cast<const char*>(tgt) + (size_t)J.trow * (size_t)V * es;
  const char* drow = reinterpret_cast<const char*>(dft) + (size_t)J.drow * (size_t)V * es;
  const int ntile = (V + kSTile - 1) / kSTile;
  TileRec* R = recs + (long long)b * ntile;
  for (int base = g * kTPG; base < ntile; base += G * kTPG) {
    if (J.kind == JOB_RESIDUAL)
      wave_tile<DT, true>(trow, drow, V, ntile, base + wv, J, R, lists, stage, exp2tab, wv, lane);
    else
      wave_tile<DT, false>(trow, trow, V, ntile, base + wv, J, R, lists, stage, exp2tab, wv, lane);
  }
}

template <int DT>
__global__ __launch_bounds__(kVT) void k_pick(const void* __restrict__ tgt, const void* __restrict__ dft, int V,
                                              const SampleJob* __restrict__ jobs, TileRec* __restrict__ recs,
                                              int32_t* __restrict__ out, int out_width, int force_exact) {
  __shared__ PickShared S;
  if (threadIdx.x < 64) S.exp2tab[threadIdx.x] = exp2_f64((double)threadIdx.x * 0.015625);
  if (threadIdx.x == 0) S.job = jobs[blockIdx.x];
  __syncthreads();
  const SampleJob J = uniform_job(S.job);
  if (J.kind == JOB_NONE) return;
  const int b = blockIdx.x;
  constexpr int es = sizeof(typename Elem<DT>::T);
  const char* trow = reinterpret_cast<const char*>(tgt) + (size_t)J.trow * (size_t)V * es;
  const char* drow = reinterpret_cast<const char*>(dft) + (size_t)J.drow * (size_t)V * es;
  const int ntile = (V + kSTile - 1) / kSTile;
  pick<DT>(trow, drow, V, ntile, J, recs + (long long)b * ntile, out + (long long)b * out_width + J.pos, force_exact,
           S.pick, S.exp2tab);
}

// ---------------------------------------------------------------------------
// Launchers.

// Workgroups per request of k_tiles: one per kTPG tiles, capped so that the
// grid stays within 2^20 workgroups.
static int tiles_groups(int B, int V) {
  const int ntile = (V + kSTile - 1) / kSTile;
  int G = (ntile + kTPG - 1) / kTPG;
  const long long cap = (1ll << 20) / (B > 0 ? B : 1);
  if (G > cap) G = (int)cap;
  return G < 1 ? 1 : G;
}

template <int DT>
static hipError_t launch_draw(const void* tgt, const void* dft, int V, int B, SampleJob* jobs, TileRec* recs,
                              int32_t* out, int out_width, int force_exact, hipStream_t st) {
  const int G = tiles_groups(B, V);
  hipLaunchKernelGGL(k_tiles<DT>, dim3((unsigned)(B * G)), dim3(kVT), 0, st, tgt, dft, V, G, jobs, recs);
  hipLaunchKernelGGL(k_pick<DT>, dim3((unsigned)B), dim3(kVT), 0, st, tgt, dft, V, jobs, recs, out, out_width,
                     force_exact);
  return hipGetLastError();
}

template <int DT>
static hipError_t launch_chain(const void* tgt, const void* dft, int V, int B, const ChainArgs& A, SampleJob* jobs,
                               TileRec* recs, int32_t* out, int out_width, int force_exact, hipStream_t st) {
  hipLaunchKernelGGL(k_accept_chain<DT>, dim3((unsigned)B), dim3(kVT), 0, st, tgt, dft, V, A, jobs, recs, out,
                     out_width);
  return launch_draw<DT>(tgt, dft, V, B, jobs, recs, out, out_width, force_exact, st);
}

hipError_t launch_finish_chain(int dt, const void* tgt, const void* dft, int V, const Layout& L,
                               const int32_t* tokens, const float* ua, const float* us, const float* temperature,
                               const Partial* part, int nchunk, int chunk_vecs, int32_t* out, int out_width,
                               int32_t* num_acc, float* diag, SampleJob* jobs, TileRec* recs, int force_exact,
                               hipStream_t st) {
  if (L.B == 0) return hipSuccess;
  const ChainArgs A{L, tokens, ua, us, temperature, part, nchunk, chunk_vecs, num_acc, diag};
  return dt == 1 ? launch_chain<1>(tgt, dft, V, L.B, A, jobs, recs, out, out_width, force_exact, st)
                 : launch_chain<0>(tgt, dft, V, L.B, A, jobs, recs, out, out_width, force_exact, st);
}

hipError_t launch_finish_jobs(int dt, const void* tgt, const void* dft, int V, int B, SampleJob* jobs,
                              TileRec* recs, int32_t* out, int out_width, int force_exact, hipStream_t st) {
  if (B == 0) return hipSuccess;
  return dt == 1 ? launch_draw<1>(tgt, dft, V, B, jobs, recs, out, out_width, force_exact, st)
                 : launch_draw<0>(tgt, dft, V, B, jobs, recs, out, out_width, force_exact, st);
}

}  // namespace sv
