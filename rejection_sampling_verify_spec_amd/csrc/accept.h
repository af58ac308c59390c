// accept.h -- acceptance decisions per request (device code).
//
// Chain [Primer 考点2 / 第二章]: drafted position i keeps its token x_i when
// u_accept[i] * p_d,i(x_i) < p_t,i(x_i), i.e. with probability
// min(1, p_t/p_d); the first rejected position n ends the scan. Greedy
// requests (T == 0) keep x_i while it equals the target argmax and emit the
// argmax at n. p(x) = 2^{(l_x - m) c} / Z, with Z merged here in fp64 from the
// per-chunk partials of the row-statistics kernel.
#pragma once

#include "sv_internal.h"

namespace sv {

struct RowStat {
  float m;   // row max
  double Z;  // sum 2^{(x-m)c32}
  int idx;   // greedy argmax
  bool ok;
};

// Merge the chunk partials of one row (chunks in ascending token order, so a
// strict comparison keeps the lowest index of a tied maximum). Partials are
// read four at a time so their loads overlap.
__device__ __forceinline__ RowStat merge_row(const Partial* __restrict__ p, int nchunk, float c32, bool greedy) {
  float M = -INFINITY;
  int idx = -1;
  bool nan = false;
  double Z = 0.0;
  const double c = (double)c32;
  for (int k0 = 0; k0 < nchunk; k0 += 4) {
    Partial q[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) q[u] = k0 + u < nchunk ? p[k0 + u] : Partial{-INFINITY, 0.0f, -1, 0};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      nan |= q[u].s != q[u].s;
      if (q[u].m > M) {
        // new running maximum: rescale what was summed so far
        if (!greedy && M > -INFINITY) Z *= exp2_f64(((double)M - (double)q[u].m) * c);
        M = q[u].m;
        idx = q[u].idx;
        if (!greedy) Z += (double)q[u].s;
      } else if (!greedy && q[u].m > -INFINITY) {
        Z += (double)q[u].s * exp2_f64(((double)q[u].m - (double)M) * c);
      }
    }
  }
  RowStat r{M, 0.0, idx, !nan && M > -INFINITY && M < INFINITY};
  if (greedy || !r.ok) return r;
  r.Z = Z;
  r.ok = Z > 0.0 && Z < 1e308;
  return r;
}

// probability of token x in a row with statistics st
template <int DT>
__device__ __forceinline__ double prob_at(const void* base, long long row, int V, int x, const RowStat& st, float c32) {
  float l = Elem<DT>::at(base, row * (long long)V + x);
  return exp2_f64(((double)l - (double)st.m) * (double)c32) / st.Z;
}

constexpr int kMaxPos = 1025;  // SV_MAX_GAMMA + 1

struct AcceptShared {
  float pt[kMaxPos], pd[kMaxPos];
  int amax[kMaxPos];
};

// Acceptance scan of chain request b by one wave (lane = position within a
// group of 64). Every workgroup of the request runs it on the same inputs and
// gets the same result; only the one with `write` set stores the outputs
// (out_tokens row, num_accepted, diagnostics, the request's job). The job is
// left in `sj` (LDS) for the calling workgroup.
template <int DT>
__device__ void accept_chain_wave(const void* __restrict__ tgt, const void* __restrict__ dft, int V,
                                  const Layout& L, int b, const int32_t* __restrict__ tokens,
                                  const float* __restrict__ ua, const float* __restrict__ us,
                                  const float* __restrict__ temperature, const Partial* __restrict__ part,
                                  int nchunk, int32_t* __restrict__ out, int out_width,
                                  int32_t* __restrict__ num_acc, float* __restrict__ diag,
                                  SampleJob* __restrict__ jobs, bool write, AcceptShared& S, SampleJob& sj,
                                  int lane) {
  // --- locate the request's rows
  bool layout_ok = true;
  int g;
  long long t0, d0;
  if (L.mode == LAYOUT_RAGGED) {
    const int32_t* cu = L.cu;
    bool ok = true;
    if (lane == 0) ok = cu[0] == 0 && cu[L.B] == L.total_draft;
    for (int k = lane; k < L.B; k += 64) {
      int lo = cu[k], hi = cu[k + 1];
      ok = ok && hi >= lo && hi - lo <= L.gamma;
    }
    layout_ok = __all(ok);
    g = layout_ok ? cu[b + 1] - cu[b] : 0;
    d0 = layout_ok ? cu[b] : 0;
    t0 = d0 + b;
  } else {
    g = L.gamma;
    d0 = (long long)b * g;
    t0 = (long long)b * (g + 1);
  }
  int32_t* orow = out + (long long)b * out_width;
  const float T = temperature[b];
  bool bad = !layout_ok || !temperature_ok(T);
  const bool greedy = T == 0.0f;
  const float c32 = bad || greedy ? 0.0f : c32_of(T);

  // --- pass A: validation and acceptance decisions. The lane holding the final
  // position n (first rejection, or gamma) writes the sampling job from its statistics.
  int n = g;  // first rejected position
  bool found = false;
  for (int base = 0; base <= g && !bad; base += 64) {
    const int i = base + lane;
    bool lbad = false, reject = false;
    RowStat st{0.f, 0.0, -1, true}, sd{0.f, 0.0, -1, true};
    if (i <= g) {
      int x = 0;
      float u = 0.f, usv = 0.f;
      if (i < g) {
        x = tokens[d0 + i];
        if (!greedy) u = ua[d0 + i];
      }
      if (!greedy) usv = us[t0 + i];
      st = merge_row(part + (t0 + i) * nchunk, nchunk, c32, greedy);
      lbad |= !st.ok;
      if (!greedy) lbad |= !uniform_ok(usv);
      if (i < g) {
        lbad |= x < 0 || x >= V;
        if (greedy) {
          reject = x != st.idx;
        } else {
          sd = merge_row(part + (L.RT + d0 + i) * nchunk, nchunk, c32, false);
          lbad |= !sd.ok || !uniform_ok(u);
          if (!lbad) {
            double pt = prob_at<DT>(tgt, t0 + i, V, x, st, c32);
            double pd = prob_at<DT>(dft, d0 + i, V, x, sd, c32);
            reject = !((double)u * pd < pt);
            S.pt[i] = (float)pt;
            S.pd[i] = (float)pd;
          }
        }
      }
      if (greedy) S.amax[i] = st.idx;
    }
    bad = __any(lbad) || bad;
    const unsigned long long rm = __ballot(reject && i < g);
    if (!found && rm) {
      n = base + __builtin_ctzll(rm);
      found = true;
    }
    // job of a sampling request, written by the lane of position n
    if (!greedy && i == n && (found || i == g)) {
      SampleJob J;
      J.kind = n < g ? JOB_RESIDUAL : JOB_BONUS;
      J.pos = n;
      J.trow = t0 + n;
      J.drow = d0 + n;
      J.c64 = c64_of(T);
      J.c32 = c32;
      J.u = us[t0 + n];
      J.mt = st.m;
      J.md = n < g ? sd.m : 0.0f;
      J.rho = n < g ? st.Z / sd.Z : 0.0;
      sj = J;
    }
    if (found) break;
  }
  // validation covers every position, also those after the first rejection
  for (int base = (n / 64 + 1) * 64; base <= g && !bad; base += 64) {
    const int i = base + lane;
    bool lbad = false;
    if (i <= g) {
      RowStat st = merge_row(part + (t0 + i) * nchunk, nchunk, c32, greedy);
      lbad |= !st.ok;
      if (!greedy) lbad |= !uniform_ok(us[t0 + i]);
      if (i < g) {
        const int x = tokens[d0 + i];
        lbad |= x < 0 || x >= V;
        if (!greedy) {
          RowStat sd = merge_row(part + (L.RT + d0 + i) * nchunk, nchunk, c32, false);
          lbad |= !sd.ok || !uniform_ok(ua[d0 + i]);
          if (!lbad && write) {  // per-position probabilities for the diagnostics output
            S.pt[i] = (float)prob_at<DT>(tgt, t0 + i, V, x, st, c32);
            S.pd[i] = (float)prob_at<DT>(dft, d0 + i, V, x, sd, c32);
          }
        }
      }
    }
    bad = __any(lbad) || bad;
  }
  // the job (or its absence) is final; LDS writes of one wave land in program order
  if (lane == 0 && (bad || greedy)) sj.kind = JOB_NONE;
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  __builtin_amdgcn_wave_barrier();
  if (!write) return;

  // --- outputs
  if (lane == 0) jobs[b] = sj;
  if (bad) {
    for (int k = lane; k < out_width; k += 64) orow[k] = -1;
    if (lane == 0) num_acc[b] = -1;
    return;
  }
  for (int k = lane; k < out_width; k += 64) {
    int v = -1;
    if (k < n) v = tokens[d0 + k];
    else if (k == n && greedy) v = S.amax[n];
    orow[k] = v;
  }
  if (diag)
    for (int i = lane; i < g; i += 64) {
      const float qnan = __uint_as_float(0x7fc00000u);
      diag[2 * (d0 + i)] = greedy ? qnan : S.pt[i];
      diag[2 * (d0 + i) + 1] = greedy ? qnan : S.pd[i];
    }
  if (lane == 0) num_acc[b] = n;
}

}  // namespace sv
