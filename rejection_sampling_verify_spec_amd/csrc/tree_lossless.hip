// tree_lossless.hip -- lossless multi-candidate token-tree verification.
//
// The tree of drafted tokens is verified in one target pass [Primer 考点3]; at
// the current node (from the root) the children are tried in ascending index
// order against the current distribution r, which starts as the node's target
// row: child c is accepted when u_accept[c] * p_d[c](x_c) < r(x_c) [Primer
// 考点2]. An accepted child becomes the current node. A rejected child replaces
// r by its residual max(0, r - p_d[c]) / sum [Primer 考点2, P'] before the next
// sibling is tried, which keeps every step's output distributed as the target
// row. When no child is accepted (or the node is a leaf) the final token is
// drawn from r by the inverse CDF with u_sample of the node.
//
// In unnormalised form, with R_0 = p_t[v] and S_0 = 1,
//   R_{i+1}(y) = max(0, R_i(y) - S_i p_d[c_i](y)),   S_{i+1} = sum_y R_{i+1}(y),
// so r = R_i / S_i after i rejected siblings, and child c_i is accepted when
// u * p_d[c_i](x) * S_i < R_i(x). Each rejection needs one full-vocabulary sum:
// a pass over the target row and the draft rows of the rejected siblings.
//
// One cooperative launch: a team of G workgroups per request (teams loop over
// requests). Every workgroup of a team walks the tree redundantly (the same
// inputs give the same decisions); a pass splits the row's segments (64
// vectors of 16 bytes) over the team's waves, each segment's sum of R is
// stored with a device-scope store, and the team meets at a counter (the
// launch keeps every workgroup resident, so the wait ends; it is also
// bounded). Each workgroup then sums the segment sums in the same fixed order.
// The first workgroup of the team writes the outputs and, at the end, picks
// the token inside the segment that holds u * S.
#include "accept.h"
#include "tail.h"

namespace sv {

constexpr int kLLWaves = 12;  // three per SIMD: one workgroup fills a CU, so a team meets with few members
constexpr int kLLThreads = kLLWaves * 64;
constexpr int kLLMaxNodes = SV_MAX_TREE_NODES;
constexpr int kLLSmallNodes = 128;  // trees up to this size keep most of the residual in LDS
constexpr int kSpinPolls = 1 << 24;  // bound of one team wait (a few seconds of polls)

struct LLArgs {
  const void* tgt;
  const void* dft;
  int V, N, B, max_depth;
  const int32_t* tokens;
  const int32_t* parents;
  const float* ua;
  const float* us;
  const float* temperature;
  const Partial* part;
  int nchunk;
  long long RT;      // rows of the target array (draft partials follow)
  double* sums;      // [nteams][2][nseg] segment sums, double-buffered over passes
  double* rbuf;      // [nteams][2][nseg * 64 * epv] the current node's residual R, per token (see team_pass)
  int* ctr;          // [nteams] passes completed x G, zero at launch
  int G, nteams, nseg;
  int32_t* out;
  int32_t* out_nodes;
  int32_t* num_acc;
};

// Shared memory of a workgroup for trees of up to M nodes (about 50 KB at
// 1024 nodes, 7 KB at 128; one workgroup per CU).
template <int M>
struct LLSpace {
  int par[M], tok[M];
  float mt[M];
  union {
    float md[M];  // sampling: draft-row maxima
    int idx[M];   // greedy: target-row argmax
  };
  double zt[M], zd[M];
  int kids[M];  // children of the current node, ascending (depths while the tree is checked)
  int rej[M];   // its rejected children, in order (depths while the tree is checked)
  unsigned char skip[M];  // 1 when that rejection's residual sum underflowed (r kept)
  double S[M + 1];
  double tab[64];
  int cnt[kLLWaves];
  int bad, flag, nk, wait_ok;
  int eff, have_store;  // which R buffer holds the current residual, and whether one does
};

__device__ __forceinline__ uint64_t f64_bits(double v) { return (uint64_t)__double_as_longlong(v); }

// One residual step at one token, max(0, R - s e), with the product rounded on
// its own (no fused multiply-add): when a rejected sibling's draft row equals
// the current distribution, R = fl(e' izt) and s e round to the same value and
// the step gives exactly 0, so the residual sum is 0 and r is kept, as in the
// definition. A fused form would leave the rounding error of R instead.
__device__ __forceinline__ double residual_step(double R, double s, double e) {
#pragma clang fp contract(off)
  const double se = s * e;
  return fmax(0.0, R - se);
}

// Segment sums of pass buffer `buf` read by one wave, kSegLoads per lane at a
// time with all loads in flight: lane l holds segments l + 64 k at v[k].
constexpr int kSegLoads = 8;
__device__ __forceinline__ void load_segments(const double* buf, int nseg, int k0, int lane,
                                              double (&v)[kSegLoads]) {
#pragma unroll
  for (int k = 0; k < kSegLoads; ++k) {
    const int t = (k0 + k) * 64 + lane;
    v[k] = t < nseg ? __longlong_as_double((long long)__hip_atomic_load(
                          reinterpret_cast<uint64_t*>(const_cast<double*>(buf)) + t, __ATOMIC_RELAXED,
                          __HIP_MEMORY_SCOPE_AGENT))
                    : 0.0;
  }
}

// Sum over the segments of pass buffer `buf`, in one fixed order (lane l adds
// segments l, l + 64, ... in turn; then the wave sum): the same value in every
// workgroup.
__device__ __forceinline__ double sum_segments(const double* buf, int nseg, int lane) {
  double s = 0.0;
  for (int k0 = 0; k0 * 64 < nseg; k0 += kSegLoads) {
    double v[kSegLoads];
    load_segments(buf, nseg, k0, lane, v);
#pragma unroll
    for (int k = 0; k < kSegLoads; ++k) s += v[k];
  }
  return wave_sum(s);
}

// The logit that lane l of wave 0 needs for the test of child c after nrej
// rejected siblings (l < nrej + 2 <= 64): the token's logit in the target row
// (l = 0), in rejected sibling l's draft row, or in c's draft row (l = nrej + 1).
template <int DT, class SP>
__device__ __forceinline__ float child_logit(const LLArgs& A, const SP& P, long long t0, long long d0, int v,
                                             int nrej, int c, int l) {
  const int x = P.tok[c];
  if (l == 0) return Elem<DT>::at(A.tgt, (t0 + v) * (long long)A.V + x);
  if (l >= nrej + 2) return 0.0f;
  const int w = l <= nrej ? P.rej[l - 1] : c;
  return Elem<DT>::at(A.dft, (d0 + w - 1) * (long long)A.V + x);
}

// The acceptance test of child c of node v after nrej rejected siblings: wave 0
// loads the token's logit in the target row, in each rejected sibling's draft
// row and in c's draft row at once (64 at a time) and forms their
// probabilities; the residual steps are then applied in order across the
// lanes (result in P.flag). With `pre`, lane l's logit of the first 64 was
// loaded earlier (while the pass before this test ran): `lg`.
template <int DT, class SP>
__device__ __forceinline__ void child_test(const LLArgs& A, SP& P, long long t0, long long d0, int v, int nrej,
                                           int c, double c64, bool pre = false, float lg = 0.0f) {
  const int tid = threadIdx.x, lane = tid & 63;
  if (tid < 64) {
    double R = 0.0, q = 0.0;
    for (int l0 = 0; l0 < nrej + 2; l0 += 64) {
      const int l = l0 + lane;
      const float lv = pre && l0 == 0 ? lg : child_logit<DT>(A, P, t0, d0, v, nrej, c, l);
      double m = 0.0;
      if (l == 0) {
        m = emass_t(lv, P.mt[v], c64, P.tab) * (1.0 / P.zt[v]);
      } else if (l < nrej + 2) {
        const int w = l <= nrej ? P.rej[l - 1] : c;
        m = emass_t(lv, P.md[w], c64, P.tab) * (1.0 / P.zd[w]);
      }
      const int n = min(64, nrej + 2 - l0);
      for (int k = 0; k < n; ++k) {
        const double mk = lane_f64(m, k);
        const int idx = l0 + k;
        if (idx == 0) R = mk;
        else if (idx <= nrej) R = P.skip[idx - 1] ? R : residual_step(R, P.S[idx - 1], mk);
        else q = mk;
      }
    }
    if (tid == 0) {
      P.flag = (double)A.ua[t0 + c] * q * P.S[nrej] < R;
      P.rej[nrej] = c;
      P.skip[nrej] = 0;
    }
  }
  __syncthreads();
}

// Next rejected sibling at or after k whose residual step applies (nrej if none).
template <class SP>
__device__ __forceinline__ int next_live(const SP& P, int k, int nrej) {
  while (k < nrej && P.skip[k]) ++k;
  return k;
}

// Segments of the pass: 64 consecutive 16-byte vectors of a row (64 * epv
// tokens), one vector per lane.
template <int DT> struct Seg { static constexpr int tok = 64 * Elem<DT>::kPerVec; };
constexpr int kSegBatch = 2;  // segments of one wave whose loads are in flight together

// Segments whose residual a wave keeps in LDS (small trees): 12 KB per wave,
// 144 KB for the workgroup's 12 waves, and 8 KB more as one extra segment for
// each of the workgroup's first waves (the waves that hold one segment more
// than the others when a row's segments do not divide evenly). The rest go to
// the workspace.
template <int DT> struct LdsSlots { static constexpr int n = 12288 / (Seg<DT>::tok * 8); };
template <int DT> struct LdsExtra { static constexpr int n = 8192 / (Seg<DT>::tok * 8); };

// A wave's LDS residual: slots 0 .. LdsSlots-1 in its own region, slot
// LdsSlots (when n says so) from the workgroup's extra segments.
struct LdsRes {
  double2* base;   // the wave's region (none when n == 0)
  double2* extra;  // its extra segment (none when n <= LdsSlots)
  int n;           // segments held in LDS
};

// LDS residual of one segment slot: token (lane*epv + e) of the segment at
// double2 (e/2)*64 + lane of the slot, component e % 2, so that a wave's
// 16-byte accesses are consecutive.
template <int DT>
__device__ __forceinline__ double2* lds_slot(const LdsRes& L, int slot, int lane) {
  return (slot < LdsSlots<DT>::n ? L.base + slot * (Seg<DT>::tok / 2) : L.extra) + lane;
}

// R at the lane's vector of up to kSegBatch segments (seg[i] < 0: none) of the
// current node: R[i*epv + e] for token (seg[i]*64 + lane)*epv + e. The vectors
// of one row are loaded together, and the next rejected sibling's row is in
// flight while the current one is applied. With `rin` (the residual this wave
// stored for the same segments in an earlier pass), R starts from it and only
// the steps step_from .. nrej-1 are applied: the same operations in the same
// order as from the rows, so the same values. The wave's segments j0 + i below
// lres.n hold that residual in LDS, the others at `rin`.
template <int DT, class SP>
__device__ __forceinline__ void residual_segs(const LLArgs& A, const SP& P, const char* trow, long long d0,
                                              int v, int nrej, const int (&seg)[kSegBatch], int lane, double c64,
                                              double (&R)[kSegBatch * Elem<DT>::kPerVec], const double* rin = nullptr,
                                              int step_from = 0, const LdsRes& lres = LdsRes{nullptr, nullptr, 0},
                                              int j0 = 0) {
  constexpr int epv = Elem<DT>::kPerVec;
  constexpr int es = sizeof(typename Elem<DT>::T);
  auto drow = [&](int k) {
    return reinterpret_cast<const char*>(A.dft) + (size_t)(d0 + P.rej[k] - 1) * (size_t)A.V * es;
  };
  // tokens past V (and absent segments) read as -inf: zero mass
  auto tokj = [&](int i) { return seg[i] < 0 ? A.V : (seg[i] * 64 + lane) * epv; };
  uint4 w[kSegBatch], wn[kSegBatch];
  if (!rin) {
#pragma unroll
    for (int i = 0; i < kSegBatch; ++i) w[i] = load_vec<DT>(trow, tokj(i), A.V);
  }
  int k = next_live(P, rin ? step_from : 0, nrej);
  if (k < nrej) {
    const char* dr = drow(k);
#pragma unroll
    for (int i = 0; i < kSegBatch; ++i) wn[i] = load_vec<DT>(dr, tokj(i), A.V);
  }
  const Exp2Regs K = pinned_exp2();
  if (rin) {
#pragma unroll
    for (int i = 0; i < kSegBatch; ++i) {
      if (j0 + i < lres.n) {  // (uniform)
        const double2* src = lds_slot<DT>(lres, j0 + i, lane);
#pragma unroll
        for (int q = 0; q < epv / 2; ++q) {
          const double2 v2 = src[q * 64];
          R[i * epv + 2 * q] = seg[i] < 0 ? 0.0 : v2.x;
          R[i * epv + 2 * q + 1] = seg[i] < 0 ? 0.0 : v2.y;
        }
        continue;
      }
      const double2* src =
          reinterpret_cast<const double2*>(rin + (size_t)(seg[i] < 0 ? 0 : seg[i]) * Seg<DT>::tok + lane * epv);
#pragma unroll
      for (int q = 0; q < epv / 2; ++q) {
        const double2 v2 = src[q];
        R[i * epv + 2 * q] = seg[i] < 0 ? 0.0 : v2.x;
        R[i * epv + 2 * q + 1] = seg[i] < 0 ? 0.0 : v2.y;
      }
    }
  } else {
    const float mt = P.mt[v];
    const double izt = 1.0 / P.zt[v];
#pragma unroll
    for (int i = 0; i < kSegBatch; ++i) {
      float x[epv];
      unpack<DT>(w[i], x);
#pragma unroll
      for (int e = 0; e < epv; ++e) R[i * epv + e] = emass_t(x[e], mt, c64, P.tab, K) * izt;
    }
  }
  while (k < nrej) {
#pragma unroll
    for (int i = 0; i < kSegBatch; ++i) w[i] = wn[i];
    const int c = P.rej[k];
    const double s = P.S[k] / P.zd[c];
    const float md = P.md[c];
    const int k2 = next_live(P, k + 1, nrej);
    if (k2 < nrej) {
      const char* dr = drow(k2);
#pragma unroll
      for (int i = 0; i < kSegBatch; ++i) wn[i] = load_vec<DT>(dr, tokj(i), A.V);
    }
#pragma unroll
    for (int i = 0; i < kSegBatch; ++i) {
      float x[epv];
      unpack<DT>(w[i], x);
#pragma unroll
      for (int e = 0; e < epv; ++e) R[i * epv + e] = residual_step(R[i * epv + e], s, emass_t(x[e], md, c64, P.tab, K));
    }
    k = k2;
  }
}

// One pass: the team's waves take the segments in turn (wave g of the team:
// segments g, g + nw, ...), kSegBatch at a time, and store each segment's sum
// of R; then the team meets. Returns false when the wait ran out of polls.
// A wave takes the same segments in every pass, so it can keep R for them:
// with `rin`, R is its stored residual plus the steps step_from .. nrej-1
// (one new rejected sibling's row instead of all of them), else it is formed
// from the rows; with `rout`, the new R is stored there. The wave's first
// lres.n segments keep R in LDS instead, updated in place (only this wave
// reads them, and it reads a segment before it writes it). Wave w of
// workgroup `rank` takes segments w G + rank + j nw, j = 0, 1, ...: where the
// segments do not divide evenly, the waves with one more are spread over the
// workgroups (their first waves) rather than gathered in one.
template <int DT, class SP>
__device__ bool team_pass(const LLArgs& A, SP& P, long long t0, long long d0, int v, int nrej, double* buf,
                          int* ctr, int target, int rank, double c64, const double* rin, int step_from,
                          double* rout, const LdsRes& lres) {
  constexpr int epv = Elem<DT>::kPerVec;
  constexpr int es = sizeof(typename Elem<DT>::T);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // (uniform: segment indices in scalar registers)
  const int nw = A.G * kLLWaves;
  const char* trow = reinterpret_cast<const char*>(A.tgt) + (size_t)(t0 + v) * (size_t)A.V * es;
  int j0 = 0;  // the wave's index of segment s0 among its own segments
  for (int s0 = wv * A.G + rank; s0 < A.nseg; s0 += nw * kSegBatch, j0 += kSegBatch) {
    int seg[kSegBatch];
#pragma unroll
    for (int i = 0; i < kSegBatch; ++i) seg[i] = s0 + i * nw < A.nseg ? s0 + i * nw : -1;
    double R[kSegBatch * epv];
    residual_segs<DT>(A, P, trow, d0, v, nrej, seg, lane, c64, R, rin, step_from, lres, j0);
    if (rout) {
#pragma unroll
      for (int i = 0; i < kSegBatch; ++i) {
        if (seg[i] < 0) continue;
        if (j0 + i < lres.n) {
          double2* dst = lds_slot<DT>(lres, j0 + i, lane);
#pragma unroll
          for (int q = 0; q < epv / 2; ++q) dst[q * 64] = make_double2(R[i * epv + 2 * q], R[i * epv + 2 * q + 1]);
          continue;
        }
        double* dst = rout + (size_t)seg[i] * Seg<DT>::tok + lane * epv;
#pragma unroll
        for (int e = 0; e < epv; ++e) dst[e] = R[i * epv + e];
      }
    }
#pragma unroll
    for (int i = 0; i < kSegBatch; ++i) {
      double s = 0.0;
#pragma unroll
      for (int e = 0; e < epv; ++e) s += R[i * epv + e];
      s = wave_sum(s);
      if (lane == 0 && seg[i] >= 0)
        __hip_atomic_store(reinterpret_cast<uint64_t*>(buf) + seg[i], f64_bits(s), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  // the segment sums are complete before the count
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // (every value the team exchanges is a device-scope atomic access, so the
  // completed stores need no fence: a fence would write back the whole L2)
  if (tid == 0) {
    atomicAdd(ctr, 1);
    int seen = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int polls = 0;
    while (seen < target && polls < kSpinPolls) {
      __builtin_amdgcn_s_sleep(8);
      seen = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ++polls;
    }
    P.wait_ok = seen >= target;
  }
  __syncthreads();
  return P.wait_ok != 0;
}

// Children of node v in ascending index order into P.kids / P.nk.
template <class SP>
__device__ __forceinline__ void list_children(SP& P, int N, int v) {
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  int base = 0;
  for (int c0 = 1; c0 < N; c0 += kLLThreads) {
    const int c = c0 + tid;
    const bool f = c < N && P.par[c] == v;
    const unsigned long long m = __ballot(f);
    if (lane == 0) P.cnt[wv] = __popcll(m);
    __syncthreads();
    int off = base;
    for (int w = 0; w < wv; ++w) off += P.cnt[w];
    if (f) P.kids[off + __popcll(m & ((1ull << lane) - 1ull))] = c;
    for (int w = 0; w < kLLWaves; ++w) base += P.cnt[w];
    __syncthreads();
  }
  if (tid == 0) P.nk = base;
  __syncthreads();
}

// The inverse-CDF pick of the final token by wave 0 of the team's first
// workgroup: the segment whose running sum first exceeds u * S, then the token
// in it; the last token of positive mass when rounding leaves none.
template <int DT, class SP>
__device__ int pick_token(const LLArgs& A, SP& P, long long t0, long long d0, int v, int nrej,
                          const double* buf, double thr, double c64, int lane) {
  constexpr int epv = Elem<DT>::kPerVec;
  // the segment
  double base = 0.0;
  int sg = -1, last_pos = -1;
  for (int k0 = 0; k0 * 64 < A.nseg && sg < 0; k0 += kSegLoads) {
    double sv[kSegLoads];
    load_segments(buf, A.nseg, k0, lane, sv);
#pragma unroll
    for (int k = 0; k < kSegLoads; ++k) {
      if (sg >= 0) break;
      const int t0w = (k0 + k) * 64;
      const double s = sv[k];
      const double incl = wave_incl_scan(s) + base;
      const unsigned long long hit = __ballot(incl > thr && s > 0.0);
      const unsigned long long pos = __ballot(s > 0.0);
      if (pos) last_pos = t0w + 63 - __clzll(pos);
      if (hit) {
        const int l = __ffsll((long long)hit) - 1;
        sg = t0w + l;
        base = l > 0 ? lane_f64(incl, l - 1) : base;
      } else {
        base = lane_f64(incl, 63);
      }
    }
  }
  const bool fallback = sg < 0;
  if (fallback) sg = last_pos;
  if (sg < 0) return -1;
  // the token inside the segment, in ascending order (lane, element)
  constexpr int es = sizeof(typename Elem<DT>::T);
  const char* trow = reinterpret_cast<const char*>(A.tgt) + (size_t)(t0 + v) * (size_t)A.V * es;
  int seg[kSegBatch];
  seg[0] = sg;
#pragma unroll
  for (int i = 1; i < kSegBatch; ++i) seg[i] = -1;
  double R[kSegBatch * epv];
  residual_segs<DT>(A, P, trow, d0, v, nrej, seg, lane, c64, R);
  const int jl = (sg * 64 + lane) * epv;
  double s = 0.0;
#pragma unroll
  for (int e = 0; e < epv; ++e) s += R[e];
  const double incl = wave_incl_scan(s) + base;
  int mylast = -1;
#pragma unroll
  for (int e = 0; e < epv; ++e)
    if (R[e] > 0.0) mylast = jl + e;
  const int ylast = wave_minmax<true>(mylast);
  int y = -1;
  const unsigned long long hit = fallback ? 0ull : __ballot(incl > thr && s > 0.0);
  if (hit) {
    const int l = __ffsll((long long)hit) - 1;
    const double excl = l > 0 ? lane_f64(incl, l - 1) : base;
    int mine = -1;
    if (lane == l) {
      double C = excl;
#pragma unroll
      for (int e = 0; e < epv; ++e) {
        C += R[e];
        if (mine < 0 && R[e] > 0.0 && C > thr) mine = jl + e;
      }
    }
    y = __builtin_amdgcn_readlane(mine, l);
  }
  return y >= 0 ? y : ylast;
}

// kSmall: trees of up to kLLSmallNodes nodes, with the residual of each wave's
// first segments in LDS.
template <int DT, bool kSmall>
__global__ __launch_bounds__(kLLThreads) __attribute__((amdgpu_waves_per_eu(3))) void k_tree_lossless(LLArgs A) {
  __shared__ LLSpace<kSmall ? kLLSmallNodes : kLLMaxNodes> P;
  constexpr int kSlots = kSmall ? LdsSlots<DT>::n : 0;
  constexpr int kExtra = kSmall ? LdsExtra<DT>::n : 0;
  constexpr int kS2 = Seg<DT>::tok / 2;  // double2 per segment
  __shared__ double2 RL[kSmall ? (kLLWaves * kSlots + kExtra) * kS2 : 1];
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int wvu = __builtin_amdgcn_readfirstlane(wv);
  const LdsRes lres = kSmall ? LdsRes{RL + wvu * kSlots * kS2, wvu < kExtra ? RL + (kLLWaves * kSlots + wvu) * kS2 : nullptr,
                                      kSlots + (wvu < kExtra ? 1 : 0)}
                             : LdsRes{nullptr, nullptr, 0};
  // a team's workgroups on one XCD when the teams fill whole XCD rounds
  // (workgroup i of the grid runs on XCD i mod 8)
  const JobPart jp = A.nteams % kXcds == 0 ? xcd_job_part(blockIdx.x, A.G) : JobPart{(int)blockIdx.x / A.G, (int)blockIdx.x % A.G};
  const int team = jp.job, rank = jp.part;
  const int N = A.N, width = A.max_depth + 1;
  if (tid < 64) P.tab[tid] = exp2_f64((double)tid * 0.015625);
  int passes = 0;  // passes of this team so far (the same in all its workgroups)
  bool alive = true;
  double* const sums = A.sums + (size_t)team * 2 * A.nseg;
  int* const ctr = A.ctr + team;
  const size_t slab = (size_t)A.nseg * Seg<DT>::tok;  // one R buffer
  double* const rbuf = A.rbuf + (size_t)team * 2 * slab;
  for (int b = team; b < A.B; b += A.nteams) {
    const float T = A.temperature[b];
    const bool greedy = T == 0.0f;
    const bool t_ok = temperature_ok(T);
    const float c32 = (!t_ok || greedy) ? 0.0f : c32_of(T);
    const double c64 = (!t_ok || greedy) ? 0.0 : c64_of(T);
    const long long t0 = (long long)b * N, d0 = (long long)b * (N - 1);
    int32_t* orow = A.out + (long long)b * width;
    int32_t* nrow = A.out_nodes + (long long)b * width;
    __syncthreads();
    if (tid == 0) P.bad = (t_ok && alive) ? 0 : 1;
    __syncthreads();
    // --- tree, validation and the statistics of every row
    bool lbad = false;
    // one row per thread: target rows 0..N-1, then (sampling) draft rows of nodes 1..N-1
    const int nrows = greedy ? N : 2 * N - 1;
    for (int r = tid; r < nrows && t_ok; r += kLLThreads) {
      if (r < N) {
        const int v = r;
        const int p = A.parents[t0 + v], x = A.tokens[t0 + v];
        P.par[v] = p;
        P.tok[v] = x;
        lbad |= v == 0 ? p != -1 : (p < 0 || p >= v || x < 0 || x >= A.V);
        const RowStat st = merge_row<4>(A.part + (t0 + v) * A.nchunk, A.nchunk, c32, greedy);
        lbad |= !st.ok;
        P.mt[v] = st.m;
        P.zt[v] = st.Z;
        if (greedy) P.idx[v] = st.idx;
        else lbad |= !uniform_ok(A.us[t0 + v]);
        P.kids[v] = v == 0 ? 0 : (1 << 20);  // depth
      } else {
        const int v = r - N + 1;
        lbad |= !uniform_ok(A.ua[t0 + v]);
        const RowStat sd = merge_row<4>(A.part + (A.RT + d0 + v - 1) * A.nchunk, A.nchunk, c32, false);
        lbad |= !sd.ok;
        P.md[v] = sd.m;
        P.zd[v] = sd.Z;
      }
    }
    if (lbad) P.bad = 1;
    __syncthreads();
    if (!P.bad) {
      // depths by repeated relaxation (parents precede children), in kids / rej
      int* dcur = P.kids;
      int* dnext = P.rej;
      for (int it = 0; it <= A.max_depth; ++it) {
        for (int v = tid; v < N; v += kLLThreads) dnext[v] = v == 0 ? 0 : min(dcur[P.par[v]] + 1, 1 << 20);
        __syncthreads();
        int* t = dcur;
        dcur = dnext;
        dnext = t;
      }
      for (int v = tid; v < N; v += kLLThreads)
        if (dcur[v] > A.max_depth) P.bad = 1;
    }
    __syncthreads();
    if (rank == 0)
      for (int k = tid; k < width; k += kLLThreads) {
        orow[k] = -1;
        nrow[k] = -1;
      }
    if (P.bad) {
      if (rank == 0 && tid == 0) A.num_acc[b] = -1;
      continue;
    }
    // --- greedy: follow the first child holding the argmax
    if (greedy) {
      if (rank != 0) continue;
      int v = 0, d = 0;
      for (;;) {
        if (tid == 0) P.flag = 0x7fffffff;
        __syncthreads();
        for (int c = 1 + tid; c < N; c += kLLThreads)
          if (P.par[c] == v && P.tok[c] == P.idx[v]) atomicMin(&P.flag, c);
        __syncthreads();
        const int c = P.flag;
        __syncthreads();
        if (c == 0x7fffffff) break;
        if (tid == 0) {
          orow[d] = P.tok[c];
          nrow[d] = c;
        }
        ++d;
        v = c;
      }
      if (tid == 0) {
        orow[d] = P.idx[v];
        A.num_acc[b] = d;
      }
      continue;
    }
    // --- sampling walk
    int v = 0, d = 0, nrej = 0;
    bool have_sums = false;  // the last pass's segment sums are those of the current R
    bool failed = false;
    for (;;) {
      list_children(P, N, v);
      if (tid == 0) {
        P.S[0] = 1.0;
        P.eff = 0;
        P.have_store = 0;  // a new node: no stored residual yet
      }
      // (every wave reads this state next: at a leaf, in the final pass)
      __syncthreads();
      nrej = 0;
      have_sums = false;
      int accepted = -1;
      bool pre = false;  // lg holds wave 0's logits for the next child's test
      float lg = 0.0f;
      for (int i = 0; i < P.nk; ++i) {
        const int c = P.kids[i];
        child_test<DT>(A, P, t0, d0, v, nrej, c, c64, pre, lg);
        if (P.flag) {
          accepted = c;
          break;
        }
        // rejected: the next residual's total (from the stored residual when
        // one holds the current R, the new one stored in the other buffer)
        ++nrej;
        ++passes;
        // the next child's logits, loaded while the pass runs
        pre = i + 1 < P.nk && nrej + 2 <= 64;
        if (pre && tid < 64) lg = child_logit<DT>(A, P, t0, d0, v, nrej, P.kids[i + 1], lane);
        const double* rin = P.have_store ? rbuf + (size_t)P.eff * slab : nullptr;
        double* rout = rbuf + (size_t)(1 - P.eff) * slab;
        if (!team_pass<DT>(A, P, t0, d0, v, nrej, sums + (size_t)(passes & 1) * A.nseg, ctr, passes * A.G,
                                   rank, c64, rin, nrej - 1, rout, lres)) {
          failed = true;
          break;
        }
        if (wv == 0) {
          const double S = sum_segments(sums + (size_t)(passes & 1) * A.nseg, A.nseg, lane);
          if (lane == 0) {
            if (S > 0.0) {
              P.S[nrej] = S;
            } else {  // underflow: keep r
              P.skip[nrej - 1] = 1;
              P.S[nrej] = P.S[nrej - 1];
            }
          }
        }
        __syncthreads();
        have_sums = !P.skip[nrej - 1];
        // the new residual is the current one unless its sum underflowed (r
        // kept); then the LDS part holds the discarded one, and the next pass
        // forms R from the rows again
        if (tid == 0) {
          if (have_sums) P.eff = 1 - P.eff;
          P.have_store = have_sums ? 1 : 0;
        }
        __syncthreads();
      }
      if (failed) break;
      if (accepted < 0) break;
      if (rank == 0 && tid == 0) {
        orow[d] = P.tok[accepted];
        nrow[d] = accepted;
      }
      ++d;
      v = accepted;
    }
    if (!failed && !have_sums) {
      ++passes;
      failed = !team_pass<DT>(A, P, t0, d0, v, nrej, sums + (size_t)(passes & 1) * A.nseg, ctr,
                                      passes * A.G, rank, c64, P.have_store ? rbuf + (size_t)P.eff * slab : nullptr,
                                      nrej, nullptr, lres);
    }
    if (failed) {
      // a team wait ran out of polls: this team's remaining requests report -1
      alive = false;
      if (rank == 0 && tid == 0) A.num_acc[b] = -1;
      if (rank == 0)
        for (int k = tid; k < width; k += kLLThreads) orow[k] = -1;
      continue;
    }
    if (rank == 0 && wv == 0) {
      const double* buf = sums + (size_t)(passes & 1) * A.nseg;
      const double S = sum_segments(buf, A.nseg, lane);
      const double thr = (double)A.us[t0 + v] * S;
      const int y = pick_token<DT>(A, P, t0, d0, v, nrej, buf, thr, c64, lane);
      if (lane == 0) {
        orow[d] = y;
        A.num_acc[b] = d;
      }
    }
  }
}

int lossless_segments(int V, int dt) {
  const int tok = 64 * (dt == 1 ? 8 : 4);
  return (V + tok - 1) / tok;
}

hipError_t launch_tree_lossless(int dt, const void* tgt, const void* dft, int V, const Layout& L, int max_depth,
                                const int32_t* tokens, const int32_t* parents, const float* ua, const float* us,
                                const float* temperature, const Partial* part, int nchunk, double* sums,
                                double* rbuf, int* ctr, int32_t* out, int32_t* out_nodes, int32_t* num_acc,
                                hipStream_t st) {
  if (L.B == 0) return hipSuccess;
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 1;
  const bool small = L.gamma <= kLLSmallNodes;
  const void* fn = dt == 1 ? (small ? reinterpret_cast<const void*>(&k_tree_lossless<1, true>)
                                    : reinterpret_cast<const void*>(&k_tree_lossless<1, false>))
                           : (small ? reinterpret_cast<const void*>(&k_tree_lossless<0, true>)
                                    : reinterpret_cast<const void*>(&k_tree_lossless<0, false>));
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kLLThreads, 0);
  if (e != hipSuccess) return e;
  if (per_cu < 1) return hipErrorInvalidConfiguration;
  const long long resident = (long long)per_cu * cus;
  // workgroups per request: every resident slot in use, at most 32 (a pass
  // then has up to 128 waves), and every workgroup of the launch resident at once
  const long long want = resident / L.B;
  int G = (int)(want < 1 ? 1 : (want > 32 ? 32 : want));
  if (G > resident) G = (int)resident;
  long long nteams = resident / G;
  if (nteams > L.B) nteams = L.B;
  if (nteams > kLLMaxTeams) nteams = kLLMaxTeams;  // (the workspace holds that many teams' residuals)
  LLArgs A;
  A.tgt = tgt;
  A.dft = dft;
  A.V = V;
  A.N = L.gamma;
  A.B = L.B;
  A.max_depth = max_depth;
  A.tokens = tokens;
  A.parents = parents;
  A.ua = ua;
  A.us = us;
  A.temperature = temperature;
  A.part = part;
  A.nchunk = nchunk;
  A.RT = L.RT;
  A.sums = sums;
  A.rbuf = rbuf;
  A.ctr = ctr;
  A.G = G;
  A.nteams = (int)nteams;
  A.nseg = lossless_segments(V, dt);
  A.out = out;
  A.out_nodes = out_nodes;
  A.num_acc = num_acc;
  void* args[] = {&A};
  return hipLaunchCooperativeKernel(fn, dim3((unsigned)(nteams * G)), dim3(kLLThreads), args, 0, st);
}

}  // namespace sv
