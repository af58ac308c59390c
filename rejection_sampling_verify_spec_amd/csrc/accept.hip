// accept.hip -- acceptance walk of token trees (one workgroup per request);
// chains are scanned inside the finishing kernel (finish.hip).
//
// Token trees [Primer 考点3; Edge pipeline figure]: each node is tested against
// its parent's target row with the chain rule (accept.h); the kept nodes are
// those accepted together with all their ancestors; the end node is the
// deepest kept node (lowest index among equals). Its path is emitted, and the
// final token is drawn from the residual against the draft row of its first
// child, or from its own target row when it has no children (bonus).
#include "accept.h"

namespace sv {

// ---------------------------------------------------------------------------
// Token trees: one workgroup per request, one thread per node.

constexpr int kMaxNodes = 1024;

template <int DT>
__global__ __launch_bounds__(kMaxNodes) void k_accept_tree(
    const void* __restrict__ tgt, const void* __restrict__ dft, int V, Layout L, int max_depth,
    const int32_t* __restrict__ tokens, const int32_t* __restrict__ parents, const float* __restrict__ ua,
    const float* __restrict__ us, const float* __restrict__ temperature, const Partial* __restrict__ part,
    int nchunk, int32_t* __restrict__ out, int32_t* __restrict__ out_nodes, int32_t* __restrict__ num_acc,
    SampleJob* __restrict__ jobs) {
  const int N = L.gamma;
  const int b = blockIdx.x, v = threadIdx.x;
  const long long t0 = (long long)b * N, d0 = (long long)b * (N - 1);
  const int width = max_depth + 1;
  __shared__ int s_par[kMaxNodes], s_tok[kMaxNodes], s_depth[2][kMaxNodes], s_ok[2][kMaxNodes];
  __shared__ float s_mt[kMaxNodes], s_md[kMaxNodes], s_us[kMaxNodes];
  __shared__ double s_zt[kMaxNodes], s_zd[kMaxNodes];
  __shared__ int s_idx[kMaxNodes];
  __shared__ int s_bad;
  __shared__ unsigned long long s_best;
  __shared__ int s_child;

  // the per-node inputs load in one round with the temperature
  const float T = temperature[b];
  int p = -1, x = -1;
  float uav = 0.f, usv = 0.f;
  if (v < N) {
    p = parents[t0 + v];
    x = tokens[t0 + v];
    usv = us[t0 + v];
    if (v >= 1) uav = ua[t0 + v];
  }
  const bool greedy = T == 0.0f;
  const bool t_ok = temperature_ok(T);
  const float c32 = (!t_ok || greedy) ? 0.0f : c32_of(T);
  if (v == 0) { s_bad = t_ok ? 0 : 1; s_best = 0ull; s_child = 0x7fffffff; }
  __syncthreads();

  bool lbad = false;
  RowStat sd{0.f, 0.0, -1, true};
  float lt = 0.f, ld = 0.f;  // the node's logit in its parent's target row and in its draft row
  if (v < N && t_ok) {
    s_par[v] = p;
    s_tok[v] = x;
    if (v == 0) lbad |= p != -1;
    else lbad |= p < 0 || p >= v || x < 0 || x >= V;
    // the logits at x load while the partials are merged
    if (!greedy && v >= 1 && p >= 0 && p < v && x >= 0 && x < V) {
      lt = Elem<DT>::at(tgt, (t0 + p) * (long long)V + x);
      ld = Elem<DT>::at(dft, (d0 + v - 1) * (long long)V + x);
    }
    RowStat st;
    merge_rows2(part + (t0 + v) * nchunk, greedy, part + (L.RT + d0 + v - 1) * nchunk, !greedy && v >= 1, nchunk,
                c32, st, sd);
    lbad |= !st.ok;
    s_mt[v] = st.m;
    s_zt[v] = st.Z;
    s_idx[v] = st.idx;
    if (!greedy) {
      lbad |= !uniform_ok(usv);
      s_us[v] = usv;
      if (v >= 1) {
        lbad |= !uniform_ok(uav);
        lbad |= !sd.ok;
        s_md[v] = sd.m;
        s_zd[v] = sd.Z;
      }
    }
    s_depth[0][v] = v == 0 ? 0 : (1 << 20);
  }
  if (lbad) s_bad = 1;
  __syncthreads();
  const bool bad0 = s_bad != 0;

  // depths by repeated relaxation (parents precede children)
  int cur = 0;
  if (!bad0) {
    for (int it = 0; it <= max_depth; ++it) {
      if (v < N) s_depth[cur ^ 1][v] = v == 0 ? 0 : min(s_depth[cur][s_par[v]] + 1, 1 << 20);
      __syncthreads();
      cur ^= 1;
    }
    if (v < N && s_depth[cur][v] > max_depth) s_bad = 1;
  }
  __syncthreads();
  int32_t* orow = out + (long long)b * width;
  int32_t* nrow = out_nodes + (long long)b * width;
  if (s_bad) {
    for (int k = v; k < width; k += blockDim.x) { orow[k] = -1; nrow[k] = -1; }
    if (v == 0) { num_acc[b] = -1; jobs[b].kind = JOB_NONE; }
    return;
  }
  const int depth = v < N ? s_depth[cur][v] : 0;

  // acceptance per node against the parent's target row
  int acc = 0;
  if (v >= 1 && v < N) {
    if (greedy) {
      acc = x == s_idx[p];
    } else {
      const double pt = exp2_f64(((double)lt - (double)s_mt[p]) * (double)c32) / s_zt[p];
      const double pd = exp2_f64(((double)ld - (double)sd.m) * (double)c32) / sd.Z;
      acc = (double)uav * pd < pt;
    }
  }
  int oc = 0;
  if (v < N) s_ok[0][v] = v == 0 ? 1 : acc;
  __syncthreads();
  for (int it = 0; it < max_depth; ++it) {
    if (v < N) s_ok[oc ^ 1][v] = v == 0 ? 1 : (acc && s_ok[oc][s_par[v]]);
    __syncthreads();
    oc ^= 1;
  }
  // end node: deepest kept node, lowest index on ties
  if (v < N && s_ok[oc][v]) {
    unsigned long long key = ((unsigned long long)depth << 32) | (unsigned)(0x7fffffff - v);
    atomicMax(&s_best, key);
  }
  __syncthreads();
  const int e = 0x7fffffff - (int)(unsigned)(s_best & 0xffffffffull);
  const int de = (int)(s_best >> 32);
  if (v >= 1 && v < N && s_par[v] == e) atomicMin(&s_child, v);
  __syncthreads();
  if (v == 0) {
    for (int k = 0; k < width; ++k) { orow[k] = -1; nrow[k] = -1; }
    int w = e;
    for (int k = de - 1; k >= 0; --k) {
      orow[k] = s_tok[w];
      nrow[k] = w;
      w = s_par[w];
    }
    num_acc[b] = de;
    SampleJob J;
    J.pos = de;
    J.c32 = c32;
    J.skip = 0ull;
    J.chunk_tiles = 0;
    J.pad = 0;
    J.slow = 0.0;
    J.trow = t0 + e;
    J.drow = 0;
    J.rho = 0.0;
    J.md = 0.0f;
    J.mt = s_mt[e];
    if (greedy) {
      orow[de] = s_idx[e];
      J.kind = JOB_NONE;
      J.c64 = 0.0;
      J.u = 0.0f;
    } else {
      J.c64 = c64_of(T);
      J.u = s_us[e];
      const int c = s_child;
      if (c == 0x7fffffff) {
        J.kind = JOB_BONUS;
      } else {
        J.kind = JOB_RESIDUAL;
        J.drow = d0 + c - 1;
        J.md = s_md[c];
        J.rho = s_zt[e] / s_zd[c];
      }
    }
    jobs[b] = J;
  }
}

hipError_t launch_accept_tree(int dt, const void* tgt, const void* dft, int V, const Layout& L, int max_depth,
                              const int32_t* tokens, const int32_t* parents, const float* ua, const float* us,
                              const float* temperature, const Partial* part, int nchunk, int32_t* out,
                              int32_t* out_nodes, int32_t* num_acc, SampleJob* jobs, hipStream_t st) {
  if (L.B == 0) return hipSuccess;
  int threads = ((L.gamma + 63) / 64) * 64;
  if (dt == 1)
    hipLaunchKernelGGL(k_accept_tree<1>, dim3(L.B), dim3(threads), 0, st, tgt, dft, V, L, max_depth, tokens, parents,
                       ua, us, temperature, part, nchunk, out, out_nodes, num_acc, jobs);
  else
    hipLaunchKernelGGL(k_accept_tree<0>, dim3(L.B), dim3(threads), 0, st, tgt, dft, V, L, max_depth, tokens, parents,
                       ua, us, temperature, part, nchunk, out, out_nodes, num_acc, jobs);
  return hipGetLastError();
}

}  // namespace sv
