// row_stats.hip -- streaming per-row softmax statistics (the HBM-bound pass).
//
// For every logit row the verify step reads (all target rows; draft rows of
// requests with T > 0) one workgroup per (row, chunk) computes, in one read of
// the chunk:
//   T > 0 : m = max x and s = sum 2^{(x - m) c} with c = log2(e)/T, i.e. the
//           max and sum of exp((x - m)/T) of the temperature softmax
//           [Edge page, scheduler section: per-row max, then the sum of
//           exp((l - max)/T)];
//   T == 0: m = max x and the lowest index holding it (greedy argmax), plus a
//           NaN/+inf flag.
// Per-thread work is organised in groups of kU 16-byte vectors (32 bf16 or 16
// fp32 values). Inside a group the exponent argument is fma(x, c, -K) with
// K = fl(m c) an exact fp32 number, so every term of the group shares one
// exactly known offset; the thread statistic is converted to the offset m c
// once at the end with the exact remainder r = m c - K (error-free product).
// The remainder is at most half an ulp of K, so the trick needs |K| < 2^22
// (then |r| <= 1/4 and no term can overflow); a chunk where some |m c| is
// larger (tiny temperatures, huge logits) is recomputed with (x - m) c.
#include "sv_internal.h"

#include <float.h>

namespace sv {

__device__ __forceinline__ long long request_of_row(const Layout& L, long long r, bool draft) {
  switch (L.mode) {
    case LAYOUT_DENSE:
      return draft ? r / L.gamma : r / (L.gamma + 1);
    case LAYOUT_TREE:
      return draft ? r / (L.gamma - 1) : r / L.gamma;
    case LAYOUT_RAGGED: {
      // largest b in [0, B) with key(b) <= r; key(b) = cu[b] (+ b for target rows)
      int lo = 0, hi = L.B - 1;
      while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        long long key = (long long)L.cu[mid] + (draft ? 0 : mid);
        if (key <= r) lo = mid; else hi = mid - 1;
      }
      return lo;
    }
    default:
      return r;
  }
}

// Merge two (max, sum 2^{(x-max)c}) statistics.
__device__ __forceinline__ void merge_ms(float& m, float& s, float m2, float s2, float c) {
  float M = fmaxf(m, m2);
  if (M == -INFINITY) {
    s = s + s2;  // both empty (0) or NaN-flagged
  } else {
    s = s * exp2_f32((m - M) * c) + s2 * exp2_f32((m2 - M) * c);
  }
  m = M;
}

// Logits are read exactly once here: nontemporal 16-byte loads (streaming
// hint) measured ~10% faster than plain loads for this pass on MI355X.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 stream_load(const uint4* p) {
  u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// A full group: kU unpredicated 16-byte loads per thread (every index < v1).
__device__ __forceinline__ void load_group_full(const uint4* vp, int vb, int tid, uint4* w) {
#pragma unroll
  for (int u = 0; u < kU; ++u) w[u] = stream_load(vp + vb + u * kTPB + tid);
}

// The last, partial group of a chunk: out-of-range vectors read a valid
// address and are replaced by -inf (they add nothing to max or sum).
template <int DT>
__device__ __forceinline__ void load_group_tail(const uint4* vp, int vb, int v1, int tid, uint4* w) {
  const uint32_t ni = DT == 1 ? 0xff80ff80u : 0xff800000u;
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    int v = vb + u * kTPB + tid;
    uint4 t = stream_load(vp + min(v, v1 - 1));
    bool in = v < v1;
    w[u] = make_uint4(in ? t.x : ni, in ? t.y : ni, in ? t.z : ni, in ? t.w : ni);
  }
}

// Visit the 16-byte vectors [v0, v1) of a chunk in groups; f(w, vb) gets each group.
template <int DT, typename F>
__device__ __forceinline__ void for_each_group(const uint4* vp, int v0, int v1, int tid, F f) {
  int vb = v0;
  for (; vb + kU * kTPB <= v1; vb += kU * kTPB) {
    uint4 w[kU];
    load_group_full(vp, vb, tid, w);
    f(w, vb);
  }
  if (vb < v1) {
    uint4 w[kU];
    load_group_tail<DT>(vp, vb, v1, tid, w);
    f(w, vb);
  }
}

// One group of n values into the thread statistic (m, K, s): s = sum 2^{x c - K}.
template <int N>
__device__ __forceinline__ void group_update(float& m, float& K, float& s, bool& ovf, const float* x, float c) {
  float gm = x[0];
#pragma unroll
  for (int i = 1; i < N; ++i) gm = fmaxf(gm, x[i]);
  float mn = fmaxf(m, gm);
  float Kn = mn == -INFINITY ? 0.0f : mn * c;
  ovf |= !(fabsf(Kn) <= 0x1p22f);  // also catches +inf maxima
  float f = m == -INFINITY ? 0.0f : exp2_f32(K - Kn);
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
  for (int i = 0; i < N; i += 4) {
    a0 += exp2_f32(__builtin_fmaf(x[i], c, -Kn));
    if (i + 1 < N) a1 += exp2_f32(__builtin_fmaf(x[i + 1], c, -Kn));
    if (i + 2 < N) a2 += exp2_f32(__builtin_fmaf(x[i + 2], c, -Kn));
    if (i + 3 < N) a3 += exp2_f32(__builtin_fmaf(x[i + 3], c, -Kn));
  }
  s = __builtin_fmaf(s, f, (a0 + a1) + (a2 + a3));
  m = mn;
  K = Kn;
}

// Block-wide merge of (m, s) in a fixed order; result valid in thread 0.
__device__ __forceinline__ void block_merge_ms(float& m, float& s, float c, float* sm, float* ss) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    float m2 = __shfl_xor(m, off, 64), s2 = __shfl_xor(s, off, 64);
    merge_ms(m, s, m2, s2, c);
  }
  if (lane == 0) { sm[wv] = m; ss[wv] = s; }
  __syncthreads();
  if (threadIdx.x == 0) {
    m = sm[0]; s = ss[0];
    for (int w = 1; w < kTPB / 64; ++w) merge_ms(m, s, sm[w], ss[w], c);
  }
}

template <int DT>
__device__ void stats_sampling(const void* rowp, const RowSplit& sp, int v0, int v1, bool do_head, bool do_tail,
                               float c, Partial* out) {
  using E = Elem<DT>;
  constexpr int EPV = E::kPerVec;
  constexpr int G = kU * EPV;
  const int tid = threadIdx.x;
  const uint4* vp = reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(rowp) +
                                                   (size_t)sp.head * sizeof(typename E::T));
  float m = -INFINITY, K = 0.f, s = 0.f;
  bool ovf = false;
  for_each_group<DT>(vp, v0, v1, tid, [&](const uint4* w, int) {
    float x[G];
#pragma unroll
    for (int u = 0; u < kU; ++u) unpack<DT>(w[u], x + u * EPV);
    group_update<G>(m, K, s, ovf, x, c);
  });
  if (do_head && tid < sp.head) {
    float x1 = E::at(rowp, tid);
    group_update<1>(m, K, s, ovf, &x1, c);
  }
  if (do_tail && tid < sp.tail) {
    float x1 = E::at(rowp, (long long)sp.head + (long long)sp.nvec * EPV + tid);
    group_update<1>(m, K, s, ovf, &x1, c);
  }
  // to the offset m c: 2^{x c - K} = 2^{(x - m) c} 2^{m c - K}
  if (m != -INFINITY && !ovf) s *= exp2_f32(-__builtin_fmaf(m, c, -K));

  __shared__ float sm[kTPB / 64], ss[kTPB / 64];
  __shared__ int sovf;
  if (tid == 0) sovf = 0;
  __syncthreads();
  if (ovf) sovf = 1;
  __syncthreads();
  const bool any_ovf = sovf != 0;
  if (!any_ovf) {
    block_merge_ms(m, s, c, sm, ss);
    if (tid == 0) *out = Partial{m, s, -1, 1};
    return;
  }
  // Rare path: |max * c| >= 2^22 somewhere in the chunk. Exact maximum first, then sum 2^{(x-M)c}.
  float mm = m;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mm = fmaxf(mm, __shfl_xor(mm, off, 64));
  __syncthreads();
  if ((tid & 63) == 0) sm[tid >> 6] = mm;
  __syncthreads();
  float M = sm[0];
  for (int w = 1; w < kTPB / 64; ++w) M = fmaxf(M, sm[w]);
  float acc = 0.f;
  for_each_group<DT>(vp, v0, v1, tid, [&](const uint4* w, int) {
    float x[G];
#pragma unroll
    for (int u = 0; u < kU; ++u) unpack<DT>(w[u], x + u * EPV);
#pragma unroll
    for (int i = 0; i < G; ++i) acc += exp2_f32((x[i] - M) * c);
  });
  if (do_head && tid < sp.head) acc += exp2_f32((E::at(rowp, tid) - M) * c);
  if (do_tail && tid < sp.tail)
    acc += exp2_f32((E::at(rowp, (long long)sp.head + (long long)sp.nvec * EPV + tid) - M) * c);
  acc = wave_reduce(acc, [](float a, float b) { return a + b; });
  __syncthreads();
  if ((tid & 63) == 0) ss[tid >> 6] = acc;
  __syncthreads();
  if (tid == 0) {
    float t = ss[0];
    for (int w = 1; w < kTPB / 64; ++w) t += ss[w];
    if (M == INFINITY) t = __uint_as_float(0x7fc00000u);
    *out = Partial{M, t, -1, 1};
  }
}

typedef unsigned short us2_t __attribute__((ext_vector_type(2)));

template <int DT>
__device__ void stats_greedy(const void* rowp, const RowSplit& sp, int v0, int v1, bool do_head, bool do_tail,
                             Partial* out) {
  using E = Elem<DT>;
  constexpr int EPV = E::kPerVec;
  constexpr int G = kU * EPV;
  const int tid = threadIdx.x;
  const uint4* vp = reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(rowp) +
                                                   (size_t)sp.head * sizeof(typename E::T));
  float m = -INFINITY;
  int idx = -1;
  bool nan_seen = false;
  us2_t mag2 = {0, 0};
  uint32_t mag = 0;
  for_each_group<DT>(vp, v0, v1, tid, [&](const uint4* w, int vb) {
    float x[G];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      unpack<DT>(w[u], x + u * EPV);
      uint32_t ws[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (DT == 1) {
          mag2 = __builtin_elementwise_max(mag2, __builtin_bit_cast(us2_t, ws[q] & 0x7fff7fffu));
        } else {
          mag = max(mag, ws[q] & 0x7fffffffu);
        }
      }
    }
    float gm = x[0];
#pragma unroll
    for (int i = 1; i < G; ++i) gm = fmaxf(gm, x[i]);
    if (gm > m) {
      int gi = 0;
#pragma unroll
      for (int u = kU - 1; u >= 0; --u)
#pragma unroll
        for (int e = EPV - 1; e >= 0; --e)
          gi = x[u * EPV + e] == gm ? sp.head + (vb + u * kTPB + tid) * EPV + e : gi;
      m = gm;
      idx = gi;
    }
  });
  auto scalar = [&](long long j) {
    float x1 = E::at(rowp, j);
    nan_seen |= x1 != x1;
    // head elements precede every vector element: a tie goes to the lower index
    if (x1 > m || (x1 == m && (unsigned)j < (unsigned)idx)) { m = x1; idx = (int)j; }
  };
  if (do_head && tid < sp.head) scalar(tid);
  if (do_tail && tid < sp.tail) scalar((long long)sp.head + (long long)sp.nvec * EPV + tid);
  if (DT == 1) nan_seen |= mag2.x > 0x7f80u || mag2.y > 0x7f80u;
  else nan_seen |= mag > 0x7f800000u;

  // block argmax: larger value, then lower index
  const int lane = tid & 63, wv = tid >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    float m2 = __shfl_xor(m, off, 64);
    int i2 = __shfl_xor(idx, off, 64);
    if (m2 > m || (m2 == m && (unsigned)i2 < (unsigned)idx)) { m = m2; idx = i2; }
  }
  __shared__ float sm[kTPB / 64];
  __shared__ int si[kTPB / 64];
  __shared__ int snan;
  if (tid == 0) snan = 0;
  __syncthreads();
  if (nan_seen) snan = 1;
  if (lane == 0) { sm[wv] = m; si[wv] = idx; }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < kTPB / 64; ++w)
      if (sm[w] > m || (sm[w] == m && (unsigned)si[w] < (unsigned)idx)) { m = sm[w]; idx = si[w]; }
    bool bad = snan != 0 || m == INFINITY;
    *out = Partial{m, bad ? __uint_as_float(0x7fc00000u) : 0.0f, idx, 1};
  }
}

template <int DT>
__global__ __launch_bounds__(kTPB) void k_row_stats(const void* __restrict__ tgt, const void* __restrict__ dft,
                                                    int V, Layout L, const float* __restrict__ temperature,
                                                    int chunk_vecs, int nchunk, Partial* __restrict__ part) {
  using E = Elem<DT>;
  const long long item = blockIdx.x;
  const long long row = item / nchunk;
  const int chunk = (int)(item - row * nchunk);
  const bool draft = row >= L.RT;
  const long long r = draft ? row - L.RT : row;
  long long b = request_of_row(L, r, draft);
  if (b < 0) b = 0;
  if (b >= L.B) b = L.B - 1;
  const float T = temperature[b];
  if (!temperature_ok(T) || (draft && T == 0.0f)) return;
  const void* rowp = reinterpret_cast<const char*>(draft ? dft : tgt) + (size_t)r * (size_t)V * sizeof(typename E::T);
  const RowSplit sp = split_row<DT>(rowp, V);
  const int v0 = chunk * chunk_vecs;
  const int v1 = min(sp.nvec, v0 + chunk_vecs);
  const int last = max(0, (sp.nvec + chunk_vecs - 1) / chunk_vecs - 1);
  Partial* out = part + item;
  if (T > 0.0f)
    stats_sampling<DT>(rowp, sp, v0, v1, chunk == 0, chunk == last, c32_of(T), out);
  else
    stats_greedy<DT>(rowp, sp, v0, v1, chunk == 0, chunk == last, out);
}

hipError_t launch_row_stats(int dt, const void* tgt, const void* dft, int V, const Layout& L,
                            const float* temperature, int chunk_vecs, int nchunk, Partial* part, hipStream_t st) {
  long long grid = (L.RT + L.RD) * (long long)nchunk;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  if (dt == 1)
    hipLaunchKernelGGL(k_row_stats<1>, dim3((unsigned)grid), dim3(kTPB), 0, st, tgt, dft, V, L, temperature,
                       chunk_vecs, nchunk, part);
  else
    hipLaunchKernelGGL(k_row_stats<0>, dim3((unsigned)grid), dim3(kTPB), 0, st, tgt, dft, V, L, temperature,
                       chunk_vecs, nchunk, part);
  return hipGetLastError();
}

// Per-row finalisation for the statistics entry point.
__global__ __launch_bounds__(64) void k_stats_finalize(const Partial* __restrict__ part, int nchunk, int rows,
                                                       const float* __restrict__ temperature,
                                                       float* __restrict__ out_max, float* __restrict__ out_logz,
                                                       int32_t* __restrict__ out_argmax) {
  int r = blockIdx.x * 64 + threadIdx.x;
  if (r >= rows) return;
  float T = temperature[r];
  const float qnan = __uint_as_float(0x7fc00000u);
  if (!temperature_ok(T)) {
    out_max[r] = qnan; out_logz[r] = qnan; out_argmax[r] = -1;
    return;
  }
  const Partial* p = part + (long long)r * nchunk;
  float M = -INFINITY;
  int idx = -1;
  bool nan = false;
  for (int k = 0; k < nchunk; ++k) {
    Partial q = p[k];
    nan |= q.s != q.s;
    if (q.m > M) { M = q.m; idx = q.idx; }
  }
  bool ok = !nan && M > -INFINITY && M < INFINITY;
  if (T == 0.0f) {
    out_max[r] = ok ? M : qnan;
    out_logz[r] = qnan;
    out_argmax[r] = ok ? idx : -1;
    return;
  }
  double c = (double)c32_of(T), Z = 0.0;
  for (int k = 0; k < nchunk; ++k)
    if (p[k].m > -INFINITY) Z += (double)p[k].s * exp2_f64(((double)p[k].m - (double)M) * c);
  ok = ok && Z > 0.0 && Z < 1e308;
  out_max[r] = ok ? M : qnan;
  out_logz[r] = ok ? (float)log(Z) : qnan;
  out_argmax[r] = -1;
}

hipError_t launch_stats_finalize(const Partial* part, int nchunk, int rows, const float* temperature,
                                 float* out_max, float* out_logz, int32_t* out_argmax, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(k_stats_finalize, dim3((rows + 63) / 64), dim3(64), 0, st, part, nchunk, rows, temperature,
                     out_max, out_logz, out_argmax);
  return hipGetLastError();
}

}  // namespace sv
