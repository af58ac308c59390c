// stream.h -- per-(row, chunk) softmax statistics, the HBM-bound streaming
// pass of a verify call (device code of the row-statistics kernel).
//
// One workgroup computes, in one read of its chunk:
//   T > 0 : m = max x and s = sum 2^{(x - m) c} with c = log2(e)/T, i.e. the
//           max and sum of exp((x - m)/T) of the temperature softmax
//           [Edge page, scheduler section: per-row max, then the sum of
//           exp((l - max)/T)];
//   T == 0: m = max x and the lowest index holding it (greedy argmax), plus a
//           NaN/+inf flag.
// Per-thread work is organised in groups of kU 16-byte vectors (32 bf16 or 16
// fp32 values). Inside a group the exponent argument is
// fma(x, c, -K) with K = fl(m c) an exact fp32 number, so every term of the
// group shares one exactly known offset; the thread statistic is converted to
// the offset m c once at the end with the exact remainder r = m c - K
// (error-free product). The remainder is at most half an ulp of K, so the
// trick needs |K| < 2^22 (then |r| <= 1/4 and no term can overflow); a chunk
// where some |m c| is larger (tiny temperatures, huge logits) is recomputed
// with (x - m) c.
#pragma once

#include "sv_internal.h"

namespace sv {

// Workgroup barrier for exchanges through LDS only: waits for the caller's LDS
// accesses, not for its outstanding global loads, so that loads of the next
// chunk issued into LDS (or registers) stay in flight across it. The signal
// fences keep the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void wg_sync() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt not waited for
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
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

// Logits are read exactly once here: nontemporal 16-byte loads (streaming hint).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 stream_load(const uint4* p) {
  u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// n full groups: kU unpredicated 16-byte loads per thread and group (every index < v1).
template <int NG>
__device__ __forceinline__ void load_groups_full(const uint4* vp, int vb, int tid, uint4* w) {
#pragma unroll
  for (int u = 0; u < NG * kU; ++u) w[u] = stream_load(vp + vb + u * kTPB + tid);
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

// Visit the 16-byte vectors [v0, v1) of a chunk in groups; f(w, vb) gets each
// group. NB full groups are loaded at once (then the rest one at a time): more
// bytes in flight per thread, at the price of the registers that hold them.
template <int DT, int NB = 1, typename F>
__device__ __forceinline__ void for_each_group(const uint4* vp, int v0, int v1, int tid, F f) {
  int vb = v0;
  if constexpr (NB > 1) {  // NB groups' loads in flight at once
    for (; vb + NB * kU * kTPB <= v1; vb += NB * kU * kTPB) {
      uint4 w[NB * kU];
      load_groups_full<NB>(vp, vb, tid, w);
#pragma unroll
      for (int g = 0; g < NB; ++g) f(w + g * kU, vb + g * kU * kTPB);
    }
  }
  for (; vb + kU * kTPB <= v1; vb += kU * kTPB) {
    uint4 w[kU];
    load_groups_full<1>(vp, vb, tid, w);
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

// Wave-wide merge of (m, s): the wave maximum, each thread's sum rescaled to
// it once, then the wave sum (an empty thread has s = 0, a NaN-flagged one
// keeps its NaN); the result in every lane.
__device__ __forceinline__ void wave_merge_ms(float& m, float& s, float c) {
  float M = m;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  float t = M == -INFINITY || m == M ? s : s * exp2_f32((m - M) * c);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) t += __shfl_xor(t, off, 64);
  m = M;
  s = t;
}

// Rare path of the sampling statistics: |max * c| >= 2^22 somewhere in the
// chunk. Exact maximum first (from the per-thread maxima m), then the chunk is
// read again and sum 2^{(x-M)c} taken directly. Thread 0 publishes.
template <int DT>
__device__ void stats_sampling_wide(const void* rowp, const RowSplit& sp, int v0, int v1,
                                                              bool do_head, bool do_tail, float c, float m,
                                                              Partial* out, float* sm, float* ss) {
  using E = Elem<DT>;
  constexpr int EPV = E::kPerVec;
  constexpr int G = kU * EPV;
  const int tid = threadIdx.x;
  const uint4* vp = reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(rowp) +
                                                   (size_t)sp.head * sizeof(typename E::T));
  float mm = m;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mm = fmaxf(mm, __shfl_xor(mm, off, 64));
  if ((tid & 63) == 0) sm[tid >> 6] = mm;
  wg_sync();
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
  if ((tid & 63) == 0) ss[tid >> 6] = acc;
  wg_sync();
  if (tid == 0) {
    float t = ss[0];
    for (int w = 1; w < kTPB / 64; ++w) t += ss[w];
    if (M == INFINITY) t = __uint_as_float(0x7fc00000u);
    publish_partial(out, sampling_partial(M, t));
  }
  wg_sync();  // sm / ss are reused by the workgroup's next chunk
}

// Finish of the sampling statistics from per-thread (m, K, s): the scalar head
// and tail, the offset correction, the fixed-order block merge; thread 0
// publishes.
template <int DT>
__device__ __forceinline__ void sampling_finish(const void* rowp, const RowSplit& sp, int v0, int v1, bool do_head,
                                                bool do_tail, float c, float m, float K, float s, bool ovf,
                                                Partial* out) {
  using E = Elem<DT>;
  constexpr int EPV = E::kPerVec;
  const int tid = threadIdx.x;
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

  // the wave merges and the waves' overflow flags, exchanged over one barrier;
  // then thread 0 merges the waves in a fixed order and publishes
  __shared__ float sm[kTPB / 64], ss[kTPB / 64];
  __shared__ int so[kTPB / 64];
  const int lane = tid & 63, wv = tid >> 6;
  wave_merge_ms(m, s, c);
  const bool wovf = __ballot(ovf) != 0ull;
  if (lane == 0) {
    sm[wv] = m;
    ss[wv] = s;
    so[wv] = wovf;
  }
  wg_sync();
  int any_ovf = 0;
#pragma unroll
  for (int k = 0; k < kTPB / 64; ++k) any_ovf |= so[k];
  if (!any_ovf) {
    if (tid == 0) {
      m = sm[0];
      s = ss[0];
      for (int w = 1; w < kTPB / 64; ++w) merge_ms(m, s, sm[w], ss[w], c);
      publish_partial(out, sampling_partial(m, s));
    }
    return;
  }
  // (m is now the wave maximum: the wide path only needs the block maximum)
  stats_sampling_wide<DT>(rowp, sp, v0, v1, do_head, do_tail, c, m, out, sm, ss);
}

// Statistics of vectors [v0, v1) of a row (plus the scalar head / tail when
// asked) at temperature coefficient c; thread 0 publishes the partial.
template <int DT, int NB>
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
  for_each_group<DT, NB>(vp, v0, v1, tid, [&](const uint4* w, int) {
    float x[G];
#pragma unroll
    for (int u = 0; u < kU; ++u) unpack<DT>(w[u], x + u * EPV);
    group_update<G>(m, K, s, ovf, x, c);
  });
  sampling_finish<DT>(rowp, sp, v0, v1, do_head, do_tail, c, m, K, s, ovf, out);
}

typedef unsigned short us2_t __attribute__((ext_vector_type(2)));

// Greedy statistics of one group of kU vectors starting at vector vb (thread
// tid holds vectors vb + u*kTPB + tid): running maximum, lowest index holding
// it, and the largest magnitude bits (NaN / +inf detection).
template <int DT>
__device__ __forceinline__ void greedy_group(const uint4* w, int vb, int head, int tid, float& m, int& idx,
                                             us2_t& mag2, uint32_t& mag) {
  constexpr int EPV = Elem<DT>::kPerVec;
  constexpr int G = kU * EPV;
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
        gi = x[u * EPV + e] == gm ? head + (vb + u * kTPB + tid) * EPV + e : gi;
    m = gm;
    idx = gi;
  }
}

// Finish of the greedy statistics: the scalar head and tail, the block argmax
// (larger value, then lower index); thread 0 publishes.
template <int DT>
__device__ __forceinline__ void greedy_finish(const void* rowp, const RowSplit& sp, bool do_head, bool do_tail,
                                              float m, int idx, us2_t mag2, uint32_t mag, Partial* out) {
  using E = Elem<DT>;
  constexpr int EPV = E::kPerVec;
  const int tid = threadIdx.x;
  bool nan_seen = false;
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

  const int lane = tid & 63, wv = tid >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    float m2 = __shfl_xor(m, off, 64);
    int i2 = __shfl_xor(idx, off, 64);
    if (m2 > m || (m2 == m && (unsigned)i2 < (unsigned)idx)) { m = m2; idx = i2; }
  }
  // the waves' results and NaN flags over one barrier; thread 0 merges
  __shared__ float sm[kTPB / 64];
  __shared__ int si[kTPB / 64], sn[kTPB / 64];
  const bool wnan = __ballot(nan_seen) != 0ull;
  if (lane == 0) { sm[wv] = m; si[wv] = idx; sn[wv] = wnan; }
  wg_sync();
  if (tid == 0) {
    bool any_nan = sn[0] != 0;
    for (int w = 1; w < kTPB / 64; ++w) {
      any_nan |= sn[w] != 0;
      if (sm[w] > m || (sm[w] == m && (unsigned)si[w] < (unsigned)idx)) { m = sm[w]; idx = si[w]; }
    }
    publish_partial(out, greedy_partial(m, idx, any_nan || m == INFINITY));
  }
}

template <int DT, int NB>
__device__ void stats_greedy(const void* rowp, const RowSplit& sp, int v0, int v1, bool do_head, bool do_tail,
                             Partial* out) {
  using E = Elem<DT>;
  const int tid = threadIdx.x;
  const uint4* vp = reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(rowp) +
                                                   (size_t)sp.head * sizeof(typename E::T));
  float m = -INFINITY;
  int idx = -1;
  us2_t mag2 = {0, 0};
  uint32_t mag = 0;
  for_each_group<DT, NB>(vp, v0, v1, tid,
                         [&](const uint4* w, int vb) { greedy_group<DT>(w, vb, sp.head, tid, m, idx, mag2, mag); });
  greedy_finish<DT>(rowp, sp, do_head, do_tail, m, idx, mag2, mag, out);
}

// Statistics of chunk `chunk` of one row (the chunk covers 16-byte vectors
// [chunk * chunk_vecs, (chunk + 1) * chunk_vecs) of the row's vector part;
// chunk 0 also takes the scalar head, the last chunk the scalar tail).
template <int DT, int NB = 1>
__device__ __forceinline__ void row_chunk_stats(const void* rowp, int V, int chunk, int chunk_vecs, float T,
                                                Partial* out) {
  const RowSplit sp = split_row<DT>(rowp, V);
  const int v0 = chunk * chunk_vecs;
  const int v1 = min(sp.nvec, v0 + chunk_vecs);
  const int last = max(0, (sp.nvec + chunk_vecs - 1) / chunk_vecs - 1);
  if (T > 0.0f)
    stats_sampling<DT, NB>(rowp, sp, v0, v1, chunk == 0, chunk == last, c32_of(T), out);
  else
    stats_greedy<DT, NB>(rowp, sp, v0, v1, chunk == 0, chunk == last, out);
}

}  // namespace sv
