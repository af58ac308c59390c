// cache.hip -- the KV-cache steps around verification.
//
// Commit [Edge 环形上下文与注意力沉淀机制; Edge C++ 环形 KV 缓存管理内核实现]:
// the target pass over a request's pending token and gamma drafts produces
// keys and values for positions P .. P+gamma; after verification the first
// n+1 of them (the pending token and the n accepted drafts) are kept
// [Primer 考点1, 考点4]. They are copied from the caller's staging buffer into
// the cache at Slot(pos); rejected positions are never written, so the ring
// keeps every position of the window that precedes them. Writing all gamma+1
// positions into the ring and moving the length back afterwards would
// overwrite up to gamma-n live window positions once the ring has wrapped.
//
// One workgroup per (request, block of rows) copies the kept positions of those
// rows with 16-, 4- or 1-byte accesses: consecutive positions sit in adjacent
// ring slots, so each row is written as runs of (n+1)*E bytes (two runs where
// the ring wraps) instead of single rows of E bytes at a stride of (S+W)*E.
//
// Draft window [Window 窗口数学; Window block table 的裁剪方式]: one wave per
// request computes its windowed length and gathers its block-table row from
// the start block into the windowed table, zero past the blocks needed.
#include "cache.h"

namespace svc {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;         // accesses in flight per thread and tensor
constexpr int kBlockAccesses = 512;  // accesses per workgroup and tensor, at most (measured best)
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));  // one 16-byte access

template <typename VT>
__global__ __launch_bounds__(kThreads) void k_kv_commit(char* __restrict__ kc, char* __restrict__ vc,
                                                        const char* __restrict__ kn, const char* __restrict__ vn,
                                                        const int32_t* __restrict__ len_in,
                                                        const int32_t* __restrict__ nacc,
                                                        int32_t* __restrict__ len_out, int gamma, int R, long long E,
                                                        int S, int W, int rpb, int nchunk) {
  const long long blk = blockIdx.x;
  const int c = (int)(blk % nchunk);
  const long long b = blk / nchunk;
  const int P = len_in[b];
  const int n = nacc[b];
  const bool ok = n >= 0 && n <= gamma && P >= 0 && (long long)P + n + 1 <= 0x7fffffffLL;
  if (c == 0 && threadIdx.x == 0) len_out[b] = ok ? P + n + 1 : P;
  if (!ok) return;
  // kept positions P + j0 .. P + n: a later kept position takes the ring slot of
  // any earlier one W positions before it
  int j0 = 0;
  while (j0 <= n && (long long)P + j0 >= S && (long long)P + j0 + W <= (long long)P + n) ++j0;
  const int np = n + 1 - j0;
  const long long cap = (long long)S + W;
  const int r0 = c * rpb;
  const int nr = min(rpb, R - r0);
  const int vpr = (int)(E / (long long)sizeof(VT));
  const int per_row = np * vpr;
  const int total = nr * per_row;
  const long long row_stride = cap * E;
  for (int base = threadIdx.x; base < total; base += kThreads * kUnroll) {
    VT a[kUnroll], v[kUnroll];
    long long dst[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int i = base + u * kThreads;
      if (i < total) {
        const int r = i / per_row;
        const int rem = i - r * per_row;
        const int jj = rem / vpr;
        const int w = rem - jj * vpr;
        const int j = j0 + jj;
        const long long src = ((b * (gamma + 1) + j) * R + r0 + r) * E + (long long)w * (long long)sizeof(VT);
        a[u] = *reinterpret_cast<const VT*>(kn + src);
        v[u] = *reinterpret_cast<const VT*>(vn + src);
        dst[u] = (b * R + r0 + r) * row_stride + ring_slot((long long)P + j, S, W) * E + (long long)w * (long long)sizeof(VT);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int i = base + u * kThreads;
      if (i < total) {
        *reinterpret_cast<VT*>(kc + dst[u]) = a[u];
        *reinterpret_cast<VT*>(vc + dst[u]) = v[u];
      }
    }
  }
}

hipError_t launch_kv_commit(char* kc, char* vc, const char* kn, const char* vn, const int32_t* len_in,
                            const int32_t* nacc, int32_t* len_out, int B, int gamma, int R, long long E, int S,
                            int W, hipStream_t st) {
  if (B == 0) return hipSuccess;
  auto al = [](const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; };
  const bool a16 = E % 16 == 0 && al(kc, 16) && al(vc, 16) && al(kn, 16) && al(vn, 16);
  const bool a4 = E % 4 == 0 && al(kc, 4) && al(vc, 4) && al(kn, 4) && al(vn, 4);
  const int vb = a16 ? 16 : a4 ? 4 : 1;
  const long long vpr = E / vb;
  const long long per_row_max = vpr * (gamma + 1);
  const int rpb = (int)(per_row_max >= kBlockAccesses ? 1 : (kBlockAccesses / per_row_max < R ? kBlockAccesses / per_row_max : R));
  const int nchunk = (R + rpb - 1) / rpb;
  const long long grid = (long long)B * nchunk;
  if (grid > 0x7fffffffLL || (long long)rpb * per_row_max > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const dim3 g((unsigned)grid), t(kThreads);
  if (vb == 16)
    hipLaunchKernelGGL(k_kv_commit<u32x4>, g, t, 0, st, kc, vc, kn, vn, len_in, nacc, len_out, gamma, R, E, S, W,
                       rpb, nchunk);
  else if (vb == 4)
    hipLaunchKernelGGL(k_kv_commit<uint32_t>, g, t, 0, st, kc, vc, kn, vn, len_in, nacc, len_out, gamma, R, E, S,
                       W, rpb, nchunk);
  else
    hipLaunchKernelGGL(k_kv_commit<uint8_t>, g, t, 0, st, kc, vc, kn, vn, len_in, nacc, len_out, gamma, R, E, S,
                       W, rpb, nchunk);
  return hipGetLastError();
}

// Valid slots of every request in logical order: all positions while the
// length P is at most S+W, else the S sinks and then the last W positions
// [Edge C++ 环形 KV 缓存管理内核实现]; -1 past the count.
__global__ __launch_bounds__(kThreads) void k_kv_valid_slots(const int32_t* __restrict__ len, int S, int W,
                                                             int nblk, int32_t* __restrict__ slots,
                                                             int32_t* __restrict__ positions,
                                                             int32_t* __restrict__ counts) {
  const long long b = blockIdx.x / nblk;
  const int i = (int)(blockIdx.x % nblk) * kThreads + threadIdx.x;
  const int cap = S + W;
  if (i >= cap) return;
  const long long P = len[b];
  const int count = P <= 0 ? 0 : (int)(P < cap ? P : cap);
  if (i == 0) counts[b] = count;
  int sl = -1, ps = -1;
  if (i < count) {
    const long long pos = (P <= cap || i < S) ? i : P - W + (i - S);
    ps = (int)pos;
    sl = (int)ring_slot(pos, S, W);
  }
  slots[b * cap + i] = sl;
  if (positions) positions[b * cap + i] = ps;
}

hipError_t launch_kv_valid_slots(const int32_t* len, int B, int S, int W, int32_t* slots, int32_t* positions,
                                 int32_t* counts, hipStream_t st) {
  if (B == 0) return hipSuccess;
  const int nblk = (S + W + kThreads - 1) / kThreads;
  const long long grid = (long long)B * nblk;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(k_kv_valid_slots, dim3((unsigned)grid), dim3(kThreads), 0, st, len, S, W, nblk, slots,
                     positions, counts);
  return hipGetLastError();
}

constexpr int kWindowRows = kThreads / 64;  // one wave per request

__global__ __launch_bounds__(kThreads) void k_draft_window(const int32_t* seq_lens, int B, int W, int bs, int K,
                                                           const int32_t* __restrict__ table, int full_cols,
                                                           int32_t* out_lens, int32_t* __restrict__ out_table,
                                                           int out_cols) {
  const int lane = threadIdx.x & 63;
  const long long i = (long long)blockIdx.x * kWindowRows + (threadIdx.x >> 6);
  if (i >= B) return;
  const int len = seq_lens[i];
  const int wl = window_len(len, W, bs, K);
  const long long start = wl < 0 ? 0 : (long long)len - wl;
  const long long sb = start / bs;
  const long long needed = wl < 0 ? 0 : ((long long)wl + bs - 1) / bs;
  for (int j = lane; j < out_cols; j += 64) {
    int32_t v = 0;
    if (j < needed && sb + j < full_cols) v = table[i * full_cols + sb + j];
    out_table[i * out_cols + j] = v;
  }
  // every lane of the wave read seq_lens[i] above, so the output may replace it
  if (lane == 0) out_lens[i] = wl;
}

hipError_t launch_draft_window(const int32_t* seq_lens, int B, int W, int bs, int K, const int32_t* table,
                               int full_cols, int32_t* out_lens, int32_t* out_table, int out_cols, hipStream_t st) {
  if (B == 0) return hipSuccess;
  const long long grid = ((long long)B + kWindowRows - 1) / kWindowRows;
  hipLaunchKernelGGL(k_draft_window, dim3((unsigned)grid), dim3(kThreads), 0, st, seq_lens, B, W, bs, K, table,
                     full_cols, out_lens, out_table, out_cols);
  return hipGetLastError();
}

}  // namespace svc
