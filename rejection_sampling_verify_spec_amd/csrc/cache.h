// cache.h -- the KV-cache steps around verification (cache.hip): the commit
// of the kept positions into a sink + ring cache, the list of valid slots, and
// the draft-KV window over a paged block table.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace svc {

// Physical slot of logical position pos in a cache of S sink slots followed by
// a ring of W slots [Edge 环形上下文与注意力沉淀机制, Slot(pos) equation].
__host__ __device__ __forceinline__ long long ring_slot(long long pos, int S, int W) {
  return pos < S ? pos : S + (pos - S) % W;
}

// Windowed length of one request for a draft window of W tokens over blocks of
// bs tokens, the window end K tokens past the length [Window 窗口数学]: the
// start is max(len + K - W, 0) rounded down to a block boundary. -1 for a
// negative length.
__host__ __device__ __forceinline__ int window_len(int len, int W, int bs, int K) {
  if (len < 0) return -1;
  long long d = (long long)len + K - W;
  long long start = d > 0 ? (d / bs) * bs : 0;
  return (int)(len - start);
}

hipError_t launch_kv_commit(char* kc, char* vc, const char* kn, const char* vn, const int32_t* len_in,
                            const int32_t* nacc, int32_t* len_out, int B, int gamma, int R, long long E, int S,
                            int W, hipStream_t st);
hipError_t launch_kv_valid_slots(const int32_t* len, int B, int S, int W, int32_t* slots, int32_t* positions,
                                 int32_t* counts, hipStream_t st);
hipError_t launch_draft_window(const int32_t* seq_lens, int B, int W, int bs, int K, const int32_t* table,
                               int full_cols, int32_t* out_lens, int32_t* out_table, int out_cols, hipStream_t st);

}  // namespace svc
