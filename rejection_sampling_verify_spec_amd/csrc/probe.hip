// probe.hip -- a plain read of a buffer with the load pattern of the streaming
// statistics kernel (256 threads, 2048 16-byte vectors per workgroup, all
// eight of a thread's nontemporal loads in flight at once), folding the bits
// into one word per wave so that no load can be dropped. It measures the read rate this part
// reaches in practice, next to the 8 TB/s peak the streaming kernel is priced
// against.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace svp {

constexpr int kThreads = 256;
constexpr int kVecPerBlock = 2048;
constexpr int kU = 8;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void k_read_probe(const u32x4* __restrict__ src, long long nvec,
                                                         uint32_t* __restrict__ out) {
  const long long v0 = (long long)blockIdx.x * kVecPerBlock;
  uint32_t acc = 0;
  for (int k = threadIdx.x; k < kVecPerBlock; k += kThreads * kU) {
    u32x4 w[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const long long i = v0 + k + u * kThreads;
      w[u] = i < nvec ? __builtin_nontemporal_load(src + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) acc ^= w[u].x ^ w[u].y ^ w[u].z ^ w[u].w;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
  if ((threadIdx.x & 63) == 0) out[(long long)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)] = acc;
}

long long probe_blocks(long long nvec) { return (nvec + kVecPerBlock - 1) / kVecPerBlock; }

hipError_t launch_read_probe(const void* src, long long nvec, uint32_t* out, hipStream_t st) {
  const long long g = probe_blocks(nvec);
  if (g == 0) return hipSuccess;
  if (g > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(k_read_probe, dim3((unsigned)g), dim3(kThreads), 0, st, static_cast<const u32x4*>(src), nvec,
                     out);
  return hipGetLastError();
}

}  // namespace svp
