// verify.hip -- the tail of chain verification (dense and ragged layouts),
// after the streaming statistics kernel: G workgroups of 4 waves per request.
//
// Every workgroup of request b runs the request's acceptance scan
// [Primer 考点2 / 第二章] (the chunk partials of its rows merged in fp64, the
// test at every drafted position, the first rejection n) -- a few microseconds
// of latency, repeated rather than handed over -- and workgroup 0 writes the
// accepted tokens, num_accepted, the greedy token and the diagnostics. The
// workgroups then split the tiles of the drawn row(s) between them
// [Primer 考点2 residual max(0, p_t - p_d); 考点4 bonus from p_t], publish
// their tile records, and the last one to finish (a per-request counter that
// the streaming kernel zeroes) runs the inverse-CDF pick. Splitting a request
// over several CUs matters when its drawn row has mass everywhere: the exact
// double-precision work of its tiles is then spread out.
#include "tail.h"

#include <stdlib.h>

#include <mutex>

namespace sv {

constexpr int kReqWaves = 4;  // waves per workgroup

struct RequestArgs {
  const void* tgt;
  const void* dft;
  int V;
  ChainArgs A;     // layout, per-position inputs, partials, num_accepted, diag
  TileRec* recs;   // [B, ntile]
  int* done;       // [B] workgroups of the request finished with their tiles; [B]: ragged layout valid
  int32_t* out;
  int out_width;
  int ntile;       // tiles per row
  int G;           // workgroups per request
  int force_exact;
};

template <int DT, bool STAGED>
__global__ __launch_bounds__(kReqWaves * 64) __attribute__((amdgpu_waves_per_eu(4))) void k_request(RequestArgs R) {
  constexpr int NW = kReqWaves, NT = NW * 64;
  __shared__ union {
    AcceptSpace acc;
    TileSpace<NW> ts;
    PickSpace<NW> pick;
  } u;
  __shared__ double tab[64];         // 2^{j/64}
  __shared__ double mass_t[64], mass_d[64];  // masses of the skipped chunks of the drawn row(s)
  __shared__ SampleJob job;
  __shared__ int s_n, s_bad, s_last;
  const JobPart jp = xcd_job_part(blockIdx.x, R.G);
  if (jp.job >= R.A.L.B) return;  // padding of the grid to whole XCD rounds
  const int b = jp.job, g = jp.part;
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const Layout& L = R.A.L;
  if (tid < 64) tab[tid] = exp2_f64((double)tid * 0.015625);

  // a ragged layout's validity, checked once by the streaming kernel
  const bool layout_ok = L.mode != LAYOUT_RAGGED || R.done[L.B] != 0;
  const ChainRows rows = layout_ok ? chain_rows(L, b) : ChainRows{0, 0, 0};
  int32_t* orow = R.out + (long long)b * R.out_width;
  accept_chain<DT, NW>(R.tgt, R.dft, R.V, R.A, b, rows, layout_ok, g == 0, orow, R.out_width, u.acc, job, mass_t,
                       mass_d, s_n, s_bad);
  const SampleJob J = uniform_job(job);
  if (J.kind == JOB_NONE) return;
  constexpr int es = sizeof(typename Elem<DT>::T);
  const char* trow = reinterpret_cast<const char*>(R.tgt) + (size_t)J.trow * (size_t)R.V * es;
  const char* drow = reinterpret_cast<const char*>(R.dft) + (size_t)J.drow * (size_t)R.V * es;
  TileRec* recs = R.recs + (long long)b * R.ntile;
  // this workgroup's tiles: wave wv takes tiles (g + i G) NW + wv
  if (J.kind == JOB_RESIDUAL)
    wave_tiles<DT, true, NW>(trow, drow, R.V, R.ntile, g * NW + wv, R.G * NW, J, recs, mass_t, mass_d, u.ts, tab,
                             wv, lane);
  else
    wave_tiles<DT, false, NW>(trow, drow, R.V, R.ntile, g * NW + wv, R.G * NW, J, recs, mass_t, mass_d, u.ts, tab,
                              wv, lane);
  // the records are complete before the count; the last workgroup picks
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) s_last = atomicAdd(R.done + b, 1) == R.G - 1;
  __syncthreads();
  if (!s_last) return;
  pick<DT, NW, STAGED>(trow, drow, R.V, R.ntile, J, recs, orow + J.pos, R.force_exact, u.pick, tab);
}

namespace {

int env_int(const char* name, int dflt, int lo, int hi) {
  const char* e = getenv(name);
  if (!e) return dflt;
  const int v = atoi(e);
  return v >= lo && v <= hi ? v : dflt;
}

// Compute units of a device, read once.
int device_cus(int dev) {
  static int cus[64];
  static std::once_flag once[64];
  if (dev < 0 || dev >= 64) dev = 0;
  std::call_once(once[dev], [dev]() {
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c < 1) c = 1;
    cus[dev] = c;
  });
  return cus[dev];
}

}  // namespace

hipError_t launch_verify_chain(int dt, const void* tgt, const void* dft, int V, const Layout& L,
                               const int32_t* tokens, const float* ua, const float* us, const float* temperature,
                               const Partial* part, int nchunk, int chunk_vecs, TileRec* recs, int* done,
                               int32_t* out, int out_width, int32_t* num_acc, float* diag, int force_exact,
                               hipStream_t st) {
  if (L.B == 0) return hipSuccess;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
  const int cus = device_cus(dev);
  // workgroups per request: enough for about four per CU, and 4 to 8 (large
  // batches queue their workgroups: four per request balance dense rows better
  // than one, measured on 1024 requests over 151,936 tokens)
  const long long want = (4ll * cus + L.B - 1) / L.B;
  int G = (int)(want < 4 ? 4 : (want > 8 ? 8 : want));
  G = env_int("SPECVERIFY_REQUEST_GROUPS", G, 1, 64);
  if (xcd_grid(L.B, G) > 0x7fffffffLL) G = 1;
  RequestArgs R;
  R.tgt = tgt;
  R.dft = dft;
  R.V = V;
  R.A = ChainArgs{L, tokens, ua, us, temperature, part, nchunk, chunk_vecs, num_acc, diag};
  R.recs = recs;
  R.done = done;
  R.out = out;
  R.out_width = out_width;
  R.ntile = tiles_per_row(V, dt);
  R.G = G;
  R.force_exact = force_exact;
  const dim3 grid((unsigned)xcd_grid(L.B, G)), block(kReqWaves * 64);
  const bool staged = R.ntile <= kPickStage;
  if (dt == 1) {
    if (staged) hipLaunchKernelGGL((k_request<1, true>), grid, block, 0, st, R);
    else hipLaunchKernelGGL((k_request<1, false>), grid, block, 0, st, R);
  } else {
    if (staged) hipLaunchKernelGGL((k_request<0, true>), grid, block, 0, st, R);
    else hipLaunchKernelGGL((k_request<0, false>), grid, block, 0, st, R);
  }
  return hipGetLastError();
}

}  // namespace sv
