// api.hip -- C ABI of libspecverify (declared in include/specverify.h).
//
// Host side only: validates arguments, carves the caller's workspace and
// enqueues the kernels on the caller's stream. It never allocates device
// memory and never synchronises.
#include "specverify.h"
#include "sv_internal.h"
#include "cache.h"

#include <stdlib.h>

#include <atomic>
#include <algorithm>
#include <mutex>
#include <vector>

using namespace sv;

namespace sv {
hipError_t launch_tree_lossless(int dt, const void* tgt, const void* dft, int V, const Layout& L, int max_depth,
                                const int32_t* tokens, const int32_t* parents, const float* ua, const float* us,
                                const float* temperature, const Partial* part, int nchunk, double* sums,
                                double* rbuf, int* ctr, int32_t* out, int32_t* out_nodes, int32_t* num_acc,
                                hipStream_t st);
int lossless_segments(int V, int dt);
}  // namespace sv
namespace svp {
long long probe_blocks(long long nvec);
hipError_t launch_read_probe(const void* src, long long nvec, uint32_t* out, hipStream_t st);
}  // namespace svp

static_assert(sizeof(Partial) == 8, "Partial layout");

// ---- scratch of the allocation-free entry point
// A fixed array in every device's copy of the library's code object, held until
// the process ends. In host code `scratch` names a host-side stand-in, never the
// device memory: kernels and copies take the address that hipGetSymbolAddress
// returns for the current device (each device has its own copy of the array).
constexpr size_t kScratchBytes = SV_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

static_assert(sizeof(TileRec) == 128, "TileRec layout");

namespace {

// Chunk of a row handled by one row-statistics workgroup, in 16-byte vectors
// (a multiple of kTPB * kU). Calls over many rows take 2048 vectors (32 KB of
// logits per workgroup); calls whose rows would then give fewer than 8192
// workgroups (four per resident slot of a 256-CU part at eight per CU) take
// 1024, so that small batches still spread over every CU and their last round
// of workgroups is short. The choice depends only on the call's sizes, so the
// workspace queries and the calls agree. SPECVERIFY_CHUNK_VECS overrides it.
int per_vec(int dt) { return dt == SV_BF16 ? 8 : 4; }

int env_chunk_vecs() {
  static std::atomic<int> cached{-1};
  int v = cached.load(std::memory_order_relaxed);
  if (v >= 0) return v;
  v = 0;
  if (const char* e = getenv("SPECVERIFY_CHUNK_VECS")) {
    int x = atoi(e);
    if (x >= kTPB * kU && x % (kTPB * kU) == 0 && x <= (1 << 22)) v = x;
  }
  cached.store(v, std::memory_order_relaxed);
  return v;
}

struct Chunking {
  int cv;   // 16-byte vectors per chunk
  int nch;  // chunks per row
};

Chunking chunking(long long rows, int V, int dt) {
  const int nvec = V / per_vec(dt);
  auto nch_of = [&](int cv) { const int n = (nvec + cv - 1) / cv; return n < 1 ? 1 : n; };
  int cv = env_chunk_vecs();
  if (!cv) cv = rows * nch_of(2 * kTPB * kU) < 8192 ? kTPB * kU : 2 * kTPB * kU;
  return Chunking{cv, nch_of(cv)};
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace layout: row-chunk partials | sampling jobs | tile records |
// per-request counters (and the ragged layout's validity flag after them).
struct Carve {
  size_t part, jobs, recs, done, total;
};

Carve carve(long long rows, int B, int V, int dt) {
  Carve c;
  const int nchunk = chunking(rows, V, dt).nch;
  const int ntile = tiles_per_row(V, dt);
  c.part = 0;
  c.jobs = align256((size_t)rows * nchunk * sizeof(Partial));
  c.recs = c.jobs + align256((size_t)B * sizeof(SampleJob));
  c.done = c.recs + align256((size_t)B * ntile * sizeof(TileRec));
  c.total = c.done + align256((size_t)(B + 1) * sizeof(int));
  return c;
}

// SPECVERIFY_FORCE_EXACT_RESIDUAL=1 recomputes every residual tile token by
// token instead of using the fp32 estimate of Z_t/Z_d (same results; slower).
// Read on every call so tests can cover that path in-process.
int force_exact_residual() {
  const char* e = getenv("SPECVERIFY_FORCE_EXACT_RESIDUAL");
  return e && e[0] == '1';
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
size_t esize(int dt) { return dt == SV_BF16 ? 2 : 4; }

// ---- optional timing of the row-statistics kernel
struct Timing {
  bool on = false;
  std::vector<hipEvent_t> ev;  // pairs
  int used = 0;
  static constexpr int kMax = 4096;
} g_timing;
std::mutex g_timing_mu;

void timing_mark(hipStream_t st, bool start) {
  if (!g_timing.on) return;
  int i = g_timing.used;
  if (i >= Timing::kMax) return;
  (void)hipEventRecord(g_timing.ev[2 * i + (start ? 0 : 1)], st);
  if (!start) g_timing.used = i + 1;
}

int launch_stats(int dt, const void* tgt, const void* dft, int V, const Layout& L, const float* temperature,
                 Partial* part, hipStream_t st, int* zero_counts = nullptr) {
  const Chunking ch = chunking(L.RT + L.RD, V, dt);
  timing_mark(st, true);
  hipError_t e = launch_row_stats(dt, tgt, dft, V, L, temperature, ch.cv, ch.nch, part, zero_counts, st);
  timing_mark(st, false);
  return e == hipSuccess ? SV_OK : SV_EHIP;
}

// The chain kernels (streaming statistics, then one workgroup per request) on a
// carved workspace.
int launch_chain(int dt, const void* tgt, const void* dft, int V, const Layout& L, const int32_t* tokens,
                 const float* ua, const float* us, const float* temperature, int32_t* out, int out_width,
                 int32_t* num_acc, float* diag, char* ws, const Carve& cv, hipStream_t st) {
  Partial* part = reinterpret_cast<Partial*>(ws + cv.part);
  int* done = reinterpret_cast<int*>(ws + cv.done);
  int rc = launch_stats(dt, tgt, dft, V, L, temperature, part, st, done);
  if (rc) return rc;
  const Chunking ch = chunking(L.RT + L.RD, V, dt);
  hipError_t e = launch_verify_chain(dt, tgt, dft, V, L, tokens, ua, us, temperature, part, ch.nch,
                                     ch.cv, reinterpret_cast<TileRec*>(ws + cv.recs), done, out, out_width,
                                     num_acc, diag, force_exact_residual(), st);
  return e == hipSuccess ? SV_OK : SV_EHIP;
}

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's scratch address, looked up once per device (with that
// device current) on its first call.
int scratch_for_current_device(char** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SV_EHIP;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SV_EHIP;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = static_cast<char*>(p);
  return SV_OK;
}

}  // namespace

extern "C" {

size_t spec_verify_workspace_bytes(int32_t B, int32_t gamma, int32_t V, int32_t dtype) {
  if (B < 0 || gamma < 0 || gamma > SV_MAX_GAMMA || V < 1 || V > SV_MAX_VOCAB || (dtype != 0 && dtype != 1))
    return 0;
  return carve((long long)B * (2 * gamma + 1), B, V, dtype).total;
}

size_t spec_verify_ragged_workspace_bytes(int32_t B, int32_t total_draft, int32_t gamma_max, int32_t V,
                                          int32_t dtype) {
  if (B < 0 || total_draft < 0 || gamma_max < 0 || gamma_max > SV_MAX_GAMMA || V < 1 || V > SV_MAX_VOCAB ||
      (dtype != 0 && dtype != 1))
    return 0;
  return carve((long long)2 * total_draft + B, B, V, dtype).total;
}

size_t spec_verify_tree_workspace_bytes(int32_t B, int32_t N, int32_t V, int32_t dtype) {
  if (B < 0 || N < 1 || N > SV_MAX_TREE_NODES || V < 1 || V > SV_MAX_VOCAB || (dtype != 0 && dtype != 1)) return 0;
  return carve((long long)B * (2 * N - 1), B, V, dtype).total;
}

// Lossless tree workspace: row-chunk partials | per-team segment sums (two
// buffers) | per-team counters | per-team residuals (two buffers of one row in
// fp64, for at most kLLMaxTeams teams).
struct CarveLL {
  size_t part, sums, ctr, rbuf, total;
};
static CarveLL carve_ll(int B, int N, int V, int dt) {
  CarveLL c;
  c.part = 0;
  const long long rows = (long long)B * (2 * N - 1);
  const size_t nseg = (size_t)lossless_segments(V, dt);
  const size_t seg_tok = 64 * (dt == SV_BF16 ? 8 : 4);
  c.sums = align256((size_t)rows * chunking(rows, V, dt).nch * sizeof(Partial));
  c.ctr = c.sums + align256((size_t)B * 2 * nseg * sizeof(double));
  c.rbuf = c.ctr + align256((size_t)B * sizeof(int));
  c.total = c.rbuf + align256((size_t)std::min(B, kLLMaxTeams) * 2 * nseg * seg_tok * sizeof(double));
  return c;
}

size_t spec_verify_tree_lossless_workspace_bytes(int32_t B, int32_t N, int32_t V, int32_t dtype) {
  if (B < 0 || N < 1 || N > SV_MAX_TREE_NODES || V < 1 || V > SV_MAX_VOCAB || (dtype != 0 && dtype != 1)) return 0;
  return carve_ll(B, N, V, dtype).total;
}

size_t spec_sample_rows_workspace_bytes(int32_t rows, int32_t V, int32_t dtype) {
  if (rows < 0 || V < 1 || V > SV_MAX_VOCAB || (dtype != 0 && dtype != 1)) return 0;
  return carve(rows, rows, V, dtype).total;
}

size_t spec_row_softmax_stats_workspace_bytes(int32_t rows, int32_t V, int32_t dtype) {
  if (rows < 0 || V < 1 || V > SV_MAX_VOCAB || (dtype != 0 && dtype != 1)) return 0;
  return align256((size_t)rows * chunking(rows, V, dtype).nch * sizeof(Partial));
}

static int check_common(const void* tgt, const void* dft, bool need_dft, int32_t dtype, int32_t V) {
  if (dtype != SV_F32 && dtype != SV_BF16) return SV_EDTYPE;
  if (V < 1 || V > SV_MAX_VOCAB) return SV_EINVAL;
  if (!tgt || (need_dft && !dft)) return SV_EINVAL;
  if (!aligned(tgt, esize(dtype)) || (need_dft && !aligned(dft, esize(dtype)))) return SV_EALIGN;
  return SV_OK;
}

static int check_ws(const void* ws, size_t have, size_t need) {
  if (need == 0 || !ws || have < need || !aligned(ws, 256)) return SV_ENOWS;
  return SV_OK;
}

// Argument checks of the dense chain entry points (everything but the workspace).
static int check_chain_args(const void* target_logits, const void* draft_logits, int32_t dtype,
                            const int32_t* draft_tokens, const float* u_accept, const float* u_sample,
                            const float* temperature, int32_t B, int32_t gamma, int32_t V, int32_t* out_tokens,
                            int32_t* num_accepted) {
  if (B < 0 || gamma < 0 || gamma > SV_MAX_GAMMA) return SV_EINVAL;
  if (B == 0) return SV_OK;
  int rc = check_common(target_logits, draft_logits, gamma > 0, dtype, V);
  if (rc) return rc;
  if (!u_sample || !temperature || !out_tokens || !num_accepted) return SV_EINVAL;
  if (gamma > 0 && (!draft_tokens || !u_accept)) return SV_EINVAL;
  return SV_OK;
}

int spec_verify(const void* target_logits, const void* draft_logits, int32_t dtype, const int32_t* draft_tokens,
                const float* u_accept, const float* u_sample, const float* temperature, int32_t B, int32_t gamma,
                int32_t V, int32_t* out_tokens, int32_t* num_accepted, float* diag_probs, void* workspace,
                size_t workspace_bytes, void* stream) {
  int rc = check_chain_args(target_logits, draft_logits, dtype, draft_tokens, u_accept, u_sample, temperature, B,
                            gamma, V, out_tokens, num_accepted);
  if (rc || B == 0) return rc;
  const long long RT = (long long)B * (gamma + 1), RD = (long long)B * gamma;
  Carve cv = carve(RT + RD, B, V, dtype);
  rc = check_ws(workspace, workspace_bytes, cv.total);
  if (rc) return rc;
  Layout L{LAYOUT_DENSE, B, gamma, nullptr, 0, RT, RD};
  return launch_chain(dtype, target_logits, draft_logits, V, L, draft_tokens, u_accept, u_sample, temperature,
                      out_tokens, gamma + 1, num_accepted, diag_probs, static_cast<char*>(workspace), cv,
                      static_cast<hipStream_t>(stream));
}

int spec_verify_noalloc(const void* target_logits, const void* draft_logits, int32_t dtype,
                        const int32_t* draft_tokens, const float* u_accept, const float* u_sample,
                        const float* temperature, int32_t B, int32_t gamma, int32_t V, int32_t* out_tokens,
                        int32_t* num_accepted, float* diag_probs, void* stream) {
  int rc = check_chain_args(target_logits, draft_logits, dtype, draft_tokens, u_accept, u_sample, temperature, B,
                            gamma, V, out_tokens, num_accepted);
  if (rc || B == 0) return rc;
  const long long RT = (long long)B * (gamma + 1), RD = (long long)B * gamma;
  const Carve cv = carve(RT + RD, B, V, dtype);
  if (cv.total > kScratchBytes) return SV_ESCRATCH;
  char* ws = nullptr;
  if ((rc = scratch_for_current_device(&ws))) return rc;
  // nothing in the scratch needs clearing: the streaming kernel writes every
  // partial and zeroes the per-request counters before the tail kernel reads them
  Layout L{LAYOUT_DENSE, B, gamma, nullptr, 0, RT, RD};
  return launch_chain(dtype, target_logits, draft_logits, V, L, draft_tokens, u_accept, u_sample, temperature,
                      out_tokens, gamma + 1, num_accepted, diag_probs, ws, cv, static_cast<hipStream_t>(stream));
}

int spec_verify_ragged(const void* target_logits, const void* draft_logits, int32_t dtype, const int32_t* cu_gamma,
                       int32_t total_draft, const int32_t* draft_tokens, const float* u_accept,
                       const float* u_sample, const float* temperature, int32_t B, int32_t gamma_max, int32_t V,
                       int32_t* out_tokens, int32_t* num_accepted, float* diag_probs, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (B < 0 || total_draft < 0 || gamma_max < 0 || gamma_max > SV_MAX_GAMMA) return SV_EINVAL;
  if (B == 0) return SV_OK;
  if ((long long)total_draft > (long long)B * gamma_max) return SV_EINVAL;
  int rc = check_common(target_logits, draft_logits, total_draft > 0, dtype, V);
  if (rc) return rc;
  if (!cu_gamma || !u_sample || !temperature || !out_tokens || !num_accepted) return SV_EINVAL;
  if (total_draft > 0 && (!draft_tokens || !u_accept)) return SV_EINVAL;
  const long long RT = (long long)total_draft + B, RD = total_draft;
  Carve cv = carve(RT + RD, B, V, dtype);
  rc = check_ws(workspace, workspace_bytes, cv.total);
  if (rc) return rc;
  Layout L{LAYOUT_RAGGED, B, gamma_max, cu_gamma, total_draft, RT, RD};
  return launch_chain(dtype, target_logits, draft_logits, V, L, draft_tokens, u_accept, u_sample, temperature,
                      out_tokens, gamma_max + 1, num_accepted, diag_probs, static_cast<char*>(workspace), cv,
                      static_cast<hipStream_t>(stream));
}

int spec_verify_tree(const void* target_logits, const void* draft_logits, int32_t dtype, const int32_t* node_tokens,
                     const int32_t* parents, const float* u_accept, const float* u_sample, const float* temperature,
                     int32_t B, int32_t N, int32_t V, int32_t max_depth, int32_t* out_tokens, int32_t* out_nodes,
                     int32_t* num_accepted, void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 0 || N < 1 || N > SV_MAX_TREE_NODES || max_depth < 0 || max_depth >= N) return SV_EINVAL;
  if (B == 0) return SV_OK;
  int rc = check_common(target_logits, draft_logits, N > 1, dtype, V);
  if (rc) return rc;
  if (!node_tokens || !parents || !u_accept || !u_sample || !temperature || !out_tokens || !out_nodes ||
      !num_accepted)
    return SV_EINVAL;
  const long long RT = (long long)B * N, RD = (long long)B * (N - 1);
  Carve cv = carve(RT + RD, B, V, dtype);
  rc = check_ws(workspace, workspace_bytes, cv.total);
  if (rc) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  Partial* part = reinterpret_cast<Partial*>(ws + cv.part);
  SampleJob* jobs = reinterpret_cast<SampleJob*>(ws + cv.jobs);
  TileRec* recs = reinterpret_cast<TileRec*>(ws + cv.recs);
  Layout L{LAYOUT_TREE, B, N, nullptr, 0, RT, RD};
  int* done = reinterpret_cast<int*>(ws + cv.done);
  if ((rc = launch_stats(dtype, target_logits, draft_logits, V, L, temperature, part, st, done))) return rc;
  if (launch_accept_tree(dtype, target_logits, draft_logits, V, L, max_depth, node_tokens, parents, u_accept,
                         u_sample, temperature, part, chunking(RT + RD, V, dtype).nch, out_tokens, out_nodes,
                         num_accepted,
                         jobs, st) != hipSuccess)
    return SV_EHIP;
  if (launch_finish_jobs(dtype, target_logits, draft_logits, V, B, jobs, recs, part, chunking(RT + RD, V, dtype).nch,
                         RT, done,
                         out_tokens, max_depth + 1, force_exact_residual(), st) != hipSuccess)
    return SV_EHIP;
  return SV_OK;
}

int spec_verify_tree_lossless(const void* target_logits, const void* draft_logits, int32_t dtype,
                              const int32_t* node_tokens, const int32_t* parents, const float* u_accept,
                              const float* u_sample, const float* temperature, int32_t B, int32_t N, int32_t V,
                              int32_t max_depth, int32_t* out_tokens, int32_t* out_nodes, int32_t* num_accepted,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 0 || N < 1 || N > SV_MAX_TREE_NODES || max_depth < 0 || max_depth >= N) return SV_EINVAL;
  if (B == 0) return SV_OK;
  int rc = check_common(target_logits, draft_logits, N > 1, dtype, V);
  if (rc) return rc;
  if (!node_tokens || !parents || !u_accept || !u_sample || !temperature || !out_tokens || !out_nodes ||
      !num_accepted)
    return SV_EINVAL;
  const long long RT = (long long)B * N, RD = (long long)B * (N - 1);
  const CarveLL cv = carve_ll(B, N, V, dtype);
  rc = check_ws(workspace, workspace_bytes, cv.total);
  if (rc) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  Partial* part = reinterpret_cast<Partial*>(ws + cv.part);
  double* sums = reinterpret_cast<double*>(ws + cv.sums);
  double* rbuf = reinterpret_cast<double*>(ws + cv.rbuf);
  int* ctr = reinterpret_cast<int*>(ws + cv.ctr);
  Layout L{LAYOUT_TREE, B, N, nullptr, 0, RT, RD};
  if ((rc = launch_stats(dtype, target_logits, draft_logits, V, L, temperature, part, st, ctr))) return rc;
  timing_mark(st, true);
  const hipError_t e = launch_tree_lossless(dtype, target_logits, draft_logits, V, L, max_depth, node_tokens, parents,
                                            u_accept, u_sample, temperature, part, chunking(RT + RD, V, dtype).nch,
                                            sums, rbuf, ctr, out_tokens, out_nodes, num_accepted, st);
  timing_mark(st, false);
  return e == hipSuccess ? SV_OK : SV_EHIP;
}

int spec_row_softmax_stats(const void* logits, int32_t dtype, int32_t rows, int32_t V, const float* temperature,
                           float* out_max, float* out_logz, int32_t* out_argmax, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (rows < 0) return SV_EINVAL;
  if (rows == 0) return SV_OK;
  int rc = check_common(logits, nullptr, false, dtype, V);
  if (rc) return rc;
  if (!temperature || !out_max || !out_logz || !out_argmax) return SV_EINVAL;
  rc = check_ws(workspace, workspace_bytes, spec_row_softmax_stats_workspace_bytes(rows, V, dtype));
  if (rc) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Partial* part = static_cast<Partial*>(workspace);
  Layout L{LAYOUT_ROWS, rows, 0, nullptr, 0, rows, 0};
  if ((rc = launch_stats(dtype, logits, nullptr, V, L, temperature, part, st))) return rc;
  if (launch_stats_finalize(part, chunking(rows, V, dtype).nch, rows, temperature, out_max, out_logz, out_argmax,
                            st) !=
      hipSuccess)
    return SV_EHIP;
  return SV_OK;
}

int spec_sample_rows(const void* logits, int32_t dtype, int32_t rows, int32_t V, const float* temperature,
                     const float* u, int32_t* out_tokens, void* workspace, size_t workspace_bytes, void* stream) {
  if (rows < 0) return SV_EINVAL;
  if (rows == 0) return SV_OK;
  int rc = check_common(logits, nullptr, false, dtype, V);
  if (rc) return rc;
  if (!temperature || !u || !out_tokens) return SV_EINVAL;
  Carve cv = carve(rows, rows, V, dtype);
  rc = check_ws(workspace, workspace_bytes, cv.total);
  if (rc) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  Partial* part = reinterpret_cast<Partial*>(ws + cv.part);
  TileRec* recs = reinterpret_cast<TileRec*>(ws + cv.recs);
  int* done = reinterpret_cast<int*>(ws + cv.done);
  Layout L{LAYOUT_ROWS, rows, 0, nullptr, 0, rows, 0};
  if ((rc = launch_stats(dtype, logits, nullptr, V, L, temperature, part, st, done))) return rc;
  const Chunking ch = chunking(rows, V, dtype);
  // each row's job is built by its draw workgroups (no job table)
  if (launch_finish_jobs(dtype, logits, logits, V, rows, nullptr, recs, part, ch.nch, rows, done, out_tokens, 1,
                         force_exact_residual(), st, ch.cv, temperature, u) != hipSuccess)
    return SV_EHIP;
  return SV_OK;
}

static bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

int spec_kv_commit(void* k_cache, void* v_cache, const void* k_new, const void* v_new, const int32_t* lengths,
                   const int32_t* num_accepted, int32_t* new_lengths, int32_t B, int32_t gamma, int32_t rows,
                   int64_t row_bytes, int32_t sink, int32_t window, void* stream) {
  if (B < 0 || gamma < 0 || gamma > SV_MAX_GAMMA || rows < 1 || row_bytes < 1 || row_bytes > SV_MAX_KV_ROW_BYTES ||
      sink < 0 || window < 1 || (int64_t)sink + window > SV_MAX_KV_SLOTS)
    return SV_EINVAL;
  if (B == 0) return SV_OK;
  if (!k_cache || !v_cache || !k_new || !v_new || !lengths || !num_accepted || !new_lengths) return SV_EINVAL;
  if (k_cache == v_cache || ranges_overlap(lengths, (size_t)B * 4, new_lengths, (size_t)B * 4)) return SV_EINVAL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  timing_mark(st, true);
  hipError_t e = svc::launch_kv_commit(static_cast<char*>(k_cache), static_cast<char*>(v_cache),
                                       static_cast<const char*>(k_new), static_cast<const char*>(v_new), lengths,
                                       num_accepted, new_lengths, B, gamma, rows, row_bytes, sink, window, st);
  timing_mark(st, false);
  return e == hipSuccess ? SV_OK : SV_EHIP;
}

int spec_kv_valid_slots(const int32_t* lengths, int32_t B, int32_t sink, int32_t window, int32_t* slots,
                        int32_t* positions, int32_t* counts, void* stream) {
  if (B < 0 || sink < 0 || window < 1 || (int64_t)sink + window > SV_MAX_KV_SLOTS) return SV_EINVAL;
  if (B == 0) return SV_OK;
  if (!lengths || !slots || !counts) return SV_EINVAL;
  return svc::launch_kv_valid_slots(lengths, B, sink, window, slots, positions, counts,
                                    static_cast<hipStream_t>(stream)) == hipSuccess
             ? SV_OK
             : SV_EHIP;
}

int32_t spec_draft_window_max_blocks(int32_t window, int32_t block_size) {
  if (window < 1 || block_size < 1) return -1;
  return (int32_t)(((int64_t)window + 2 * (int64_t)block_size - 2) / block_size);
}

static int check_window_args(int32_t window, int32_t block_size, int32_t future_offset) {
  return (window < 1 || block_size < 1 || future_offset < 0 || future_offset > window) ? SV_EINVAL : SV_OK;
}

int spec_draft_window(const int32_t* seq_lens, int32_t B, int32_t window, int32_t block_size, int32_t future_offset,
                      const int32_t* block_table, int32_t full_cols, int32_t* windowed_lens, int32_t* window_table,
                      int32_t window_cols, void* stream) {
  if (B < 0 || full_cols < 0 || check_window_args(window, block_size, future_offset)) return SV_EINVAL;
  if (window_cols < spec_draft_window_max_blocks(window, block_size)) return SV_EINVAL;
  if (B == 0) return SV_OK;
  if (!seq_lens || !windowed_lens || !window_table || (full_cols > 0 && !block_table)) return SV_EINVAL;
  if (seq_lens != windowed_lens && ranges_overlap(seq_lens, (size_t)B * 4, windowed_lens, (size_t)B * 4))
    return SV_EINVAL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  timing_mark(st, true);
  hipError_t e = svc::launch_draft_window(seq_lens, B, window, block_size, future_offset, block_table, full_cols,
                                          windowed_lens, window_table, window_cols, st);
  timing_mark(st, false);
  return e == hipSuccess ? SV_OK : SV_EHIP;
}

int spec_draft_window_host(const int32_t* seq_lens, int32_t n, int32_t window, int32_t block_size,
                           int32_t future_offset, int32_t* windowed_lens) {
  if (n < 0 || check_window_args(window, block_size, future_offset)) return SV_EINVAL;
  if (n > 0 && (!seq_lens || !windowed_lens)) return SV_EINVAL;
  for (int32_t i = 0; i < n; ++i) windowed_lens[i] = svc::window_len(seq_lens[i], window, block_size, future_offset);
  return SV_OK;
}

size_t spec_read_probe_words(size_t bytes) { return (size_t)svp::probe_blocks((long long)(bytes / 16)) * 4; }

int spec_read_probe(const void* src, size_t bytes, uint32_t* out, void* stream) {
  if (bytes == 0) return SV_OK;
  if (!src || !out || bytes % 16 != 0 || bytes > ((size_t)1 << 46)) return SV_EINVAL;
  if (!aligned(src, 16)) return SV_EALIGN;
  return svp::launch_read_probe(src, (long long)(bytes / 16), out, static_cast<hipStream_t>(stream)) == hipSuccess
             ? SV_OK
             : SV_EHIP;
}

const char* spec_verify_strerror(int status) {
  switch (status) {
    case SV_OK: return "success";
    case SV_EINVAL: return "invalid argument (null pointer, size or count out of range)";
    case SV_EDTYPE: return "unsupported dtype (expected SV_F32 or SV_BF16)";
    case SV_ENOWS: return "workspace missing, too small or not 256-byte aligned";
    case SV_EALIGN: return "logits pointer not aligned to its element size";
    case SV_EHIP: return "HIP runtime or kernel launch failure";
    case SV_ESCRATCH: return "sizes need more scratch than the allocation-free entry point holds";
    default: return "unknown status";
  }
}

int spec_verify_version(void) { return 1; }

int spec_verify_timing_enable(int enable) {
  std::lock_guard<std::mutex> lk(g_timing_mu);
  if (enable) {
    if (g_timing.ev.empty()) {
      g_timing.ev.resize(2 * Timing::kMax);
      for (auto& e : g_timing.ev)
        if (hipEventCreate(&e) != hipSuccess) return SV_EHIP;
    }
    g_timing.on = true;
  } else {
    g_timing.on = false;
  }
  return SV_OK;
}

int spec_verify_timing_reset(void) {
  std::lock_guard<std::mutex> lk(g_timing_mu);
  g_timing.used = 0;
  return SV_OK;
}

int spec_verify_timing_read(float* ms_out, int32_t max, int32_t* count) {
  std::lock_guard<std::mutex> lk(g_timing_mu);
  if (count) *count = g_timing.used;
  for (int i = 0; i < g_timing.used && i < max; ++i) {
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, g_timing.ev[2 * i], g_timing.ev[2 * i + 1]) != hipSuccess) return SV_EHIP;
    if (ms_out) ms_out[i] = ms;
  }
  return SV_OK;
}

}  // extern "C"
