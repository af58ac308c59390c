/*
 * specverify.h -- C ABI of libspecverify: batched speculative-decoding
 * verification (rejection sampling with residual / bonus resampling) for
 * AMD Instinct MI355X (gfx950).
 *
 * Method (cited by page and section):
 *   [Primer] "猜想解码 (Speculative Decoding) 全景" (talentme.airsota.com):
 *     考点 1  - the target model scores gamma+1 positions in one pass;
 *     考点 2  - accept a drafted token x with probability
 *               min(1, p_target(x) / p_draft(x)); on rejection draw from the
 *               residual max(0, p_target - p_draft) / sum;
 *     考点 4  - every step yields at least one token; all gamma accepted
 *               yields gamma + 1 (the extra, "bonus", token);
 *     第二章 / 第三章 - the same acceptance rule per position.
 *   [Edge] lqnn.cn/news/249899, "动态推迟投机验证调度器设计": probabilities
 *     are softmax(logits / T) with one temperature T for both models; the
 *     pipeline figure in "嵌入式流式推理的访存墙与投机瓶颈" places an
 *     accept/reject evaluation kernel after a batched target pass over a
 *     token tree.
 *
 * Conventions shared by every entry point
 *   - All array arguments are DEVICE pointers owned by the caller. The
 *     library never allocates, frees or retains them, and keeps no per-call
 *     state; scratch memory is the caller's `workspace` (spec_verify_noalloc
 *     instead uses a fixed array that the library holds on each device).
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL is the default
 *     stream). Outputs are valid after the caller synchronises that stream.
 *   - Logits are row-major with the vocabulary contiguous; `dtype` is
 *     SV_F32 (float) or SV_BF16 (bfloat16 bit patterns, uint16). Target and
 *     draft share one dtype. Pointers must be aligned to the element size;
 *     rows need not be 16-byte aligned.
 *   - Temperature is per request (float). T == 0 selects greedy decoding:
 *     accept while the draft token equals the target argmax (lowest index on
 *     ties) and emit the argmax at the first mismatch; draft logits and the
 *     uniforms of that request are not read.
 *   - The random numbers of the method are inputs: u_accept decides the
 *     acceptance test u * p_draft(x) < p_target(x) (equivalently
 *     u < min(1, p_target/p_draft)); u_sample drives the inverse-CDF draw
 *     y = min{ j : C_j > u * S } over the residual (or bonus) masses in
 *     ascending token order. Uniforms must lie in [0, 1).
 *   - num_accepted counts accepted draft tokens (0..gamma); the request emits
 *     num_accepted + 1 tokens; later columns of out_tokens are -1.
 *   - Host-side argument errors return a negative sv_status before anything
 *     is enqueued. Per-request data errors (temperature NaN, negative,
 *     infinite or subnormal; a token outside [0, V); for T > 0 a uniform NaN
 *     or outside [0, 1); a logit row that is read and holds a NaN, a +inf or
 *     no finite value; for the ragged and tree layouts a malformed layout)
 *     are reported on the device: num_accepted = -1 and that request's
 *     out_tokens row filled with -1. No call synchronises the stream.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sv_status {
    SV_OK = 0,
    SV_EINVAL = -1,  /* null pointer, bad size or count                        */
    SV_EDTYPE = -2,  /* dtype not SV_F32 / SV_BF16                              */
    SV_ENOWS = -3,   /* workspace null, too small or not 256-byte aligned       */
    SV_EALIGN = -4,  /* a logits pointer not aligned to its element size        */
    SV_EHIP = -5,    /* a HIP runtime call or kernel launch failed              */
    SV_ESCRATCH = -6, /* spec_verify_noalloc: the sizes need more than its scratch */
} sv_status;

typedef enum sv_dtype { SV_F32 = 0, SV_BF16 = 1 } sv_dtype;

/* Largest sizes accepted (host-side validation). */
#define SV_MAX_GAMMA 256       /* drafted positions per request          */
#define SV_MAX_TREE_NODES 1024 /* nodes per token tree (root included)    */
#define SV_MAX_VOCAB (1 << 28)
#define SV_MAX_KV_SLOTS (1 << 30)     /* sink + window slots of one KV cache      */
#define SV_MAX_KV_ROW_BYTES (1 << 30) /* bytes of one cache row (one head, one position) */
#define SV_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20) /* scratch of spec_verify_noalloc, per device */

/* Workspace bytes needed by spec_verify for these sizes (0 on bad sizes). */
size_t spec_verify_workspace_bytes(int32_t B, int32_t gamma, int32_t V, int32_t dtype);

/*
 * Linear (chain) verification of B requests with gamma drafted tokens each
 * [Primer 考点1, 考点2, 考点4].
 *   target_logits  [B, gamma+1, V]  row i = target distribution at position i
 *   draft_logits   [B, gamma,   V]  row i = distribution draft token i came from
 *   draft_tokens   [B, gamma]  int32
 *   u_accept       [B, gamma]  float, uniform for the test at position i
 *   u_sample       [B, gamma+1] float, uniform for the draw at the final
 *                  position n (residual if n < gamma, bonus if n == gamma)
 *   temperature    [B] float
 *   out_tokens     [B, gamma+1] int32 (written)
 *   num_accepted   [B] int32 (written)
 *   diag_probs     [B, gamma, 2] float or NULL: (p_target(x_i), p_draft(x_i))
 *                  for T > 0 requests (NaN otherwise); for parity checks.
 *   workspace      >= spec_verify_workspace_bytes(B, gamma, V, dtype) bytes,
 *                  256-byte aligned; contents need no initialisation.
 * B == 0 is a no-op. Errors: SV_EINVAL (B < 0, gamma outside [0,
 * SV_MAX_GAMMA], V outside [1, SV_MAX_VOCAB], a required pointer NULL),
 * SV_EDTYPE, SV_EALIGN, SV_ENOWS, SV_EHIP.
 */
int spec_verify(const void* target_logits, const void* draft_logits, int32_t dtype,
                const int32_t* draft_tokens, const float* u_accept, const float* u_sample,
                const float* temperature, int32_t B, int32_t gamma, int32_t V, int32_t* out_tokens,
                int32_t* num_accepted, float* diag_probs, void* workspace, size_t workspace_bytes,
                void* stream);

/*
 * spec_verify for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. The same
 * arguments (without the workspace), results and errors as spec_verify; it
 * calls no allocating routine. Its scratch is a fixed array of
 * SV_NOALLOC_SCRATCH_BYTES (32 MiB) that the library holds on every device it
 * runs on until the process ends (its address is looked up on the first call on
 * a device). Sizes whose workspace (spec_verify_workspace_bytes) exceeds it
 * return SV_ESCRATCH before anything is enqueued. Every call on a device uses
 * that device's one array: calls that overlap on one device (on different
 * streams, or from different threads) race and must be serialised by the caller;
 * calls in one stream are ordered and safe.
 */
int spec_verify_noalloc(const void* target_logits, const void* draft_logits, int32_t dtype,
                        const int32_t* draft_tokens, const float* u_accept, const float* u_sample,
                        const float* temperature, int32_t B, int32_t gamma, int32_t V, int32_t* out_tokens,
                        int32_t* num_accepted, float* diag_probs, void* stream);

/* Workspace bytes for spec_verify_ragged. */
size_t spec_verify_ragged_workspace_bytes(int32_t B, int32_t total_draft, int32_t gamma_max, int32_t V,
                                          int32_t dtype);

/*
 * Ragged (mixed gamma and temperature) verification [Primer 考点1, 考点2,
 * 考点4]: request b owns gamma_b = cu_gamma[b+1] - cu_gamma[b] drafted
 * positions, draft rows cu_gamma[b] .. cu_gamma[b+1]-1 and target rows
 * cu_gamma[b]+b .. cu_gamma[b+1]+b.
 *   target_logits  [total_draft + B, V]     draft_logits [total_draft, V]
 *   cu_gamma       [B+1] int32, device     total_draft  host copy of cu_gamma[B]
 *   draft_tokens, u_accept [total_draft]   u_sample [total_draft + B]
 *   temperature    [B]
 *   out_tokens     [B, gamma_max+1]         num_accepted [B]
 *   diag_probs     [total_draft, 2] or NULL
 * The layout is valid when cu_gamma[0] == 0, it never decreases, every
 * gamma_b <= gamma_max and cu_gamma[B] == total_draft; otherwise every
 * request reports -1.
 */
int spec_verify_ragged(const void* target_logits, const void* draft_logits, int32_t dtype,
                       const int32_t* cu_gamma, int32_t total_draft, const int32_t* draft_tokens,
                       const float* u_accept, const float* u_sample, const float* temperature, int32_t B,
                       int32_t gamma_max, int32_t V, int32_t* out_tokens, int32_t* num_accepted,
                       float* diag_probs, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes for spec_verify_tree. */
size_t spec_verify_tree_workspace_bytes(int32_t B, int32_t N, int32_t V, int32_t dtype);

/*
 * Token-tree verification [Primer 考点3: multi-head drafts verified as a
 * tree in one target pass; Edge pipeline figure: token tree -> accept/reject
 * evaluation]. Node 0 is the root (already emitted context); node v >= 1
 * carries draft token node_tokens[v] and parent parents[v] < v.
 *   target_logits  [B, N, V]   row v = target distribution after the path to v
 *   draft_logits   [B, N-1, V] row v-1 = distribution node v's token came from
 *   node_tokens, parents, u_accept, u_sample [B, N] int32/float
 *   out_tokens, out_nodes [B, max_depth+1]; num_accepted [B]
 * Node v is accepted when u_accept[v] * p_draft[v](x_v) < p_target[parent(v)](x_v)
 * (greedy: x_v == argmax of the parent's target row); a node is kept when it
 * and all its ancestors are accepted; the end node e is the deepest kept node
 * (lowest index on ties). out_tokens holds the tokens of the path root->e
 * (root excluded) and then one drawn token with u_sample[e]: from p_target[e]
 * when e has no children, else from the residual of p_target[e] against the
 * draft row of e's lowest-index child. out_nodes holds the path's node
 * indices. A tree with parents[0] != -1, a parent index >= its child, or a
 * depth above max_depth reports -1 for that request.
 */
int spec_verify_tree(const void* target_logits, const void* draft_logits, int32_t dtype,
                     const int32_t* node_tokens, const int32_t* parents, const float* u_accept,
                     const float* u_sample, const float* temperature, int32_t B, int32_t N, int32_t V,
                     int32_t max_depth, int32_t* out_tokens, int32_t* out_nodes, int32_t* num_accepted,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes for spec_verify_tree_lossless. */
size_t spec_verify_tree_lossless_workspace_bytes(int32_t B, int32_t N, int32_t V, int32_t dtype);

/*
 * Lossless multi-candidate token-tree verification [Primer 考点3: a token
 * tree verified in one target pass; Primer 考点2: acceptance
 * min(1, p_target/p_draft) and the residual max(0, p_target - p_draft)/sum].
 * Same tree layout, arguments, outputs and error reports as spec_verify_tree;
 * only the walk differs. From the root, the current distribution r is the
 * current node's target row; its children are tried in ascending index order:
 * child c is accepted when u_accept[c] * p_draft[c](x_c) < r(x_c) and then
 * becomes the current node; a rejected child replaces r by
 * max(0, r - p_draft[c]) / sum before its next sibling is tried (a sum that
 * underflows to 0 keeps r). When no child is accepted, or the node is a leaf,
 * the final token is drawn from r with u_sample of that node by the inverse
 * CDF (y = min{ j : C_j > u*S }). Each emitted token then follows the target
 * distribution exactly, provided each child's token was drawn from its own
 * draft row independently of its siblings. Greedy requests (T == 0) follow the
 * first child whose token is the argmax of the current node's target row and
 * emit the argmax at the end.
 * A rejection costs one pass over the current target row and the draft rows of
 * the rejected siblings. The call runs as a cooperative launch (every
 * workgroup resident at once); it returns SV_EHIP if the device cannot launch
 * it.
 */
int spec_verify_tree_lossless(const void* target_logits, const void* draft_logits, int32_t dtype,
                              const int32_t* node_tokens, const int32_t* parents, const float* u_accept,
                              const float* u_sample, const float* temperature, int32_t B, int32_t N, int32_t V,
                              int32_t max_depth, int32_t* out_tokens, int32_t* out_nodes, int32_t* num_accepted,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes for spec_row_softmax_stats. */
size_t spec_row_softmax_stats_workspace_bytes(int32_t rows, int32_t V, int32_t dtype);

/*
 * Per-row softmax statistics, the first stage of every verify call
 * [Edge scheduler section: max and sum of exp((l - max)/T) per row]:
 *   logits [rows, V], temperature [rows]
 *   out_max    [rows] float: the row maximum
 *   out_logz   [rows] float: log sum_j exp((l_j - max)/T) for T > 0, else NaN
 *   out_argmax [rows] int32: lowest index of the maximum for T == 0, else -1
 * Unusable rows report out_max = NaN. Exposed for parity checks of the
 * streaming reduction on its own.
 */
int spec_row_softmax_stats(const void* logits, int32_t dtype, int32_t rows, int32_t V,
                           const float* temperature, float* out_max, float* out_logz, int32_t* out_argmax,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes for spec_sample_rows. */
size_t spec_sample_rows_workspace_bytes(int32_t rows, int32_t V, int32_t dtype);

/*
 * Draft-token sampling: one token per logit row, drawn from
 * p = softmax(l/T) [Edge scheduler section: the temperature softmax
 * exp((l - max)/T) / sum], the way the draft model proposes the tokens that
 * verification then tests [Primer 考点1]. The draw is the inverse CDF of the
 * verify draw: y = min{ j : C_j > u*S } in ascending token order, C the
 * running sum of p (zero-mass tokens are never drawn; if rounding leaves no
 * such j, the last token of positive mass). T == 0 takes the lowest index of
 * the maximum and ignores u.
 *   logits      [rows, V] (dtype SV_F32 or SV_BF16), row-major
 *   temperature [rows] float
 *   u           [rows] float, the caller's uniforms in [0, 1)
 *   out_tokens  [rows] int32: the drawn token, or -1 for an unusable row
 *               (temperature NaN, negative, infinite or subnormal; for T > 0 a
 *               uniform NaN or outside [0, 1); a row holding a NaN, a +inf or
 *               no finite value)
 * All pointers are device pointers owned by the caller; the call is
 * asynchronous on `stream` and allocates nothing (scratch is `workspace`,
 * 256-byte aligned, at least spec_sample_rows_workspace_bytes). Returns
 * SV_EINVAL (rows < 0, a null pointer, V out of range), SV_EDTYPE, SV_EALIGN
 * (logits not aligned to their element size), SV_ENOWS or SV_EHIP before or
 * at launch; nothing is enqueued on a host-side error.
 */
int spec_sample_rows(const void* logits, int32_t dtype, int32_t rows, int32_t V, const float* temperature,
                     const float* u, int32_t* out_tokens, void* workspace, size_t workspace_bytes, void* stream);

/*
 * KV commit after verification into a sink + ring cache.
 *
 * The cache keeps the first S positions in fixed slots and the most recent W
 * in a ring; position pos lives in slot Slot(pos) = pos for pos < S, else
 * S + ((pos - S) mod W) [Edge 环形上下文与注意力沉淀机制]. Per request the
 * pool holds, for each of R rows (R = layers * kv_heads), the S+W slots of E
 * bytes each: k_cache and v_cache are [B, R, S+W, E], as in the pool of
 * [Edge C++ 环形 KV 缓存管理内核实现] with one pool per request.
 *
 * The target pass that verified gamma drafts produced keys and values for the
 * gamma+1 positions P .. P+gamma (P = lengths[b]: the pending token, then the
 * drafts) [Primer 考点1]; the caller stages them in k_new and v_new,
 * [B, gamma+1, R, E]. Verification kept n = num_accepted[b] drafts, so the
 * request keeps n+1 positions [Primer 考点4]: positions P .. P+n are copied to
 * their slots (a later one wins when two share a slot, W < n+1) and
 * new_lengths[b] = P + n + 1. Rejected positions are never written, so the
 * window positions they would have displaced stay valid: the rollback costs
 * nothing. A request with n outside [0, gamma] (for instance the -1 that
 * verification reports for a bad request), a negative length, or a length that
 * would pass 2^31-1 writes nothing and keeps its length.
 *
 *   k_cache, v_cache  device, [B, R, S+W, E] bytes, updated in place
 *   k_new, v_new      device, [B, gamma+1, R, E] bytes, read
 *   lengths           device int32 [B], read
 *   num_accepted      device int32 [B] (the output of a verify call), read
 *   new_lengths       device int32 [B], written; must not overlap lengths
 *   rows = R >= 1, row_bytes = E in [1, SV_MAX_KV_ROW_BYTES], sink = S >= 0,
 *   window = W >= 1, S + W <= SV_MAX_KV_SLOTS, 0 <= gamma <= SV_MAX_GAMMA
 * The element type is the caller's: rows are copied as bytes (16-byte
 * accesses when E and every base pointer are 16-byte multiples). The caches
 * must not overlap each other or the staging buffers. Asynchronous on
 * `stream`, allocates nothing. Returns SV_EINVAL (bad size, null pointer,
 * k_cache == v_cache, overlapping length arrays) or SV_EHIP; nothing is
 * enqueued on a host-side error.
 */
int spec_kv_commit(void* k_cache, void* v_cache, const void* k_new, const void* v_new, const int32_t* lengths,
                   const int32_t* num_accepted, int32_t* new_lengths, int32_t B, int32_t gamma, int32_t rows,
                   int64_t row_bytes, int32_t sink, int32_t window, void* stream);

/*
 * The slots a sink + ring cache of length P holds, in logical order, for an
 * attention pass to read [Edge C++ 环形 KV 缓存管理内核实现]: while
 * P <= S+W, slots 0 .. P-1; after that the S sink slots, then the slots of
 * positions P-W .. P-1.
 *   lengths    device int32 [B]
 *   slots      device int32 [B, S+W]: the slots, -1 past the count
 *   positions  device int32 [B, S+W] or NULL: the logical position held in
 *              each listed slot (for position-dependent encodings), -1 past
 *              the count
 *   counts     device int32 [B]: min(max(P, 0), S+W)
 * Returns SV_EINVAL or SV_EHIP; asynchronous on `stream`.
 */
int spec_kv_valid_slots(const int32_t* lengths, int32_t B, int32_t sink, int32_t window, int32_t* slots,
                        int32_t* positions, int32_t* counts, void* stream);

/*
 * Draft-KV sliding window over a paged KV cache [Window 窗口数学; Window block
 * table 的裁剪方式; Window 两条贯穿始终的不变量].
 *
 * The draft model reads only a window of about W tokens ending K tokens past
 * the context length (K = future_offset: the draft query positions beyond
 * seq_lens); the target model and every KV write keep the full table. Per
 * request with length L: start = floor(max(L + K - W, 0) / b) * b (b =
 * block_size), windowed length L - start (at most W - K + b - 1), start block
 * start / b, blocks needed ceil((L - start) / b).
 *   seq_lens       device int32 [B]
 *   block_table    device int32 [B, full_cols], the full table (read only;
 *                  may be NULL when full_cols == 0)
 *   windowed_lens  device int32 [B]: L - start, -1 for a negative L; may be
 *                  seq_lens itself (in place), must not overlap it otherwise
 *   window_table   device int32 [B, window_cols]: row i holds
 *                  block_table[i, start_block + j] for j < needed while
 *                  start_block + j < full_cols, 0 elsewhere. Windowed index t
 *                  then addresses the same KV as absolute position start + t.
 * window_cols must be at least spec_draft_window_max_blocks(window,
 * block_size) = ceil((W + b - 1) / b), the most blocks a window can span
 * (W/b + 1 when b divides W). Requires W >= 1, b >= 1, 0 <= K <= W.
 * Returns SV_EINVAL or SV_EHIP; asynchronous on `stream`.
 */
int32_t spec_draft_window_max_blocks(int32_t window, int32_t block_size);
int spec_draft_window(const int32_t* seq_lens, int32_t B, int32_t window, int32_t block_size, int32_t future_offset,
                      const int32_t* block_table, int32_t full_cols, int32_t* windowed_lens, int32_t* window_table,
                      int32_t window_cols, void* stream);

/*
 * The same windowed length for HOST arrays (the host copies of the length
 * inputs of an attention pass), with the arithmetic of spec_draft_window, so
 * that every copy of a length gets one transform [Window 两条贯穿始终的不变量].
 * Synchronous; seq_lens and windowed_lens are host int32 [n] and may be the
 * same array.
 */
int spec_draft_window_host(const int32_t* seq_lens, int32_t n, int32_t window, int32_t block_size,
                           int32_t future_offset, int32_t* windowed_lens);

/*
 * Measurement aid, not a step of the method: reads `bytes` at `src` (device,
 * 16-byte aligned, a multiple of 16) with the load pattern of the streaming
 * statistics kernel and writes one folded word per wave to `out` (device,
 * spec_read_probe_words(bytes) words), so that the read rate this part
 * reaches in practice can be reported next to the HBM peak. Asynchronous on
 * `stream`; SV_EINVAL, SV_EALIGN or SV_EHIP.
 */
size_t spec_read_probe_words(size_t bytes);
int spec_read_probe(const void* src, size_t bytes, uint32_t* out, void* stream);

/* Human-readable text for an sv_status. */
const char* spec_verify_strerror(int status);

/* Library ABI version. */
int spec_verify_version(void);

/*
 * Optional timing of the streaming row-statistics kernel inside the calls
 * above (in spec_kv_commit and spec_draft_window: of their one kernel;
 * spec_verify_tree_lossless records two pairs, the streaming kernel's and then
 * the tree walk's). While recording is on, each call records a pair of HIP
 * events around that kernel on `stream`. spec_verify_timing_enable(1) starts or resumes recording,
 * spec_verify_timing_enable(0) pauses it (recorded pairs are kept),
 * spec_verify_timing_reset() forgets them. spec_verify_timing_read returns the
 * recorded per-call durations (ms), after the caller synchronised the stream;
 * at most `max` values are written and *count receives how many are available
 * (at most 4096 are kept). The first enable creates the events (host-side
 * allocation), so it is not meant for callers that forbid allocation. Not
 * thread-safe.
 */
int spec_verify_timing_enable(int enable);
int spec_verify_timing_reset(void);
int spec_verify_timing_read(float* ms_out, int32_t max, int32_t* count);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
