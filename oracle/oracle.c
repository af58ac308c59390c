/*
 * oracle.c -- plain, slow, double-precision CPU reference for batched
 * speculative-decoding verification (rejection sampling with residual /
 * bonus resampling).
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the bench's
 * CPU-baseline leg load this library. It shares no code, header, table or
 * helper with the HIP library, and the HIP library never calls it.
 *
 * Sources (cited by page and section; see the page list in the design notes):
 *   [Primer]  "猜想解码 (Speculative Decoding) 全景" (talentme.airsota.com),
 *             考点 1 (gamma+1 target positions per verify step),
 *             考点 2 (acceptance probability P_accept = min(1, P_t/P_d), the
 *             residual distribution P' = max(0, P_t-P_d)/sum, and the
 *             losslessness identity), 考点 4 (expected tokens with the
 *             always-produced extra token), 第二章 (acceptance formula with
 *             its two worked numbers), 第三章 (the per-position NumPy operator).
 *   [Edge]    lqnn.cn/news/249899, section "动态推迟投机验证调度器设计":
 *             temperature softmax exp((l - max)/T) / sum of the deferred
 *             verification scheduler, one temperature for both models.
 *
 * Readings where the pages leave a step open (each one is also listed in the
 * design notes):
 *   - accept iff u * P_d < P_t with u in [0,1): Bernoulli(min(1, P_t/P_d))
 *     written without a division, so P_d == 0 accepts iff P_t > 0;
 *   - no epsilons in any ratio or normaliser;
 *   - the residual is taken over probabilities, not over raw logits;
 *   - when every draft passes, one extra ("bonus") token is drawn from the
 *     last target row with the sampling uniform of that position;
 *   - inverse CDF: y = min{ j : C_j > u * S } with C the running sum in
 *     ascending token order; if rounding leaves no such j, y is the last
 *     token with positive mass;
 *   - a residual whose sum underflows to 0 falls back to P_t of that row (a
 *     diagnostic flag marks such requests);
 *   - temperature 0 means greedy: accept iff the draft token is the target
 *     argmax (lowest index on ties) and emit the argmax at the first
 *     mismatch;
 *   - a request whose inputs are unusable (temperature NaN, infinite,
 *     negative or subnormal; a token outside [0,V); for T > 0 a uniform
 *     that is NaN or outside [0,1); a logit row it reads holding a NaN or
 *     +inf or no finite value) gets num_accepted = -1 and -1 tokens.
 *
 * Every loop runs in ascending index order in double precision; requests are
 * split over threads, which does not change any request's arithmetic.
 */
#include <float.h>
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_F32 0
#define OR_BF16 1

/* Mutations for negative-control tests (planted mistakes; 0 = none). */
#define MUT_NONE 0
#define MUT_LOGIT_RESIDUAL 1 /* residual over raw logits, as in the edge page's listing */
#define MUT_RESAMPLE_TARGET 2 /* on rejection resample from P_t instead of P' */
#define MUT_ALWAYS_ACCEPT 3  /* accept every draft token */
#define MUT_NO_BONUS 4       /* all drafts accepted: resample last draft row's P_t instead of the bonus row */
#define MUT_TREE_NO_UPDATE 5  /* lossless tree: siblings all tested against P_t, draw against the first child */
#define MUT_TREE_NO_RENORM 6  /* lossless tree: the residual after a rejected sibling is not renormalised */

/* ------------------------------------------------------------------------ */
/* Input decoding: exact widening to double.                                 */

static double logit_at(const void *base, int dtype, size_t i)
{
    if (dtype == OR_F32)
        return (double)((const float *)base)[i];
    /* bfloat16: the 16 stored bits are the high half of an IEEE binary32 */
    uint32_t bits = (uint32_t)((const uint16_t *)base)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static int temperature_usable(float T)
{
    if (isnan(T) || isinf(T) || T < 0.0f)
        return 0;
    if (T > 0.0f && T < FLT_MIN) /* subnormal */
        return 0;
    return 1;
}

static int uniform_usable(float u)
{
    return !isnan(u) && u >= 0.0f && u < 1.0f;
}

/* A row is usable when it holds no NaN, no +inf and at least one finite value. */
static int row_usable(const void *base, int dtype, size_t off, int V)
{
    int finite_seen = 0;
    for (int j = 0; j < V; ++j) {
        double l = logit_at(base, dtype, off + (size_t)j);
        if (isnan(l) || l == INFINITY)
            return 0;
        if (l > -INFINITY)
            finite_seen = 1;
    }
    return finite_seen;
}

/* ------------------------------------------------------------------------ */
/* Softmax at temperature T [Edge, scheduler section]:
 *   m = max_j l_j,  p_j = exp((l_j - m)/T) / sum_k exp((l_k - m)/T).        */

static void softmax_row(const void *base, int dtype, size_t off, int V, double T, double *p,
                        double *m_out, double *Z_out)
{
    double m = -INFINITY;
    for (int j = 0; j < V; ++j) {
        double l = logit_at(base, dtype, off + (size_t)j);
        if (l > m)
            m = l;
    }
    double Z = 0.0;
    for (int j = 0; j < V; ++j) {
        double e = exp((logit_at(base, dtype, off + (size_t)j) - m) / T);
        p[j] = e;
        Z += e;
    }
    for (int j = 0; j < V; ++j)
        p[j] /= Z;
    if (m_out)
        *m_out = m;
    if (Z_out)
        *Z_out = Z;
}

/* Greedy decoding picks the first index holding the maximum. */
static int argmax_row(const void *base, int dtype, size_t off, int V)
{
    double m = -INFINITY;
    int a = -1;
    for (int j = 0; j < V; ++j) {
        double l = logit_at(base, dtype, off + (size_t)j);
        if (l > m) {
            m = l;
            a = j;
        }
    }
    return a;
}

/* ------------------------------------------------------------------------ */
/* Inverse-CDF draw from unnormalised masses q (all >= 0, sum S > 0):
 * y = min{ j : C_j > u*S }, C_j = q_0 + ... + q_j.  If no such j exists the
 * last index with q_j > 0 is returned.  *margin receives the distance of
 * u*S to the nearer edge of y's interval, divided by S.                     */

static int inverse_cdf(const double *q, int V, double u, double *margin)
{
    double S = 0.0;
    for (int j = 0; j < V; ++j)
        S += q[j];
    double thr = u * S;
    double C = 0.0;
    for (int j = 0; j < V; ++j) {
        double prev = C;
        C += q[j];
        if (C > thr) {
            double lo = thr - prev, hi = C - thr;
            *margin = (lo < hi ? lo : hi) / S;
            return j;
        }
    }
    int last = -1;
    for (int j = 0; j < V; ++j)
        if (q[j] > 0.0)
            last = j;
    *margin = 0.0;
    return last;
}

/* ------------------------------------------------------------------------ */
/* One linear (chain) request.                                               */

typedef struct {
    const void *target; /* row i of this request at target + trow0*V        */
    const void *draft;  /* row i of this request at draft  + drow0*V        */
    int dtype;
    size_t trow0, drow0;
    int gamma, V;
    const int32_t *tokens; /* [gamma] */
    const float *ua;       /* [gamma] */
    const float *us;       /* [gamma+1] */
    float T;
    int mutant;
    /* outputs */
    int32_t *out;  /* [width] */
    int width;
    int32_t *num_accepted;
    double *pt_diag, *pd_diag; /* [gamma] or NULL */
    double *acc_margin;        /* min |u - min(1,r)| over examined positions */
    double *cdf_margin;
    int32_t *fallback;         /* 1 when the draw fell back to P_t (zero residual sum) */
} chain_req;

static void fail_request(int32_t *out, int width, int32_t *num_accepted)
{
    for (int k = 0; k < width; ++k)
        out[k] = -1;
    *num_accepted = -1;
}

static void verify_chain_one(const chain_req *r, double *work)
{
    const int g = r->gamma, V = r->V;
    if (r->pt_diag)
        for (int i = 0; i < g; ++i)
            r->pt_diag[i] = r->pd_diag[i] = NAN;
    *r->acc_margin = INFINITY;
    *r->cdf_margin = INFINITY;
    *r->fallback = 0;

    /* Validation of everything the request reads. */
    int ok = temperature_usable(r->T);
    for (int i = 0; ok && i < g; ++i)
        if (r->tokens[i] < 0 || r->tokens[i] >= V)
            ok = 0;
    if (ok && r->T > 0.0f) {
        for (int i = 0; ok && i < g; ++i)
            ok = uniform_usable(r->ua[i]);
        for (int i = 0; ok && i <= g; ++i)
            ok = uniform_usable(r->us[i]);
    }
    for (int i = 0; ok && i <= g; ++i)
        ok = row_usable(r->target, r->dtype, (r->trow0 + (size_t)i) * (size_t)V, V);
    if (ok && r->T > 0.0f)
        for (int i = 0; ok && i < g; ++i)
            ok = row_usable(r->draft, r->dtype, (r->drow0 + (size_t)i) * (size_t)V, V);
    if (!ok) {
        fail_request(r->out, r->width, r->num_accepted);
        return;
    }
    for (int k = 0; k < r->width; ++k)
        r->out[k] = -1;

    if (r->T == 0.0f) {
        /* Greedy: accept while the draft token equals the target argmax. */
        int n = g, y = -1;
        for (int i = 0; i <= g; ++i) {
            int a = argmax_row(r->target, r->dtype, (r->trow0 + (size_t)i) * (size_t)V, V);
            if (i == g || r->tokens[i] != a) {
                n = i;
                y = a;
                break;
            }
        }
        for (int i = 0; i < n; ++i)
            r->out[i] = r->tokens[i];
        r->out[n] = y;
        *r->num_accepted = n;
        return;
    }

    /* Sampling: p_t for rows 0..gamma, p_d for rows 0..gamma-1. */
    const double T = (double)r->T;
    double *pt = work;                          /* [(gamma+1) * V] */
    double *pd = work + (size_t)(g + 1) * V;    /* [gamma * V]     */
    double *q = pd + (size_t)g * V;             /* [V]             */
    for (int i = 0; i <= g; ++i)
        softmax_row(r->target, r->dtype, (r->trow0 + (size_t)i) * (size_t)V, V, T, pt + (size_t)i * V,
                    NULL, NULL);
    for (int i = 0; i < g; ++i)
        softmax_row(r->draft, r->dtype, (r->drow0 + (size_t)i) * (size_t)V, V, T, pd + (size_t)i * V,
                    NULL, NULL);
    if (r->pt_diag)
        for (int i = 0; i < g; ++i) {
            r->pt_diag[i] = pt[(size_t)i * V + r->tokens[i]];
            r->pd_diag[i] = pd[(size_t)i * V + r->tokens[i]];
        }

    /* Acceptance scan [Primer 考点2 / 第二章]: accept x_i with probability
     * min(1, P_t/P_d); stop at the first rejection. */
    int n = g;
    for (int i = 0; i < g; ++i) {
        double Pt = pt[(size_t)i * V + r->tokens[i]];
        double Pd = pd[(size_t)i * V + r->tokens[i]];
        double u = (double)r->ua[i];
        double ratio = Pd > 0.0 ? fmin(1.0, Pt / Pd) : (Pt > 0.0 ? 1.0 : 0.0);
        double d = fabs(u - ratio);
        if (d < *r->acc_margin)
            *r->acc_margin = d;
        int accept = (u * Pd < Pt);
        if (r->mutant == MUT_ALWAYS_ACCEPT)
            accept = 1;
        if (!accept) {
            n = i;
            break;
        }
    }

    /* Distribution of the token at position n. */
    const double *ptn = pt + (size_t)n * V;
    if (n < g) {
        /* Residual P' proportional to max(0, P_t - P_d) [Primer 考点2]. */
        const double *pdn = pd + (size_t)n * V;
        for (int j = 0; j < V; ++j)
            q[j] = fmax(0.0, ptn[j] - pdn[j]);
        if (r->mutant == MUT_RESAMPLE_TARGET)
            for (int j = 0; j < V; ++j)
                q[j] = ptn[j];
        if (r->mutant == MUT_LOGIT_RESIDUAL) {
            size_t to = (r->trow0 + (size_t)n) * (size_t)V, dof = (r->drow0 + (size_t)n) * (size_t)V;
            for (int j = 0; j < V; ++j)
                q[j] = fmax(0.0, logit_at(r->target, r->dtype, to + j) - logit_at(r->draft, r->dtype, dof + j));
        }
    } else {
        /* Bonus token from the last target row. */
        const double *src = ptn;
        if (r->mutant == MUT_NO_BONUS && g > 0)
            src = pt + (size_t)(g - 1) * V;
        for (int j = 0; j < V; ++j)
            q[j] = src[j];
    }
    double S = 0.0;
    for (int j = 0; j < V; ++j)
        S += q[j];
    if (!(S > 0.0)) {
        for (int j = 0; j < V; ++j)
            q[j] = ptn[j]; /* residual underflow: fall back to P_t of row n */
        *r->fallback = 1;
    }

    double margin;
    int y = inverse_cdf(q, V, (double)r->us[n], &margin);
    *r->cdf_margin = margin;
    for (int i = 0; i < n; ++i)
        r->out[i] = r->tokens[i];
    r->out[n] = y;
    *r->num_accepted = n;
}

/* ------------------------------------------------------------------------ */
/* Threading over requests (static interleave; each request is computed
 * entirely by one thread, so results do not depend on the thread count).    */

typedef struct {
    int nthreads, tid;
    void (*fn)(void *ctx, int b, double *work);
    void *ctx;
    int B;
    size_t work_doubles;
    int failed;
} worker_arg;

static void *worker_main(void *p)
{
    worker_arg *w = (worker_arg *)p;
    double *work = (double *)malloc(w->work_doubles * sizeof(double) + 64);
    if (!work) {
        w->failed = 1;
        return NULL;
    }
    for (int b = w->tid; b < w->B; b += w->nthreads)
        w->fn(w->ctx, b, work);
    free(work);
    return NULL;
}

static int run_parallel(int B, int nthreads, size_t work_doubles, void (*fn)(void *, int, double *), void *ctx)
{
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > B)
        nthreads = B > 0 ? B : 1;
    pthread_t th[256];
    worker_arg args[256];
    if (nthreads > 256)
        nthreads = 256;
    for (int t = 0; t < nthreads; ++t) {
        args[t] = (worker_arg){nthreads, t, fn, ctx, B, work_doubles, 0};
        if (t > 0 && pthread_create(&th[t], NULL, worker_main, &args[t]) != 0)
            return -1;
    }
    worker_main(&args[0]);
    int failed = args[0].failed;
    for (int t = 1; t < nthreads; ++t) {
        pthread_join(th[t], NULL);
        failed |= args[t].failed;
    }
    return failed ? -1 : 0;
}

/* ------------------------------------------------------------------------ */
/* Dense and ragged chain verification.                                      */

typedef struct {
    const void *target, *draft;
    int dtype;
    const int32_t *tokens;
    const float *ua, *us, *temperature;
    const int32_t *cu; /* NULL for dense */
    int total_draft;
    int B, gamma, V, mutant;
    int32_t *out, *num_accepted;
    double *pt_diag, *pd_diag, *acc_margin, *cdf_margin;
    int32_t *fallback;
} chain_batch;

/* The packed layout describes the whole batch: it is usable only when
 * cu[0] == 0, cu never decreases, every gamma_b <= gamma_max and
 * cu[B] == total_draft; otherwise no request can be located reliably. */
static int ragged_layout_valid(const int32_t *cu, int B, int gamma_max, int total_draft)
{
    if (cu[0] != 0 || cu[B] != total_draft)
        return 0;
    for (int b = 0; b < B; ++b)
        if (cu[b + 1] < cu[b] || cu[b + 1] - cu[b] > gamma_max)
            return 0;
    return 1;
}

static void chain_task(void *p, int b, double *work)
{
    const chain_batch *cb = (const chain_batch *)p;
    const int width = cb->gamma + 1;
    chain_req r;
    memset(&r, 0, sizeof r);
    int gb;
    size_t d0;
    if (cb->cu) {
        int lo = cb->cu[b], hi = cb->cu[b + 1];
        if (!ragged_layout_valid(cb->cu, cb->B, cb->gamma, cb->total_draft)) {
            fail_request(cb->out + (size_t)b * width, width, cb->num_accepted + b);
            cb->acc_margin[b] = cb->cdf_margin[b] = INFINITY;
            cb->fallback[b] = 0;
            return;
        }
        gb = hi - lo;
        d0 = (size_t)lo;
        r.trow0 = (size_t)lo + (size_t)b;
    } else {
        gb = cb->gamma;
        d0 = (size_t)b * (size_t)cb->gamma;
        r.trow0 = (size_t)b * (size_t)(cb->gamma + 1);
    }
    r.target = cb->target;
    r.draft = cb->draft;
    r.dtype = cb->dtype;
    r.drow0 = d0;
    r.gamma = gb;
    r.V = cb->V;
    r.tokens = cb->tokens + d0;
    r.ua = cb->ua + d0;
    r.us = cb->us + r.trow0;
    r.T = cb->temperature[b];
    r.mutant = cb->mutant;
    r.out = cb->out + (size_t)b * width;
    r.width = width;
    r.num_accepted = cb->num_accepted + b;
    r.pt_diag = cb->pt_diag ? cb->pt_diag + d0 : NULL;
    r.pd_diag = cb->pd_diag ? cb->pd_diag + d0 : NULL;
    r.acc_margin = cb->acc_margin + b;
    r.cdf_margin = cb->cdf_margin + b;
    r.fallback = cb->fallback + b;
    verify_chain_one(&r, work);
}

/* Dense: target [B, gamma+1, V], draft [B, gamma, V], tokens/ua [B, gamma],
 * us [B, gamma+1]; ragged (cu != NULL): packed rows, request b owns draft rows
 * cu[b]..cu[b+1]-1 and target rows cu[b]+b .. cu[b+1]+b, gamma = gamma_max.
 * out [B, gamma+1]; diag arrays are indexed like the draft rows; fallback [B] marks
 * the requests whose draw fell back to P_t because the residual summed to 0.  */
int oracle_verify_chain(const void *target, const void *draft, int dtype, const int32_t *tokens,
                        const float *u_accept, const float *u_sample, const float *temperature,
                        const int32_t *cu_gamma, int total_draft, int B, int gamma, int V, int32_t *out,
                        int32_t *num_accepted, double *pt_diag, double *pd_diag, double *acc_margin,
                        double *cdf_margin, int32_t *fallback, int mutant, int nthreads)
{
    if (B < 0 || gamma < 0 || V < 1 || (dtype != OR_F32 && dtype != OR_BF16))
        return -1;
    chain_batch cb = {target, draft,  dtype, tokens,      u_accept,     u_sample,     temperature,
                      cu_gamma, total_draft, B, gamma, V, mutant, out, num_accepted, pt_diag,
                      pd_diag, acc_margin, cdf_margin, fallback};
    size_t work = (size_t)(2 * gamma + 2) * (size_t)V;
    return run_parallel(B, nthreads, work, chain_task, &cb);
}

/* ------------------------------------------------------------------------ */
/* Token-tree verification.  Node v >= 1 has parent parents[v] < v (node 0 is
 * the root, parents[0] = -1).  Target row v is the target distribution of the
 * token after the path to v; draft row v-1 is the distribution node v's token
 * was drawn from.  Each node is tested against its parent's target row, the
 * accepted nodes form the ok-set (node and all its ancestors accepted), the
 * end node is the deepest ok node (lowest index on ties) and the final token
 * is a bonus draw from the end node's target row when it has no children,
 * else a residual draw against the draft row of its lowest-index child.       */

typedef struct {
    const void *target, *draft;
    int dtype;
    const int32_t *tokens, *parents;
    const float *ua, *us, *temperature;
    int B, N, V, max_depth;
    int32_t *out, *out_nodes, *num_accepted;
    double *acc_margin, *cdf_margin;
    int mutant;
    int32_t *fallback; /* 1: zero residual sum (lowest-child rule: draw from P_t[e];
                          lossless walk: a rejected sibling left r unchanged) */
} tree_batch;

static void tree_task(void *p, int b, double *work)
{
    const tree_batch *tb = (const tree_batch *)p;
    const int N = tb->N, V = tb->V, width = tb->max_depth + 1;
    int32_t *out = tb->out + (size_t)b * width, *onodes = tb->out_nodes + (size_t)b * width;
    const int32_t *par = tb->parents + (size_t)b * N, *tok = tb->tokens + (size_t)b * N;
    const float *ua = tb->ua + (size_t)b * N, *us = tb->us + (size_t)b * N;
    const float Tf = tb->temperature[b];
    const size_t t0 = (size_t)b * N, d0 = (size_t)b * (N - 1);
    tb->acc_margin[b] = INFINITY;
    tb->cdf_margin[b] = INFINITY;
    tb->fallback[b] = 0;
    for (int k = 0; k < width; ++k)
        onodes[k] = -1;

    int *depth = (int *)(work);               /* 3N ints in the first 2N doubles */
    int *okn = depth + N;
    int *amax = okn + N;                       /* greedy argmax per target row */
    double *dwork = work + 2 * (size_t)N;

    int ok = temperature_usable(Tf) && par[0] == -1;
    depth[0] = 0;
    for (int v = 1; ok && v < N; ++v) {
        if (par[v] < 0 || par[v] >= v) {
            ok = 0;
            break;
        }
        depth[v] = depth[par[v]] + 1;
        if (depth[v] > tb->max_depth)
            ok = 0;
        if (tok[v] < 0 || tok[v] >= V)
            ok = 0;
    }
    if (ok && Tf > 0.0f) {
        for (int v = 1; ok && v < N; ++v)
            ok = uniform_usable(ua[v]);
        for (int v = 0; ok && v < N; ++v)
            ok = uniform_usable(us[v]);
    }
    for (int v = 0; ok && v < N; ++v)
        ok = row_usable(tb->target, tb->dtype, (t0 + v) * (size_t)V, V);
    if (ok && Tf > 0.0f)
        for (int v = 1; ok && v < N; ++v)
            ok = row_usable(tb->draft, tb->dtype, (d0 + v - 1) * (size_t)V, V);
    if (!ok) {
        fail_request(out, width, tb->num_accepted + b);
        return;
    }
    for (int k = 0; k < width; ++k)
        out[k] = -1;

    /* Per-node acceptance and the ok-set. */
    double *pt = dwork;                        /* [N * V] */
    double *pd = pt + (size_t)N * V;           /* [N * V], row v for node v */
    double *q = pd + (size_t)N * V;            /* [V] */
    const double T = (double)Tf;
    if (T > 0.0) {
        for (int v = 0; v < N; ++v)
            softmax_row(tb->target, tb->dtype, (t0 + v) * (size_t)V, V, T, pt + (size_t)v * V, NULL, NULL);
        for (int v = 1; v < N; ++v)
            softmax_row(tb->draft, tb->dtype, (d0 + v - 1) * (size_t)V, V, T, pd + (size_t)v * V, NULL, NULL);
    } else {
        for (int v = 0; v < N; ++v)
            amax[v] = argmax_row(tb->target, tb->dtype, (t0 + v) * (size_t)V, V);
    }
    okn[0] = 1;
    for (int v = 1; v < N; ++v) {
        int u = par[v], accept;
        if (T > 0.0) {
            double Pt = pt[(size_t)u * V + tok[v]], Pd = pd[(size_t)v * V + tok[v]];
            accept = ((double)ua[v] * Pd < Pt);
            if (okn[u]) {
                double ratio = Pd > 0.0 ? fmin(1.0, Pt / Pd) : (Pt > 0.0 ? 1.0 : 0.0);
                double d = fabs((double)ua[v] - ratio);
                if (d < tb->acc_margin[b])
                    tb->acc_margin[b] = d;
            }
        } else {
            accept = (tok[v] == amax[u]);
        }
        okn[v] = accept && okn[u];
    }
    int e = 0;
    for (int v = 1; v < N; ++v)
        if (okn[v] && depth[v] > depth[e])
            e = v;
    int d = depth[e];
    for (int v = e, k = d - 1; v != 0; v = par[v], --k) {
        out[k] = tok[v];
        onodes[k] = v;
    }

    int y;
    if (T == 0.0) {
        y = amax[e];
    } else {
        int c = -1;
        for (int v = 1; v < N; ++v)
            if (par[v] == e) {
                c = v;
                break;
            }
        const double *pte = pt + (size_t)e * V;
        if (c < 0) {
            for (int j = 0; j < V; ++j)
                q[j] = pte[j];
        } else {
            const double *pdc = pd + (size_t)c * V;
            for (int j = 0; j < V; ++j)
                q[j] = fmax(0.0, pte[j] - pdc[j]);
        }
        double S = 0.0;
        for (int j = 0; j < V; ++j)
            S += q[j];
        if (!(S > 0.0)) {
            for (int j = 0; j < V; ++j)
                q[j] = pte[j]; /* residual underflow: fall back to P_t of the end node */
            tb->fallback[b] = 1;
        }
        double margin;
        y = inverse_cdf(q, V, (double)us[e], &margin);
        tb->cdf_margin[b] = margin;
    }
    out[d] = y;
    tb->num_accepted[b] = d;
}

/* target [B, N, V]; draft [B, N-1, V] (row v-1 for node v); tokens, parents,
 * ua, us [B, N]; out and out_nodes [B, max_depth+1].                        */
int oracle_verify_tree(const void *target, const void *draft, int dtype, const int32_t *tokens,
                       const int32_t *parents, const float *u_accept, const float *u_sample,
                       const float *temperature, int B, int N, int V, int max_depth, int32_t *out,
                       int32_t *out_nodes, int32_t *num_accepted, double *acc_margin, double *cdf_margin,
                       int32_t *fallback, int nthreads)
{
    if (B < 0 || N < 1 || V < 1 || max_depth < 0 || (dtype != OR_F32 && dtype != OR_BF16))
        return -1;
    tree_batch tb = {target,      draft,      dtype,     tokens, parents,   u_accept,     u_sample,
                     temperature, B,          N,         V,      max_depth, out,          out_nodes,
                     num_accepted, acc_margin, cdf_margin, MUT_NONE, fallback};
    size_t work = 2 * (size_t)N + (size_t)(2 * N + 1) * (size_t)V;
    return run_parallel(B, nthreads, work, tree_task, &tb);
}

/* ------------------------------------------------------------------------ */
/* Lossless multi-candidate token-tree verification.  The tree layout, the
 * validation and the row conventions are those of oracle_verify_tree.  At the
 * current node v (from the root) the current distribution is r = P_t[v]; the
 * children of v are tried in ascending index order, each with the acceptance
 * rule of [Primer 考点2] against r: child c is accepted when
 * u_accept[c] * P_d[c](x_c) < r(x_c).  An accepted child becomes the current
 * node.  A rejected child replaces r by its residual max(0, r - P_d[c]) / sum
 * [Primer 考点2, P'] before the next sibling is tried; a residual whose sum
 * underflows to 0 leaves r unchanged.  When no child is accepted (or v has no
 * children) the final token is drawn from r with u_sample[v] by the inverse
 * CDF.  Each step's output then follows P_t whatever the draft rows are, as
 * long as each child's token was drawn from its own draft row independently of
 * the others.  Greedy (T == 0): the first child whose token is the argmax of
 * P_t[v] is accepted; otherwise the argmax is emitted.                      */

static void tree_lossless_task(void *p, int b, double *work)
{
    const tree_batch *tb = (const tree_batch *)p;
    const int N = tb->N, V = tb->V, width = tb->max_depth + 1;
    int32_t *out = tb->out + (size_t)b * width, *onodes = tb->out_nodes + (size_t)b * width;
    const int32_t *par = tb->parents + (size_t)b * N, *tok = tb->tokens + (size_t)b * N;
    const float *ua = tb->ua + (size_t)b * N, *us = tb->us + (size_t)b * N;
    const float Tf = tb->temperature[b];
    const size_t t0 = (size_t)b * N, d0 = (size_t)b * (N - 1);
    tb->acc_margin[b] = INFINITY;
    tb->cdf_margin[b] = INFINITY;
    tb->fallback[b] = 0;
    for (int k = 0; k < width; ++k)
        onodes[k] = -1;

    int *depth = (int *)(work);
    int *amax = depth + N;
    double *dwork = work + 2 * (size_t)N;

    int ok = temperature_usable(Tf) && par[0] == -1;
    depth[0] = 0;
    for (int v = 1; ok && v < N; ++v) {
        if (par[v] < 0 || par[v] >= v) {
            ok = 0;
            break;
        }
        depth[v] = depth[par[v]] + 1;
        if (depth[v] > tb->max_depth)
            ok = 0;
        if (tok[v] < 0 || tok[v] >= V)
            ok = 0;
    }
    if (ok && Tf > 0.0f) {
        for (int v = 1; ok && v < N; ++v)
            ok = uniform_usable(ua[v]);
        for (int v = 0; ok && v < N; ++v)
            ok = uniform_usable(us[v]);
    }
    for (int v = 0; ok && v < N; ++v)
        ok = row_usable(tb->target, tb->dtype, (t0 + v) * (size_t)V, V);
    if (ok && Tf > 0.0f)
        for (int v = 1; ok && v < N; ++v)
            ok = row_usable(tb->draft, tb->dtype, (d0 + v - 1) * (size_t)V, V);
    if (!ok) {
        fail_request(out, width, tb->num_accepted + b);
        return;
    }
    for (int k = 0; k < width; ++k)
        out[k] = -1;

    int v = 0, d = 0;
    if (Tf == 0.0f) {
        for (int w = 0; w < N; ++w)
            amax[w] = argmax_row(tb->target, tb->dtype, (t0 + w) * (size_t)V, V);
        for (;;) {
            int next = -1;
            for (int c = 1; c < N; ++c)
                if (par[c] == v && tok[c] == amax[v]) {
                    next = c;
                    break;
                }
            if (next < 0)
                break;
            out[d] = tok[next];
            onodes[d] = next;
            ++d;
            v = next;
        }
        out[d] = amax[v];
        tb->num_accepted[b] = d;
        return;
    }

    const double T = (double)Tf;
    double *r = dwork;        /* [V] current distribution */
    double *q = r + V;        /* [V] draft distribution of the child under test */
    double *res = q + V;      /* [V] residual */
    double *first = res + V;  /* [V] draft distribution of the first child (planted mistake) */
    for (;;) {
        softmax_row(tb->target, tb->dtype, (t0 + v) * (size_t)V, V, T, r, NULL, NULL);
        int accepted = -1, nrej = 0;
        for (int c = 1; c < N; ++c) {
            if (par[c] != v)
                continue;
            softmax_row(tb->draft, tb->dtype, (d0 + c - 1) * (size_t)V, V, T, q, NULL, NULL);
            const int x = tok[c];
            const double Pt = r[x], Pd = q[x];
            double ratio = Pd > 0.0 ? fmin(1.0, Pt / Pd) : (Pt > 0.0 ? 1.0 : 0.0);
            double dm = fabs((double)ua[c] - ratio);
            if (dm < tb->acc_margin[b])
                tb->acc_margin[b] = dm;
            if ((double)ua[c] * Pd < Pt) {
                accepted = c;
                break;
            }
            if (nrej++ == 0)
                memcpy(first, q, (size_t)V * sizeof(double));
            if (tb->mutant == MUT_TREE_NO_UPDATE)
                continue;
            double Z = 0.0;
            for (int j = 0; j < V; ++j) {
                res[j] = fmax(0.0, r[j] - q[j]);
                Z += res[j];
            }
            if (Z > 0.0)
                for (int j = 0; j < V; ++j)
                    r[j] = tb->mutant == MUT_TREE_NO_RENORM ? res[j] : res[j] / Z;
            else
                tb->fallback[b] = 1; /* residual underflow: r is kept */
        }
        if (accepted < 0) {
            if (tb->mutant == MUT_TREE_NO_UPDATE && nrej > 0) {
                double Z = 0.0;
                for (int j = 0; j < V; ++j) {
                    res[j] = fmax(0.0, r[j] - first[j]);
                    Z += res[j];
                }
                if (Z > 0.0)
                    memcpy(r, res, (size_t)V * sizeof(double));
            }
            break;
        }
        out[d] = tok[accepted];
        onodes[d] = accepted;
        ++d;
        v = accepted;
    }
    double margin;
    out[d] = inverse_cdf(r, V, (double)us[v], &margin);
    tb->cdf_margin[b] = margin;
    tb->num_accepted[b] = d;
}

/* Same arguments as oracle_verify_tree, plus a planted-mistake selector. */
int oracle_verify_tree_lossless(const void *target, const void *draft, int dtype, const int32_t *tokens,
                                const int32_t *parents, const float *u_accept, const float *u_sample,
                                const float *temperature, int B, int N, int V, int max_depth, int32_t *out,
                                int32_t *out_nodes, int32_t *num_accepted, double *acc_margin, double *cdf_margin,
                                int32_t *fallback, int mutant, int nthreads)
{
    if (B < 0 || N < 1 || V < 1 || max_depth < 0 || (dtype != OR_F32 && dtype != OR_BF16))
        return -1;
    tree_batch tb = {target,      draft,      dtype,     tokens, parents,   u_accept,     u_sample,
                     temperature, B,          N,         V,      max_depth, out,          out_nodes,
                     num_accepted, acc_margin, cdf_margin, mutant, fallback};
    size_t work = 2 * (size_t)N + 4 * (size_t)V;
    return run_parallel(B, nthreads, work, tree_lossless_task, &tb);
}

/* ------------------------------------------------------------------------ */
/* Per-row statistics: max m, log Z with Z = sum exp((l - m)/T) (T > 0), and
 * the lowest-index argmax (T == 0).  Unusable rows report valid = 0.        */

typedef struct {
    const void *logits;
    int dtype, V;
    const float *temperature;
    double *m, *logZ;
    int32_t *argmax, *valid;
} stats_batch;

static void stats_task(void *p, int row, double *work)
{
    const stats_batch *sb = (const stats_batch *)p;
    size_t off = (size_t)row * sb->V;
    float T = sb->temperature[row];
    sb->m[row] = NAN;
    sb->logZ[row] = NAN;
    sb->argmax[row] = -1;
    sb->valid[row] = 0;
    if (!temperature_usable(T) || !row_usable(sb->logits, sb->dtype, off, sb->V))
        return;
    sb->valid[row] = 1;
    if (T == 0.0f) {
        int a = argmax_row(sb->logits, sb->dtype, off, sb->V);
        sb->argmax[row] = a;
        sb->m[row] = logit_at(sb->logits, sb->dtype, off + a);
        return;
    }
    double m, Z;
    softmax_row(sb->logits, sb->dtype, off, sb->V, (double)T, work, &m, &Z);
    sb->m[row] = m;
    sb->logZ[row] = log(Z);
}

int oracle_row_stats(const void *logits, int dtype, int rows, int V, const float *temperature, double *m,
                     double *logZ, int32_t *argmax, int32_t *valid, int nthreads)
{
    if (rows < 0 || V < 1 || (dtype != OR_F32 && dtype != OR_BF16))
        return -1;
    stats_batch sb = {logits, dtype, V, temperature, m, logZ, argmax, valid};
    return run_parallel(rows, nthreads, (size_t)V, stats_task, &sb);
}

/* ------------------------------------------------------------------------ */
/* Draft-token sampling: one token per row from p = softmax(l/T) [Edge,
 * scheduler section: the temperature softmax both models use], the way the
 * draft model proposes the tokens that verification then tests [Primer 考点1:
 * the draft model generates the gamma tokens one by one].  The draw is the
 * verify draw's inverse CDF, y = min{ j : C_j > u*S } over p in ascending
 * token order; T == 0 takes the lowest-index argmax.  A row whose
 * temperature, uniform (T > 0) or logits are unusable gives -1.  margin[r]
 * is the distance of u*S to the nearer edge of y's interval over S (NaN for
 * greedy and unusable rows).                                                */

typedef struct {
    const void *logits;
    int dtype, V;
    const float *temperature, *u;
    int32_t *out;
    double *margin;
} sample_batch;

static void sample_task(void *p, int row, double *work)
{
    const sample_batch *sb = (const sample_batch *)p;
    size_t off = (size_t)row * sb->V;
    float T = sb->temperature[row];
    sb->out[row] = -1;
    sb->margin[row] = NAN;
    if (!temperature_usable(T) || !row_usable(sb->logits, sb->dtype, off, sb->V))
        return;
    if (T == 0.0f) {
        sb->out[row] = argmax_row(sb->logits, sb->dtype, off, sb->V);
        return;
    }
    if (!uniform_usable(sb->u[row]))
        return;
    softmax_row(sb->logits, sb->dtype, off, sb->V, (double)T, work, NULL, NULL);
    sb->out[row] = inverse_cdf(work, sb->V, (double)sb->u[row], &sb->margin[row]);
}

int oracle_sample_rows(const void *logits, int dtype, int rows, int V, const float *temperature, const float *u,
                       int32_t *out, double *margin, int nthreads)
{
    if (rows < 0 || V < 1 || (dtype != OR_F32 && dtype != OR_BF16))
        return -1;
    sample_batch sb = {logits, dtype, V, temperature, u, out, margin};
    return run_parallel(rows, nthreads, (size_t)V, sample_task, &sb);
}

int oracle_version(void) { return 1; }
