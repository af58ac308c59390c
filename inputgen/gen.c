/*
 * gen.c -- seeded synthetic inputs for the verify path (logit rows, draft
 * tokens, uniforms). Shared by the tests, the bench and the smoke check; it
 * holds none of the verification arithmetic (no softmax normaliser, no
 * acceptance test, no residual, no inverse CDF).
 *
 * Randomness: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
 * numbers: as easy as 1, 2, 3", SC'11), a counter-based generator: every value
 * is a pure function of (seed, stream, row, column), so results do not depend
 * on thread count or generation order.
 *   counter = (column, row low 32 bits, row high 32 bits, stream)
 *   key     = (seed low 32 bits, seed high 32 bits)
 * Normals: Box-Muller on two 53-bit uniforms. Student-t(3): Z / sqrt(chi2_3/3)
 * with chi2_3 the sum of three squared normals. bf16: round to nearest even.
 * Draft tokens: Gumbel-max, x = argmax_j (l_j/T + G_j) with G_j = -log(-log U_j),
 * which draws exactly from softmax(l/T); T == 0 takes the lowest-index argmax.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Philox4x32-10                                                             */

static inline void mulhilo32(uint32_t a, uint32_t b, uint32_t *hi, uint32_t *lo)
{
    uint64_t p = (uint64_t)a * (uint64_t)b;
    *hi = (uint32_t)(p >> 32);
    *lo = (uint32_t)p;
}

void ig_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4])
{
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int r = 0; r < 10; ++r) {
        uint32_t hi0, lo0, hi1, lo1;
        mulhilo32(0xD2511F53u, c0, &hi0, &lo0);
        mulhilo32(0xCD9E8D57u, c2, &hi1, &lo1);
        uint32_t n0 = hi1 ^ c1 ^ k0, n1 = lo1, n2 = hi0 ^ c3 ^ k1, n3 = lo0;
        c0 = n0;
        c1 = n1;
        c2 = n2;
        c3 = n3;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    out[0] = c0;
    out[1] = c1;
    out[2] = c2;
    out[3] = c3;
}

static inline void draw4(uint64_t seed, uint32_t stream, uint64_t row, uint32_t col, uint32_t w[4])
{
    uint32_t ctr[4] = {col, (uint32_t)row, (uint32_t)(row >> 32), stream};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    ig_philox4x32_10(ctr, key, w);
}

static inline double u53(uint32_t hi, uint32_t lo) /* in (0,1) */
{
    uint64_t v = (((uint64_t)hi << 32) | lo) >> 11;
    return ((double)v + 0.5) * 0x1p-53;
}

/* Two standard normals from one counter value (Box-Muller). */
static inline void normal2(uint64_t seed, uint32_t stream, uint64_t row, uint32_t col, double z[2])
{
    uint32_t w[4];
    draw4(seed, stream, row, col, w);
    double a = u53(w[0], w[1]), b = u53(w[2], w[3]);
    double r = sqrt(-2.0 * log(a)), t = 6.283185307179586476925 * b;
    z[0] = r * cos(t);
    z[1] = r * sin(t);
}

static inline double normal_at(uint64_t seed, uint32_t stream, uint64_t row, uint64_t j)
{
    double z[2];
    normal2(seed, stream, row, (uint32_t)(j >> 1), z);
    return z[j & 1];
}

static inline double student_t3_at(uint64_t seed, uint32_t stream, uint64_t row, uint64_t j)
{
    double z[2], w[2];
    normal2(seed, stream, row, (uint32_t)(2 * j), z);
    normal2(seed, stream, row, (uint32_t)(2 * j + 1), w);
    double chi2 = z[1] * z[1] + w[0] * w[0] + w[1] * w[1];
    return z[0] / sqrt(chi2 / 3.0);
}

static inline uint16_t bf16_rne(float f)
{
    uint32_t b;
    memcpy(&b, &f, 4);
    if ((b & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((b >> 16) | 0x40u); /* quiet NaN */
    b += 0x7fffu + ((b >> 16) & 1u);
    return (uint16_t)(b >> 16);
}

/* ------------------------------------------------------------------------ */
/* Thread helper                                                             */

typedef struct {
    int64_t n;
    int tid, nt;
    void (*fn)(void *, int64_t, int64_t);
    void *ctx;
} job;

static void *job_main(void *p)
{
    job *j = (job *)p;
    int64_t per = (j->n + j->nt - 1) / j->nt;
    int64_t lo = per * j->tid, hi = lo + per;
    if (hi > j->n)
        hi = j->n;
    if (lo < hi)
        j->fn(j->ctx, lo, hi);
    return NULL;
}

static void run(int64_t n, int nt, void (*fn)(void *, int64_t, int64_t), void *ctx)
{
    if (nt < 1)
        nt = 1;
    if (nt > 128)
        nt = 128;
    if (n < nt)
        nt = n > 0 ? (int)n : 1;
    pthread_t th[128];
    job jobs[128];
    for (int t = 0; t < nt; ++t) {
        jobs[t] = (job){n, t, nt, fn, ctx};
        if (t > 0)
            pthread_create(&th[t], NULL, job_main, &jobs[t]);
    }
    job_main(&jobs[0]);
    for (int t = 1; t < nt; ++t)
        pthread_join(th[t], NULL);
}

/* ------------------------------------------------------------------------ */
/* Flat uniform / normal arrays: element i uses row 0, column i.             */

typedef struct {
    uint64_t seed;
    uint32_t stream;
    void *out;
} flat_ctx;

static void uniform24_fn(void *p, int64_t lo, int64_t hi)
{
    flat_ctx *c = (flat_ctx *)p;
    for (int64_t i = lo; i < hi; ++i) {
        uint32_t w[4];
        draw4(c->seed, c->stream, (uint64_t)i >> 32, (uint32_t)i, w);
        ((float *)c->out)[i] = (float)(w[0] >> 8) * 0x1p-24f;
    }
}

static void uniform53_fn(void *p, int64_t lo, int64_t hi)
{
    flat_ctx *c = (flat_ctx *)p;
    for (int64_t i = lo; i < hi; ++i) {
        uint32_t w[4];
        draw4(c->seed, c->stream, (uint64_t)i >> 32, (uint32_t)i, w);
        ((double *)c->out)[i] = u53(w[0], w[1]);
    }
}

static void normal_fn(void *p, int64_t lo, int64_t hi)
{
    flat_ctx *c = (flat_ctx *)p;
    for (int64_t i = lo; i < hi; ++i)
        ((double *)c->out)[i] = normal_at(c->seed, c->stream, 0, (uint64_t)i);
}

static void words_fn(void *p, int64_t lo, int64_t hi)
{
    flat_ctx *c = (flat_ctx *)p;
    for (int64_t i = lo; i < hi; ++i) {
        uint32_t w[4];
        draw4(c->seed, c->stream, (uint64_t)i >> 32, (uint32_t)i, w);
        for (int k = 0; k < 4; ++k)
            ((uint32_t *)c->out)[4 * i + k] = w[k];
    }
}

/* 4*n raw 32-bit words: the four outputs of counter i land at 4i .. 4i+3 */
void ig_words(uint64_t seed, uint32_t stream, int64_t n, uint32_t *out, int nthreads)
{
    flat_ctx c = {seed, stream, out};
    run(n, nthreads, words_fn, &c);
}

/* float32 uniforms on the 2^-24 grid of [0, 1 - 2^-24] */
void ig_uniform24(uint64_t seed, uint32_t stream, int64_t n, float *out, int nthreads)
{
    flat_ctx c = {seed, stream, out};
    run(n, nthreads, uniform24_fn, &c);
}

/* double uniforms in (0, 1) with 53 random bits */
void ig_uniform53(uint64_t seed, uint32_t stream, int64_t n, double *out, int nthreads)
{
    flat_ctx c = {seed, stream, out};
    run(n, nthreads, uniform53_fn, &c);
}

void ig_normal(uint64_t seed, uint32_t stream, int64_t n, double *out, int nthreads)
{
    flat_ctx c = {seed, stream, out};
    run(n, nthreads, normal_fn, &c);
}

/* ------------------------------------------------------------------------ */
/* Logit rows.  Output row r, column j:
 *   base(r,j) = scale * D(seed, stream_base, src_row[r], j) + spike(src_row[r], j)
 *   value     = base + noise_sd[r] * N(seed, stream_noise, noise_row[r], j)
 * with D standard normal (dist 0) or Student-t(3) (dist 1); spikes add
 * spike_height on n_spikes distinct columns drawn per source row.           */

#define STREAM_BASE 1u
#define STREAM_NOISE 2u
#define STREAM_SPIKE 3u

typedef struct {
    uint64_t seed;
    int dist;
    double scale;
    int n_spikes;
    double spike_height;
    int V;
    const int64_t *src_row;
    const double *noise_sd;
    const int64_t *noise_row;
    int out_dtype;
    void *out;
} rows_ctx;

static void rows_fn(void *p, int64_t lo, int64_t hi)
{
    rows_ctx *c = (rows_ctx *)p;
    const int V = c->V;
    int spikes[64];
    for (int64_t r = lo; r < hi; ++r) {
        uint64_t src = (uint64_t)c->src_row[r];
        int ns = 0;
        for (uint32_t k = 0; ns < c->n_spikes && ns < 64; ++k) {
            uint32_t w[4];
            draw4(c->seed, STREAM_SPIKE, src, k, w);
            int id = (int)(((uint64_t)w[0] * (uint64_t)V) >> 32);
            int dup = 0;
            for (int s = 0; s < ns; ++s)
                dup |= spikes[s] == id;
            if (!dup)
                spikes[ns++] = id;
        }
        double sd = c->noise_sd ? c->noise_sd[r] : 0.0;
        uint64_t nrow = c->noise_row ? (uint64_t)c->noise_row[r] : 0;
        for (int j = 0; j < V; ++j) {
            double v = c->dist == 1 ? student_t3_at(c->seed, STREAM_BASE, src, (uint64_t)j)
                                    : normal_at(c->seed, STREAM_BASE, src, (uint64_t)j);
            v *= c->scale;
            for (int s = 0; s < ns; ++s)
                if (spikes[s] == j)
                    v += c->spike_height;
            float base = (float)v; /* the fp32 logit before any noise or rounding */
            float val = base;
            if (sd != 0.0)
                val = (float)((double)base + sd * normal_at(c->seed, STREAM_NOISE, nrow, (uint64_t)j));
            size_t o = (size_t)r * (size_t)V + (size_t)j;
            if (c->out_dtype == 0)
                ((float *)c->out)[o] = val;
            else
                ((uint16_t *)c->out)[o] = bf16_rne(val);
        }
    }
}

int ig_logit_rows(uint64_t seed, int dist, double scale, int n_spikes, double spike_height, int64_t nrows, int V,
                  const int64_t *src_row, const double *noise_sd, const int64_t *noise_row, int out_dtype,
                  void *out, int nthreads)
{
    if (V < 1 || nrows < 0 || n_spikes < 0 || n_spikes > 64 || n_spikes > V)
        return -1;
    rows_ctx c = {seed, dist, scale, n_spikes, spike_height, V, src_row, noise_sd, noise_row, out_dtype, out};
    run(nrows, nthreads, rows_fn, &c);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Draft tokens by Gumbel-max.                                               */

typedef struct {
    uint64_t seed;
    uint32_t stream;
    int V, dtype;
    const void *rows;
    const float *T;
    const int64_t *row_key;
    int32_t *out;
} tok_ctx;

static inline double stored_logit(const void *rows, int dtype, size_t i)
{
    if (dtype == 0)
        return (double)((const float *)rows)[i];
    uint32_t b = (uint32_t)((const uint16_t *)rows)[i] << 16;
    float f;
    memcpy(&f, &b, 4);
    return (double)f;
}

static void tok_fn(void *p, int64_t lo, int64_t hi)
{
    tok_ctx *c = (tok_ctx *)p;
    for (int64_t r = lo; r < hi; ++r) {
        double T = (double)c->T[r];
        double best = -INFINITY;
        int arg = 0;
        for (int j = 0; j < c->V; ++j) {
            double l = stored_logit(c->rows, c->dtype, (size_t)r * (size_t)c->V + (size_t)j);
            double s = l;
            if (T > 0.0) {
                uint32_t w[4];
                draw4(c->seed, c->stream, (uint64_t)c->row_key[r], (uint32_t)j, w);
                s = l / T - log(-log(u53(w[0], w[1])));
            }
            if (s > best) {
                best = s;
                arg = j;
            }
        }
        c->out[r] = arg;
    }
}

int ig_sample_tokens(uint64_t seed, uint32_t stream, int64_t nrows, int V, int dtype, const void *rows,
                     const float *T, const int64_t *row_key, int32_t *out, int nthreads)
{
    if (V < 1 || nrows < 0)
        return -1;
    tok_ctx c = {seed, stream, V, dtype, rows, T, row_key, out};
    run(nrows, nthreads, tok_fn, &c);
    return 0;
}
