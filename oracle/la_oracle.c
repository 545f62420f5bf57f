/*
 * fp64 CPU oracle for causal linear attention.
 *
 * TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It is deliberately plain: sequential fp64 sums in
 * the order of the definition, no blocking, no fusion.  It shares no code with
 * the GPU library; inputs are widened to fp64 here, exactly.
 *
 * Sources (page titles and sections):
 *  - "MiniMax-01技术报告解读（一）模型架构" (CSDN) and "MiniMax-01技术报告解读"
 *    (qingkelab), §2.2 线性注意力: linear attention computed with the right
 *    product, through a recursively updated key-value product; no softmax.
 *  - "MiniMax-01技术报告解读", §3.2 item 1 (数据打包) and item 4 (变长特征支持):
 *    samples are packed end to end; each one is independent, so the state
 *    restarts at every document start.
 *  - "MiniMax-01技术报告解读", §3.3 item 1 (批处理内核融合) and item 2
 *    (分离预填充和解码执行): decode is a length-1 step that updates the
 *    prefix key-value cache.
 * Readings where the pages are silent (their formulas were images): no scale,
 * feature map or normaliser; the causal mask includes the current token
 * (s <= t); the state is KV = sum k^T v (key x value) and o = q . KV; a decode
 * step updates the state before reading it.
 *  - "MiniMax-01技术报告解读", §3.3 item 1 (批处理内核融合) names a decay-value
 *    computation (衰减值计算) among the fused prefill steps but never defines
 *    it.  The *_decay functions take the plainest reading that keeps the
 *    recurrence: a per-head factor lambda in [0, 1] by which the state fades
 *    before each token's update, S_t = lambda S_{t-1} + k_t^T v_t, so that
 *    o_t = sum_{s <= t} lambda^(t - s) (q_t . k_s) v_s; lambda = 1 is the
 *    undecayed operation.  The functions without _decay have no decay.
 *
 * Build: gcc -O2 -fPIC -shared -pthread la_oracle.c -o _laoracle.so
 * (no -ffast-math: the sums must stay in program order).
 */
#include "la_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdatomic.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* ------------------------------------------------------------- inputs */

static double widen(const void* p, int dtype, int64_t i) {
    if (dtype == 0) {
        uint32_t bits = (uint32_t)((const uint16_t*)p)[i] << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    if (dtype == 1) return (double)((const float*)p)[i];
    return ((const double*)p)[i];
}

/* ------------------------------------------------------------ threads */

static int g_last_threads = 1;
int ora_last_threads(void) { return g_last_threads; }

static int pick_threads(int nthreads, int64_t ntasks) {
    long n = nthreads > 0 ? nthreads : sysconf(_SC_NPROCESSORS_ONLN);
    if (n < 1) n = 1;
    if (n > 256) n = 256;
    if (n > ntasks) n = ntasks > 0 ? ntasks : 1;
    return (int)n;
}

typedef void (*task_fn)(void* ctx, int64_t task);
typedef struct {
    task_fn fn;
    void* ctx;
    int64_t ntasks;
    atomic_llong next;
} pool_t;

static void* pool_worker(void* a) {
    pool_t* p = (pool_t*)a;
    for (;;) {
        int64_t t = atomic_fetch_add(&p->next, 1);
        if (t >= p->ntasks) break;
        p->fn(p->ctx, t);
    }
    return NULL;
}

/* Runs fn(ctx, t) for t in [0, ntasks) on a pool of threads; tasks write
 * disjoint outputs, so the result does not depend on the thread count. */
static void run_tasks(int64_t ntasks, int nthreads, task_fn fn, void* ctx) {
    pool_t p;
    p.fn = fn;
    p.ctx = ctx;
    p.ntasks = ntasks;
    atomic_init(&p.next, 0);
    int n = pick_threads(nthreads, ntasks);
    g_last_threads = n;
    if (n == 1) {
        pool_worker(&p);
        return;
    }
    pthread_t tid[256];
    int started = 0;
    for (int i = 0; i < n; ++i) {
        if (pthread_create(&tid[i], NULL, pool_worker, &p) != 0) break;
        ++started;
    }
    if (started == 0) pool_worker(&p);
    for (int i = 0; i < started; ++i) pthread_join(tid[i], NULL);
}

static int check_cu(const int32_t* cu, int32_t num_seqs) {
    if (!cu || num_seqs < 1 || cu[0] != 0) return -1;
    for (int32_t s = 0; s < num_seqs; ++s)
        if (cu[s + 1] < cu[s]) return -1;
    return 0;
}

/* ----------------------------------------------------- form (b): recurrent */

/* A task is (document, head, value-column slice).  Value columns j never mix
 * in the recurrence (S[i][j] only involves v_j, o_j only column j of S), so
 * the slices are independent. */
#define ORA_COLS 16

typedef struct {
    const void *q, *k, *v;
    int dtype;
    const int32_t* cu;
    int32_t num_seqs, H, d, h0, h1, nslice;
    const double* kv_in;
    double *o, *kv_out;
    const double* decay; /* per-head factor, or NULL (no decay) */
} rec_ctx;

static void rec_task(void* cv, int64_t task) {
    const rec_ctx* c = (const rec_ctx*)cv;
    const int32_t d = c->d, H = c->H, nh = c->h1 - c->h0;
    const int32_t slice = (int32_t)(task % c->nslice);
    const int64_t dh = task / c->nslice;
    const int32_t h = c->h0 + (int32_t)(dh % nh);
    const int32_t doc = (int32_t)(dh / nh);
    const int32_t j0 = slice * ORA_COLS;
    const int32_t nj = (d - j0) < ORA_COLS ? (d - j0) : ORA_COLS;

    double* S = (double*)malloc(sizeof(double) * (size_t)d * ORA_COLS); /* S[i][jj] */
    double* kk = (double*)malloc(sizeof(double) * (size_t)d);
    double* qq = (double*)malloc(sizeof(double) * (size_t)d);
    double vv[ORA_COLS];

    const size_t sbase = ((size_t)doc * H + h) * (size_t)d * d;
    for (int32_t i = 0; i < d; ++i)
        for (int32_t jj = 0; jj < nj; ++jj) S[i * ORA_COLS + jj] = c->kv_in ? c->kv_in[sbase + (size_t)i * d + j0 + jj] : 0.0;

    for (int64_t t = c->cu[doc]; t < c->cu[doc + 1]; ++t) {
        const int64_t row = (t * H + h) * (int64_t)d;
        for (int32_t i = 0; i < d; ++i) {
            kk[i] = widen(c->k, c->dtype, row + i);
            qq[i] = widen(c->q, c->dtype, row + i);
        }
        for (int32_t jj = 0; jj < nj; ++jj) vv[jj] = widen(c->v, c->dtype, row + j0 + jj);
        /* decayed variant: S <- lambda_h S first (the state before token t fades by one step) */
        if (c->decay)
            for (int32_t i = 0; i < d; ++i)
                for (int32_t jj = 0; jj < nj; ++jj) S[i * ORA_COLS + jj] *= c->decay[h];
        /* S <- S + k_t^T v_t  (rank-1 update) */
        for (int32_t i = 0; i < d; ++i)
            for (int32_t jj = 0; jj < nj; ++jj) S[i * ORA_COLS + jj] += kk[i] * vv[jj];
        /* o_t = q_t . S  (the state already includes token t) */
        if (c->o) {
            double acc[ORA_COLS];
            for (int32_t jj = 0; jj < nj; ++jj) acc[jj] = 0.0;
            for (int32_t i = 0; i < d; ++i)
                for (int32_t jj = 0; jj < nj; ++jj) acc[jj] += qq[i] * S[i * ORA_COLS + jj];
            double* orow = c->o + (t * nh + (h - c->h0)) * (int64_t)d + j0;
            for (int32_t jj = 0; jj < nj; ++jj) orow[jj] = acc[jj];
        }
    }
    if (c->kv_out)
        for (int32_t i = 0; i < d; ++i)
            for (int32_t jj = 0; jj < nj; ++jj) c->kv_out[sbase + (size_t)i * d + j0 + jj] = S[i * ORA_COLS + jj];
    free(S);
    free(kk);
    free(qq);
}

int ora_recurrent(const void* q, const void* k, const void* v, int dtype, const int32_t* cu_seqlens,
                  int32_t num_seqs, int32_t H, int32_t d, int32_t h0, int32_t h1, const double* kv_in,
                  double* o, double* kv_out, int nthreads) {
    if (!q || !k || !v || dtype < 0 || dtype > 2 || H < 1 || d < 1 || h0 < 0 || h1 > H || h0 >= h1) return -1;
    if (check_cu(cu_seqlens, num_seqs)) return -1;
    rec_ctx c = {q, k, v, dtype, cu_seqlens, num_seqs, H, d, h0, h1, (d + ORA_COLS - 1) / ORA_COLS, kv_in, o, kv_out,
                 NULL};
    int64_t ntasks = (int64_t)num_seqs * (h1 - h0) * c.nslice;
    run_tasks(ntasks, nthreads, rec_task, &c);
    return 0;
}

static int check_decay(const double* decay, int32_t H) {
    if (!decay) return -1;
    for (int32_t h = 0; h < H; ++h)
        if (!(decay[h] >= 0.0 && decay[h] <= 1.0)) return -1;
    return 0;
}

int ora_recurrent_decay(const void* q, const void* k, const void* v, int dtype, const int32_t* cu_seqlens,
                        int32_t num_seqs, int32_t H, int32_t d, int32_t h0, int32_t h1, const double* decay,
                        const double* kv_in, double* o, double* kv_out, int nthreads) {
    if (!q || !k || !v || dtype < 0 || dtype > 2 || H < 1 || d < 1 || h0 < 0 || h1 > H || h0 >= h1) return -1;
    if (check_cu(cu_seqlens, num_seqs) || check_decay(decay, H)) return -1;
    rec_ctx c = {q, k, v, dtype, cu_seqlens, num_seqs, H, d, h0, h1, (d + ORA_COLS - 1) / ORA_COLS, kv_in, o, kv_out,
                 decay};
    int64_t ntasks = (int64_t)num_seqs * (h1 - h0) * c.nslice;
    run_tasks(ntasks, nthreads, rec_task, &c);
    return 0;
}

/* ---------------------------------------------------- form (a): quadratic */

int ora_quadratic(const void* q, const void* k, const void* v, int dtype, const int32_t* cu_seqlens,
                  int32_t num_seqs, int32_t H, int32_t d, const double* kv_in, double* o, double* kv_out) {
    if (!q || !k || !v || dtype < 0 || dtype > 2 || H < 1 || d < 1) return -1;
    if (check_cu(cu_seqlens, num_seqs)) return -1;
    g_last_threads = 1;
    for (int32_t doc = 0; doc < num_seqs; ++doc) {
        const int64_t s0 = cu_seqlens[doc], n = cu_seqlens[doc + 1] - s0;
        for (int32_t h = 0; h < H; ++h) {
            const size_t sbase = ((size_t)doc * H + h) * (size_t)d * d;
            /* A[r][c] = q_r . k_c for c <= r, 0 above the diagonal */
            double* A = (double*)calloc((size_t)(n > 0 ? n * n : 1), sizeof(double));
            for (int64_t r = 0; r < n; ++r)
                for (int64_t cc = 0; cc <= r; ++cc) {
                    double dot = 0.0;
                    for (int32_t i = 0; i < d; ++i)
                        dot += widen(q, dtype, ((s0 + r) * H + h) * d + i) * widen(k, dtype, ((s0 + cc) * H + h) * d + i);
                    A[r * n + cc] = dot;
                }
            /* o_r = sum_c A[r][c] v_c + q_r . kv_in */
            if (o)
                for (int64_t r = 0; r < n; ++r)
                    for (int32_t j = 0; j < d; ++j) {
                        double acc = 0.0;
                        for (int64_t cc = 0; cc < n; ++cc) acc += A[r * n + cc] * widen(v, dtype, ((s0 + cc) * H + h) * d + j);
                        if (kv_in)
                            for (int32_t i = 0; i < d; ++i) acc += widen(q, dtype, ((s0 + r) * H + h) * d + i) * kv_in[sbase + (size_t)i * d + j];
                        o[((s0 + r) * H + h) * d + j] = acc;
                    }
            /* kv_out = kv_in + sum_c k_c^T v_c */
            if (kv_out)
                for (int32_t i = 0; i < d; ++i)
                    for (int32_t j = 0; j < d; ++j) {
                        double acc = kv_in ? kv_in[sbase + (size_t)i * d + j] : 0.0;
                        for (int64_t cc = 0; cc < n; ++cc)
                            acc += widen(k, dtype, ((s0 + cc) * H + h) * d + i) * widen(v, dtype, ((s0 + cc) * H + h) * d + j);
                        kv_out[sbase + (size_t)i * d + j] = acc;
                    }
            free(A);
        }
    }
    return 0;
}

/* The decayed variant in form (a): the score of key c for query r carries
 * lambda^(r - c), the incoming state reaches token r faded r + 1 times, and
 * the final state holds every token faded to the document's end:
 *   A[r][c] = lambda^(r - c) q_r . k_c  (c <= r)
 *   o_r     = sum_c A[r][c] v_c + lambda^(r + 1) q_r . kv_in
 *   kv_out  = lambda^n kv_in + sum_c lambda^(n - 1 - c) k_c^T v_c
 * (pow(lambda, m) with pow(0, 0) = 1). */
int ora_quadratic_decay(const void* q, const void* k, const void* v, int dtype, const int32_t* cu_seqlens,
                        int32_t num_seqs, int32_t H, int32_t d, const double* decay, const double* kv_in, double* o,
                        double* kv_out) {
    if (!q || !k || !v || dtype < 0 || dtype > 2 || H < 1 || d < 1) return -1;
    if (check_cu(cu_seqlens, num_seqs) || check_decay(decay, H)) return -1;
    g_last_threads = 1;
    for (int32_t doc = 0; doc < num_seqs; ++doc) {
        const int64_t s0 = cu_seqlens[doc], n = cu_seqlens[doc + 1] - s0;
        for (int32_t h = 0; h < H; ++h) {
            const double lam = decay[h];
            const size_t sbase = ((size_t)doc * H + h) * (size_t)d * d;
            double* A = (double*)calloc((size_t)(n > 0 ? n * n : 1), sizeof(double));
            for (int64_t r = 0; r < n; ++r)
                for (int64_t cc = 0; cc <= r; ++cc) {
                    double dot = 0.0;
                    for (int32_t i = 0; i < d; ++i)
                        dot += widen(q, dtype, ((s0 + r) * H + h) * d + i) * widen(k, dtype, ((s0 + cc) * H + h) * d + i);
                    A[r * n + cc] = pow(lam, (double)(r - cc)) * dot;
                }
            if (o)
                for (int64_t r = 0; r < n; ++r)
                    for (int32_t j = 0; j < d; ++j) {
                        double acc = 0.0;
                        for (int64_t cc = 0; cc < n; ++cc) acc += A[r * n + cc] * widen(v, dtype, ((s0 + cc) * H + h) * d + j);
                        if (kv_in) {
                            const double f = pow(lam, (double)(r + 1));
                            for (int32_t i = 0; i < d; ++i)
                                acc += f * widen(q, dtype, ((s0 + r) * H + h) * d + i) * kv_in[sbase + (size_t)i * d + j];
                        }
                        o[((s0 + r) * H + h) * d + j] = acc;
                    }
            if (kv_out)
                for (int32_t i = 0; i < d; ++i)
                    for (int32_t j = 0; j < d; ++j) {
                        double acc = kv_in ? pow(lam, (double)n) * kv_in[sbase + (size_t)i * d + j] : 0.0;
                        for (int64_t cc = 0; cc < n; ++cc)
                            acc += pow(lam, (double)(n - 1 - cc)) * widen(k, dtype, ((s0 + cc) * H + h) * d + i) *
                                   widen(v, dtype, ((s0 + cc) * H + h) * d + j);
                        kv_out[sbase + (size_t)i * d + j] = acc;
                    }
            free(A);
        }
    }
    return 0;
}

/* ------------------------------------------------------------- backward */

/* Gradients of L = sum_t dO_t . o_t + <dKV_out, KV_out> (per document and
 * head), written from the definition o_t = q_t . S_t with
 * S_t = KV_in + sum_{s <= t} k_s^T v_s and KV_out = S_last.  The pages give no
 * backward; it follows from the forward definition by the chain rule:
 *   dq_t   = S_t dO_t                  (dq_t[i] = sum_j S_t[i][j] dO_t[j])
 *   G_s    = dKV_out + sum_{t >= s} q_t^T dO_t
 *   dk_s   = G_s v_s                   (dk_s[i] = sum_j G_s[i][j] v_s[j])
 *   dv_s   = k_s G_s                   (dv_s[j] = sum_i k_s[i] G_s[i][j])
 *   dKV_in = G_first
 * One task per (document, head): a forward sweep for dq, a backward sweep
 * for G, dk, dv. */
typedef struct {
    const void *q, *k, *v, *dout;
    int dtype;
    const int32_t* cu;
    int32_t num_seqs, H, d;
    const double *kv_in, *dkv_out;
    double *dq, *dk, *dv, *dkv_in;
} bwd_ctx;

static void bwd_task(void* cv, int64_t task) {
    const bwd_ctx* c = (const bwd_ctx*)cv;
    const int32_t d = c->d, H = c->H;
    const int32_t h = (int32_t)(task % H), doc = (int32_t)(task / H);
    const size_t sbase = ((size_t)doc * H + h) * (size_t)d * d;
    double* M = (double*)malloc(sizeof(double) * (size_t)d * d);
    double* a = (double*)malloc(sizeof(double) * (size_t)d);
    double* b = (double*)malloc(sizeof(double) * (size_t)d);

    /* forward sweep: S_t, dq_t */
    for (size_t e = 0; e < (size_t)d * d; ++e) M[e] = c->kv_in ? c->kv_in[sbase + e] : 0.0;
    for (int64_t t = c->cu[doc]; t < c->cu[doc + 1]; ++t) {
        const int64_t row = (t * H + h) * (int64_t)d;
        for (int32_t i = 0; i < d; ++i) a[i] = widen(c->k, c->dtype, row + i);
        for (int32_t j = 0; j < d; ++j) b[j] = widen(c->v, c->dtype, row + j);
        for (int32_t i = 0; i < d; ++i)
            for (int32_t j = 0; j < d; ++j) M[(size_t)i * d + j] += a[i] * b[j];
        for (int32_t j = 0; j < d; ++j) b[j] = widen(c->dout, c->dtype, row + j);
        for (int32_t i = 0; i < d; ++i) {
            double acc = 0.0;
            for (int32_t j = 0; j < d; ++j) acc += M[(size_t)i * d + j] * b[j];
            c->dq[row + i] = acc;
        }
    }
    /* backward sweep: G_s, dk_s, dv_s */
    for (size_t e = 0; e < (size_t)d * d; ++e) M[e] = c->dkv_out ? c->dkv_out[sbase + e] : 0.0;
    for (int64_t t = (int64_t)c->cu[doc + 1] - 1; t >= c->cu[doc]; --t) {
        const int64_t row = (t * H + h) * (int64_t)d;
        for (int32_t i = 0; i < d; ++i) a[i] = widen(c->q, c->dtype, row + i);
        for (int32_t j = 0; j < d; ++j) b[j] = widen(c->dout, c->dtype, row + j);
        for (int32_t i = 0; i < d; ++i)
            for (int32_t j = 0; j < d; ++j) M[(size_t)i * d + j] += a[i] * b[j];
        for (int32_t j = 0; j < d; ++j) b[j] = widen(c->v, c->dtype, row + j);
        for (int32_t i = 0; i < d; ++i) {
            double acc = 0.0;
            for (int32_t j = 0; j < d; ++j) acc += M[(size_t)i * d + j] * b[j];
            c->dk[row + i] = acc;
        }
        for (int32_t i = 0; i < d; ++i) a[i] = widen(c->k, c->dtype, row + i);
        for (int32_t j = 0; j < d; ++j) {
            double acc = 0.0;
            for (int32_t i = 0; i < d; ++i) acc += a[i] * M[(size_t)i * d + j];
            c->dv[row + j] = acc;
        }
    }
    if (c->dkv_in)
        for (size_t e = 0; e < (size_t)d * d; ++e) c->dkv_in[sbase + e] = M[e];
    free(M);
    free(a);
    free(b);
}

int ora_backward(const void* q, const void* k, const void* v, const void* dout, int dtype, const int32_t* cu_seqlens,
                 int32_t num_seqs, int32_t H, int32_t d, const double* kv_in, const double* dkv_out, double* dq,
                 double* dk, double* dv, double* dkv_in, int nthreads) {
    if (!q || !k || !v || !dout || !dq || !dk || !dv || dtype < 0 || dtype > 2 || H < 1 || d < 1) return -1;
    if (check_cu(cu_seqlens, num_seqs)) return -1;
    bwd_ctx c = {q, k, v, dout, dtype, cu_seqlens, num_seqs, H, d, kv_in, dkv_out, dq, dk, dv, dkv_in};
    run_tasks((int64_t)num_seqs * H, nthreads, bwd_task, &c);
    return 0;
}

/* ---------------------------------------------------------- decode step */

typedef struct {
    const void *q, *k, *v;
    int dtype;
    int32_t d;
    double *S, *o;
    const double* decay; /* per-pair factor, or NULL */
} dec_ctx;

static void dec_task(void* cv, int64_t p) {
    const dec_ctx* c = (const dec_ctx*)cv;
    const int32_t d = c->d;
    double* S = c->S + (size_t)p * d * d;
    const int64_t row = p * (int64_t)d;
    /* decayed variant: S <- lambda S first */
    if (c->decay)
        for (size_t e = 0; e < (size_t)d * d; ++e) S[e] *= c->decay[p];
    /* S <- S + k^T v */
    for (int32_t i = 0; i < d; ++i) {
        double ki = widen(c->k, c->dtype, row + i);
        for (int32_t j = 0; j < d; ++j) S[(size_t)i * d + j] += ki * widen(c->v, c->dtype, row + j);
    }
    /* o = q . S */
    if (c->o)
        for (int32_t j = 0; j < d; ++j) {
            double acc = 0.0;
            for (int32_t i = 0; i < d; ++i) acc += widen(c->q, c->dtype, row + i) * S[(size_t)i * d + j];
            c->o[row + j] = acc;
        }
}

int ora_decode_step(const void* q, const void* k, const void* v, int dtype, int64_t npairs, int32_t d,
                    double* S, double* o, int nthreads) {
    if (!q || !k || !v || !S || dtype < 0 || dtype > 2 || npairs < 0 || d < 1) return -1;
    dec_ctx c = {q, k, v, dtype, d, S, o, NULL};
    run_tasks(npairs, nthreads, dec_task, &c);
    return 0;
}

int ora_decode_step_decay(const void* q, const void* k, const void* v, int dtype, int64_t npairs, int32_t d,
                          const double* decay, double* S, double* o, int nthreads) {
    if (!q || !k || !v || !S || !decay || dtype < 0 || dtype > 2 || npairs < 0 || d < 1) return -1;
    for (int64_t p = 0; p < npairs; ++p)
        if (!(decay[p] >= 0.0 && decay[p] <= 1.0)) return -1;
    dec_ctx c = {q, k, v, dtype, d, S, o, decay};
    run_tasks(npairs, nthreads, dec_task, &c);
    return 0;
}
