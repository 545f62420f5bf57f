/*
 * Seeded synthetic input generators for causal linear attention workloads.
 *
 * This file is shared by the HIP path's tests/benchmark and by the CPU oracle's
 * tests: it only draws random inputs, it holds none of the attention arithmetic.
 *
 * Random numbers come from a counter-based SplitMix64 stream (Steele, Lea and
 * Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014): the
 * value at counter c of stream `key` is mix(key + (c + 1) * gamma), so any
 * element can be drawn independently and in parallel.  Normals use the
 * Box-Muller transform.  The decode-state sampler uses the Bartlett
 * decomposition of a Wishart matrix and the Marsaglia-Tsang (2000) gamma
 * sampler, both from their published descriptions.
 *
 * Build: gcc -O2 -fPIC -shared -pthread gen.c -o _lagen.so -lm
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define GOLDEN_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t sm64_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* Value number `c` of the SplitMix64 sequence seeded with `key`. */
static inline uint64_t sm64_at(uint64_t key, uint64_t c) {
    return sm64_mix(key + (c + 1) * GOLDEN_GAMMA);
}

/* Key of the stream for (seed, tensor id): two mixing rounds so that
 * neighbouring seeds and ids give unrelated streams. */
uint64_t lagen_stream_key(uint64_t seed, uint64_t tensor_id) {
    return sm64_mix(sm64_mix(seed + GOLDEN_GAMMA) ^ (tensor_id * 0xD1B54A32D192ED03ULL + 1));
}

/* uniform in (0, 1]: never 0, safe for log */
static inline double u01_open0(uint64_t r) { return ((double)(r >> 11) + 1.0) * 0x1.0p-53; }
/* uniform in [0, 1) */
static inline double u01_open1(uint64_t r) { return (double)(r >> 11) * 0x1.0p-53; }

static const double TWO_PI = 6.283185307179586476925286766559;

/* Element e of the standard-normal stream: pairs (2p, 2p+1) share one
 * Box-Muller draw; even elements take the cosine branch, odd the sine. */
static inline double normal_at(uint64_t key, uint64_t e) {
    uint64_t p = e >> 1;
    double u1 = u01_open0(sm64_at(key, 2 * p));
    double u2 = u01_open1(sm64_at(key, 2 * p + 1));
    double rad = sqrt(-2.0 * log(u1));
    double ang = TWO_PI * u2;
    return (e & 1) ? rad * sin(ang) : rad * cos(ang);
}

/* fp32 -> bf16 bits, round to nearest even (finite inputs). */
static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t bits;
    memcpy(&bits, &f, 4);
    uint32_t bias = 0x7FFFu + ((bits >> 16) & 1u);
    return (uint16_t)((bits + bias) >> 16);
}

uint16_t lagen_f32_to_bf16(float f) { return f32_to_bf16_rne(f); }

/* ---------------------------------------------------------------- threads */

typedef void (*range_fn)(void* ctx, int64_t lo, int64_t hi);
typedef struct { range_fn fn; void* ctx; int64_t lo, hi; } range_job;

static void* range_thread(void* a) {
    range_job* j = (range_job*)a;
    j->fn(j->ctx, j->lo, j->hi);
    return NULL;
}

static int resolve_threads(int nthreads) {
    if (nthreads > 0) return nthreads;
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    return n > 0 ? (int)n : 1;
}

/* Split [0, n) into contiguous ranges, one per thread. */
static void parallel_range(int64_t n, int nthreads, range_fn fn, void* ctx) {
    nthreads = resolve_threads(nthreads);
    if (nthreads > 256) nthreads = 256;
    if (n < 4096 || nthreads == 1) { fn(ctx, 0, n); return; }
    pthread_t tid[256];
    range_job jobs[256];
    int64_t per = (n + nthreads - 1) / nthreads;
    int used = 0;
    for (int t = 0; t < nthreads; ++t) {
        int64_t lo = (int64_t)t * per, hi = lo + per > n ? n : lo + per;
        if (lo >= hi) break;
        jobs[t] = (range_job){fn, ctx, lo, hi};
        if (pthread_create(&tid[t], NULL, range_thread, &jobs[t]) != 0) {
            fn(ctx, lo, hi);
            jobs[t].fn = NULL;
        }
        used = t + 1;
    }
    for (int t = 0; t < used; ++t)
        if (jobs[t].fn) pthread_join(tid[t], NULL);
}

/* ------------------------------------------------------- dense normals */

typedef struct { uint64_t key; double scale; uint64_t offset; void* out; int kind; } fill_ctx;

static void fill_range(void* c, int64_t lo, int64_t hi) {
    fill_ctx* f = (fill_ctx*)c;
    for (int64_t i = lo; i < hi; ++i) {
        double x = normal_at(f->key, f->offset + (uint64_t)i) * f->scale;
        float xf = (float)x; /* round to nearest fp32 */
        if (f->kind == 0)
            ((uint16_t*)f->out)[i] = f32_to_bf16_rne(xf);
        else
            ((float*)f->out)[i] = xf;
    }
}

/* out[i] = bf16_rne(fp32(N_i * scale)), N_i = element (offset + i) of stream (seed, tensor_id) */
void lagen_normal_bf16(uint64_t seed, uint64_t tensor_id, double scale, uint64_t offset,
                       int64_t n, uint16_t* out, int nthreads) {
    fill_ctx c = {lagen_stream_key(seed, tensor_id), scale, offset, out, 0};
    parallel_range(n, nthreads, fill_range, &c);
}

/* out[i] = fp32(N_i * scale) */
void lagen_normal_f32(uint64_t seed, uint64_t tensor_id, double scale, uint64_t offset,
                      int64_t n, float* out, int nthreads) {
    fill_ctx c = {lagen_stream_key(seed, tensor_id), scale, offset, out, 1};
    parallel_range(n, nthreads, fill_range, &c);
}

/* Exact-integer inputs in {-1, 0, 1} (for bit-exact blocking checks). */
typedef struct { uint64_t key; void* out; int kind; } tern_ctx;
static void tern_range(void* c, int64_t lo, int64_t hi) {
    tern_ctx* f = (tern_ctx*)c;
    for (int64_t i = lo; i < hi; ++i) {
        int v = (int)(sm64_at(f->key, (uint64_t)i) % 3) - 1;
        if (f->kind == 0)
            ((uint16_t*)f->out)[i] = f32_to_bf16_rne((float)v);
        else
            ((float*)f->out)[i] = (float)v;
    }
}
void lagen_ternary(uint64_t seed, uint64_t tensor_id, int64_t n, void* out, int as_f32, int nthreads) {
    tern_ctx c = {lagen_stream_key(seed, tensor_id), out, as_f32 ? 1 : 0};
    parallel_range(n, nthreads, tern_range, &c);
}

/* ------------------------------------------------------ document lengths */

/* Packs documents of length floor(exp(U[ln lo, ln hi))) until `total` tokens
 * are covered; the last one is cut to fit.  Writes cu_seqlens (capacity
 * max_docs + 1) and returns the number of documents, or -1 if max_docs is
 * too small. */
int32_t lagen_doc_lengths(uint64_t seed, uint64_t tensor_id, int64_t total, int64_t lo, int64_t hi,
                          int32_t* cu, int32_t max_docs) {
    uint64_t key = lagen_stream_key(seed, tensor_id);
    double a = log((double)lo), b = log((double)hi);
    int64_t pos = 0;
    int32_t nd = 0;
    cu[0] = 0;
    uint64_t c = 0;
    while (pos < total) {
        if (nd >= max_docs) return -1;
        int64_t len = (int64_t)floor(exp(a + (b - a) * u01_open1(sm64_at(key, c++))));
        if (len < 1) len = 1;
        if (pos + len > total) len = total - pos;
        pos += len;
        cu[++nd] = (int32_t)pos;
    }
    return nd;
}

/* --------------------------------------------- decode incoming states */

/* Sequential draws inside one pair's private stream. */
typedef struct { uint64_t key; uint64_t c; } stream_t;
static inline double st_u01_open0(stream_t* s) { return u01_open0(sm64_at(s->key, s->c++)); }
static inline double st_normal(stream_t* s) {
    double u1 = u01_open0(sm64_at(s->key, s->c++));
    double u2 = u01_open1(sm64_at(s->key, s->c++));
    return sqrt(-2.0 * log(u1)) * cos(TWO_PI * u2);
}

/* Gamma(alpha, 1), Marsaglia & Tsang (2000); for alpha < 1 their boost
 * Gamma(alpha) = Gamma(alpha + 1) * U^(1/alpha). */
static double st_gamma(stream_t* s, double alpha) {
    if (alpha < 1.0) {
        double g = st_gamma(s, alpha + 1.0);
        return g * pow(st_u01_open0(s), 1.0 / alpha);
    }
    double dd = alpha - 1.0 / 3.0, cc = 1.0 / sqrt(9.0 * dd);
    for (;;) {
        double x = st_normal(s), v = 1.0 + cc * x;
        if (v <= 0.0) continue;
        v = v * v * v;
        double u = st_u01_open0(s);
        if (u < 1.0 - 0.0331 * x * x * x * x) return dd * v;
        if (log(u) < 0.5 * x * x + dd * (1.0 - v + log(v))) return dd * v;
    }
}

/* Per-sequence prefix length n = floor(exp(U[ln lo, ln hi))). */
int64_t lagen_prefix_len(uint64_t seed, uint64_t tensor_id, int64_t seq, int64_t lo, int64_t hi) {
    uint64_t key = lagen_stream_key(seed, tensor_id);
    double a = log((double)lo), b = log((double)hi);
    return (int64_t)floor(exp(a + (b - a) * u01_open1(sm64_at(key, (uint64_t)seq))));
}

typedef struct {
    uint64_t seed, tid_state, tid_len;
    int64_t H, d, lo, hi;
    const int64_t* fixed_n; /* optional per-pair n */
    float* out;
} kv_ctx;

/* One (seq, head) pair: S = A G / d with A the Bartlett factor of
 * Wishart_d(n, I) (A_ii = sqrt(chi2_{n-i}), A_ij ~ N(0,1) for i > j) and G a
 * d x d standard normal matrix.  For K, V with n i.i.d. N(0, I/d) rows,
 * K^T V has exactly this distribution. */
static void kv_pair(const kv_ctx* c, int64_t p, double* A, double* G) {
    const int64_t d = c->d;
    int64_t n = c->fixed_n ? c->fixed_n[p] : lagen_prefix_len(c->seed, c->tid_len, p / c->H, c->lo, c->hi);
    stream_t s = {sm64_mix(lagen_stream_key(c->seed, c->tid_state) + (uint64_t)p * GOLDEN_GAMMA), 0};
    for (int64_t i = 0; i < d; ++i) {
        for (int64_t j = 0; j < i; ++j) A[i * d + j] = st_normal(&s);
        A[i * d + i] = sqrt(2.0 * st_gamma(&s, 0.5 * (double)(n - i)));
        for (int64_t j = i + 1; j < d; ++j) A[i * d + j] = 0.0;
    }
    for (int64_t i = 0; i < d * d; ++i) G[i] = st_normal(&s);
    float* out = c->out + p * d * d;
    for (int64_t i = 0; i < d; ++i) {
        double row[512];
        for (int64_t j = 0; j < d; ++j) row[j] = 0.0;
        for (int64_t m = 0; m <= i; ++m) {
            double a = A[i * d + m];
            const double* g = G + m * d;
            for (int64_t j = 0; j < d; ++j) row[j] += a * g[j];
        }
        for (int64_t j = 0; j < d; ++j) out[i * d + j] = (float)(row[j] / (double)d);
    }
}

static void kv_range(void* cv, int64_t lo, int64_t hi) {
    kv_ctx* c = (kv_ctx*)cv;
    double* A = (double*)malloc(sizeof(double) * c->d * c->d);
    double* G = (double*)malloc(sizeof(double) * c->d * c->d);
    for (int64_t p = lo; p < hi; ++p) kv_pair(c, p, A, G);
    free(A);
    free(G);
}

/* Incoming decode states for npairs = num_seqs * H pairs, fp32 [npairs, d, d],
 * state[i][j] indexed (key i, value j).  n per sequence is drawn from stream
 * (seed, tid_len) unless fixed_n (per pair) is given.  d <= 512; every n must
 * be >= d (the Bartlett factor needs n - i >= 1 degrees of freedom): returns
 * -2 otherwise. */
int lagen_decode_states(uint64_t seed, uint64_t tid_state, uint64_t tid_len, int64_t num_seqs, int64_t H,
                        int64_t d, int64_t lo, int64_t hi, const int64_t* fixed_n, float* out, int nthreads) {
    if (d < 1 || d > 512) return -1;
    if (fixed_n) {
        for (int64_t p = 0; p < num_seqs * H; ++p)
            if (fixed_n[p] < d) return -2;
    } else if (lo < d) {
        return -2;
    }
    kv_ctx c = {seed, tid_state, tid_len, H, d, lo, hi, fixed_n, out};
    int64_t np = num_seqs * H;
    nthreads = resolve_threads(nthreads);
    if (np < nthreads) nthreads = (int)(np > 0 ? np : 1);
    /* parallel_range only splits large ranges; pairs are heavy, so split here */
    if (nthreads == 1) { kv_range(&c, 0, np); return 0; }
    pthread_t tid[256];
    range_job jobs[256];
    if (nthreads > 256) nthreads = 256;
    int64_t per = (np + nthreads - 1) / nthreads;
    int used = 0;
    for (int t = 0; t < nthreads; ++t) {
        int64_t a = (int64_t)t * per, b = a + per > np ? np : a + per;
        if (a >= b) break;
        jobs[t] = (range_job){kv_range, &c, a, b};
        if (pthread_create(&tid[t], NULL, range_thread, &jobs[t]) != 0) {
            kv_range(&c, a, b);
            jobs[t].fn = NULL;
        }
        used = t + 1;
    }
    for (int t = 0; t < used; ++t)
        if (jobs[t].fn) pthread_join(tid[t], NULL);
    return 0;
}
