/*
 * cfgen.c - seeded synthetic activation trajectories.
 *
 * This module is shared by the HIP path's tests/bench and by the CPU oracle's
 * tests.  It holds none of the compression method's arithmetic: it only draws
 * the inputs (activation trajectories and the random start basis of the
 * low-rank variant), so both sides see bit-identical inputs.
 *
 * Random numbers come from one counter-based generator:
 *   mix64(z): the SplitMix64 output function (Steele, Lea & Flood, "Fast
 *             splittable pseudorandom number generators", OOPSLA 2014; the
 *             constants are those of Vigna's public-domain splitmix64.c).
 *   value(key, i) = mix64(key + (i + 1) * GAMMA), GAMMA = 0x9e3779b97f4a7c15.
 *   key(seed, kind, slot, step) =
 *       mix64(mix64(mix64(seed + GAMMA*(kind+1)) + GAMMA*(slot+1)) + GAMMA*(step+1)).
 * Uniforms use the top 53 bits: u = ((x >> 11) + 0.5) * 2^-53, in (0, 1).
 * Normals use the Box-Muller transform in double precision: element 2p and
 * 2p+1 of a stream are sqrt(-2 ln u1) * {cos, sin}(2 pi u2) with
 * u1 = U(value(key, 2p)), u2 = U(value(key, 2p+1)).
 *
 * Workload recipe (the pages' FLUX.1-dev / CogVideoX-2b activations are not
 * available; these stand in for them):
 *   channel scale c_j = exp(sigma * z_j) (lognormal), then round(frac * n)
 *   channels picked by a seeded partial Fisher-Yates shuffle are multiplied
 *   by `mult` (outlier channels);
 *   A_0[i, j]  = fp32(c_j * z)                         (kind KIND_START)
 *   A_t[i, j]  = fp32(A_{t-1}[i, j] + drift * c_j * z)  (kind KIND_DRIFT, step t)
 * with all products formed in double and rounded once to fp32.  A bf16
 * activation is the round-to-nearest-even bf16 of the fp32 state.
 * An unscaled trajectory uses c_j = 1.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GAMMA 0x9e3779b97f4a7c15ULL

enum { KIND_SCALE = 0, KIND_OUTLIER = 1, KIND_START = 2, KIND_DRIFT = 3, KIND_BASIS = 4 };

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
    return z ^ (z >> 31);
}

uint64_t cfgen_key(uint64_t seed, int64_t kind, int64_t slot, int64_t step) {
    uint64_t k = mix64(seed + GAMMA * (uint64_t)(kind + 1));
    k = mix64(k + GAMMA * (uint64_t)(slot + 1));
    return mix64(k + GAMMA * (uint64_t)(step + 1));
}

uint64_t cfgen_value(uint64_t key, int64_t i) { return mix64(key + GAMMA * (uint64_t)(i + 1)); }

static inline double unif(uint64_t x) { return ((double)(x >> 11) + 0.5) * (1.0 / 9007199254740992.0); }

/* Standard normal number `i` of the stream `key`. */
static inline double normal_at(uint64_t key, int64_t i) {
    int64_t p = i >> 1;
    double u1 = unif(cfgen_value(key, 2 * p));
    double u2 = unif(cfgen_value(key, 2 * p + 1));
    double rad = sqrt(-2.0 * log(u1));
    double th = 6.283185307179586476925286766559 * u2;
    return (i & 1) ? rad * sin(th) : rad * cos(th);
}

/* Fill out[0..count) with normals i0 .. i0+count-1 of a stream (pairs share
 * one log/sqrt evaluation when both halves are wanted). */
static void normals_range(uint64_t key, int64_t i0, int64_t count, double* out) {
    int64_t i = i0, end = i0 + count, o = 0;
    if (i < end && (i & 1)) { out[o++] = normal_at(key, i); i++; }
    for (; i + 1 < end; i += 2) {
        int64_t p = i >> 1;
        double u1 = unif(cfgen_value(key, 2 * p));
        double u2 = unif(cfgen_value(key, 2 * p + 1));
        double rad = sqrt(-2.0 * log(u1));
        double th = 6.283185307179586476925286766559 * u2;
        out[o++] = rad * cos(th);
        out[o++] = rad * sin(th);
    }
    if (i < end) out[o++] = normal_at(key, i);
}

static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t bias = 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)((u + bias) >> 16);
}

/* ---- simple static thread pool over [0, total) in chunks ---------------- */
typedef void (*range_fn)(void* ctx, int64_t begin, int64_t end);
typedef struct { range_fn fn; void* ctx; int64_t total, chunk; int64_t next; pthread_mutex_t mu; } pool_t;

static void* pool_worker(void* arg) {
    pool_t* p = (pool_t*)arg;
    for (;;) {
        pthread_mutex_lock(&p->mu);
        int64_t b = p->next;
        p->next += p->chunk;
        pthread_mutex_unlock(&p->mu);
        if (b >= p->total) break;
        int64_t e = b + p->chunk < p->total ? b + p->chunk : p->total;
        p->fn(p->ctx, b, e);
    }
    return NULL;
}

static void parallel_for(int threads, int64_t total, int64_t chunk, range_fn fn, void* ctx) {
    if (threads < 1) threads = 1;
    if (threads > 256) threads = 256;
    pool_t p = {fn, ctx, total, chunk > 0 ? chunk : 1, 0, PTHREAD_MUTEX_INITIALIZER};
    if (threads == 1 || total <= p.chunk) { fn(ctx, 0, total); return; }
    pthread_t tid[256];
    int started = 0;
    for (int t = 0; t < threads; ++t)
        if (pthread_create(&tid[t], NULL, pool_worker, &p) == 0) started++;
        else break;
    if (started == 0) { fn(ctx, 0, total); return; }
    for (int t = 0; t < started; ++t) pthread_join(tid[t], NULL);
}

/* ---- public API ----------------------------------------------------------- */

/* Standard normals of stream (seed, kind, slot, step), elements [0, count). */
int cfgen_normals(uint64_t seed, int64_t kind, int64_t slot, int64_t step, int64_t count, float* out) {
    if (!out || count < 0) return -1;
    uint64_t key = cfgen_key(seed, kind, slot, step);
    double buf[512];
    for (int64_t i = 0; i < count; i += 512) {
        int64_t c = count - i < 512 ? count - i : 512;
        normals_range(key, i, c, buf);
        for (int64_t j = 0; j < c; ++j) out[i + j] = (float)buf[j];
    }
    return 0;
}

/* Per-channel scales of one slot (n floats). */
int cfgen_channel_scales(uint64_t seed, int64_t slot, int64_t n, double sigma, double outlier_frac,
                         double outlier_mult, float* c) {
    if (!c || n <= 0) return -1;
    uint64_t key = cfgen_key(seed, KIND_SCALE, slot, 0);
    double* z = (double*)malloc(sizeof(double) * (size_t)n);
    int64_t* perm = (int64_t*)malloc(sizeof(int64_t) * (size_t)n);
    if (!z || !perm) { free(z); free(perm); return -2; }
    normals_range(key, 0, n, z);
    double* cs = z; /* reused in place: cs[j] = exp(sigma z_j) */
    for (int64_t j = 0; j < n; ++j) cs[j] = exp(sigma * z[j]);
    int64_t n_out = (int64_t)llround(outlier_frac * (double)n);
    if (n_out > n) n_out = n;
    for (int64_t j = 0; j < n; ++j) perm[j] = j;
    uint64_t okey = cfgen_key(seed, KIND_OUTLIER, slot, 0);
    for (int64_t i = 0; i < n_out; ++i) {
        int64_t j = i + (int64_t)(cfgen_value(okey, i) % (uint64_t)(n - i));
        int64_t t = perm[i]; perm[i] = perm[j]; perm[j] = t;
    }
    for (int64_t i = 0; i < n_out; ++i) cs[perm[i]] *= outlier_mult;
    for (int64_t j = 0; j < n; ++j) c[j] = (float)cs[j];
    free(z);
    free(perm);
    return 0;
}

typedef struct {
    uint64_t seed;
    int64_t slot0, step, m, n, rows_per_task, tasks_per_slot;
    const float* c;  /* nslots * n, or NULL */
    double drift;    /* 0 => start (A_0) */
    float* state;    /* nslots * m * n */
    uint16_t* out16; /* optional bf16 copy */
    float* out32;    /* optional fp32 copy */
} traj_ctx;

static void traj_range(void* vctx, int64_t b, int64_t e) {
    traj_ctx* x = (traj_ctx*)vctx;
    double buf[4096];
    for (int64_t task = b; task < e; ++task) {
        int64_t s = task / x->tasks_per_slot;
        int64_t r0 = (task % x->tasks_per_slot) * x->rows_per_task;
        int64_t r1 = r0 + x->rows_per_task < x->m ? r0 + x->rows_per_task : x->m;
        int64_t slot = x->slot0 + s;
        int start = x->drift == 0.0;
        uint64_t key = cfgen_key(x->seed, start ? KIND_START : KIND_DRIFT, slot, start ? 0 : x->step);
        const float* c = x->c ? x->c + s * x->n : NULL;
        int64_t base = s * x->m * x->n;
        for (int64_t i0 = r0 * x->n; i0 < r1 * x->n; i0 += 4096) {
            int64_t cnt = r1 * x->n - i0 < 4096 ? r1 * x->n - i0 : 4096;
            normals_range(key, i0, cnt, buf);
            for (int64_t k = 0; k < cnt; ++k) {
                int64_t idx = i0 + k;
                double cj = c ? (double)c[idx % x->n] : 1.0;
                float v;
                if (start) v = (float)(cj * buf[k]);
                else v = (float)((double)x->state[base + idx] + x->drift * cj * buf[k]);
                x->state[base + idx] = v;
                if (x->out16) x->out16[base + idx] = f32_to_bf16_rne(v);
                if (x->out32) x->out32[base + idx] = v;
            }
        }
    }
}

static int traj_run(uint64_t seed, int64_t slot0, int64_t nslots, int64_t step, int64_t m, int64_t n,
                    const float* c, double drift, float* state, uint16_t* out16, float* out32, int threads) {
    if (!state || m <= 0 || n <= 0 || nslots <= 0) return -1;
    int64_t rows = 64;
    traj_ctx x = {seed, slot0, step, m, n, rows, (m + rows - 1) / rows, c, drift, state, out16, out32};
    parallel_for(threads, nslots * x.tasks_per_slot, 1, traj_range, &x);
    return 0;
}

/* A_0 for slots slot0 .. slot0+nslots-1 (state: nslots*m*n fp32). */
int cfgen_start(uint64_t seed, int64_t slot0, int64_t nslots, int64_t m, int64_t n, const float* c,
                float* state, uint16_t* out16, float* out32, int threads) {
    return traj_run(seed, slot0, nslots, 0, m, n, c, 0.0, state, out16, out32, threads);
}

/* Advance the states in place from step-1 to step (step >= 1, drift > 0). */
int cfgen_advance(uint64_t seed, int64_t slot0, int64_t nslots, int64_t step, int64_t m, int64_t n,
                  const float* c, double drift, float* state, uint16_t* out16, float* out32, int threads) {
    if (step < 1 || !(drift > 0.0)) return -1;
    return traj_run(seed, slot0, nslots, step, m, n, c, drift, state, out16, out32, threads);
}

int cfgen_to_bf16(const float* in, uint16_t* out, int64_t count) {
    if (!in || !out || count < 0) return -1;
    for (int64_t i = 0; i < count; ++i) out[i] = f32_to_bf16_rne(in[i]);
    return 0;
}
