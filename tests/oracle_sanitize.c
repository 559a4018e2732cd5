/*
 * Memory and undefined-behaviour check of the CPU oracle (test infrastructure).
 *
 * Every oracle entry point runs on small inputs held in heap buffers of exactly
 * the documented size, so AddressSanitizer reports any access past them,
 * LeakSanitizer any allocation an early return forgets, and UBSan any undefined
 * operation (shifts, overflowing conversions, misaligned or null accesses).
 * The cases cover both activation dtypes, ragged multi-group sizes, the
 * degenerate inputs of each compressor (zero residual, dead low-rank columns,
 * full rank, k = 1 and k = 128, all-equal and signed-zero residuals, index bytes
 * with the high bit set) and the argument checks.  It prints "ok" and exits 0
 * when every return code is the expected one.
 *
 * Built and run by tests/test_sanitizers.py with
 * gcc -fsanitize=address,undefined -fno-sanitize-recover=all.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int cfo_init_state(int dtype, const void* a, float* ahat, float* err, int64_t numel);
int cfo_compress(int bits, int dtype, const void* a, float* ahat, float* err, uint8_t* codes,
                 float* scales, int64_t numel);
int cfo_decompress(int bits, const uint8_t* codes, const float* scales, float* ahat, int64_t numel);
int cfo_compress_explicit_ef(int bits, int dtype, const void* a, const void* a_prev, float* ahat,
                             float* err, uint8_t* codes, float* scales, int64_t numel);
int cfo_compress_noef(int bits, int dtype, const void* a, const void* a_prev, float* ahat,
                      uint8_t* codes, float* scales, int64_t numel);
int cfo_quantize_naive(int bits, int dtype, const void* a, float* out, uint8_t* codes,
                       float* scales, int64_t numel);
int cfo_int4_quantize(const float* x, int64_t rows, int k, uint8_t* packed, float* scales);
int cfo_int4_dequantize(const uint8_t* packed, const float* scales, int64_t rows, int k, float* x);
int cfo_lowrank_compress(int dtype, const void* a, float* ahat, float* err, int64_t m, int64_t n,
                         int rank, int iters, int factor_bits, float* q_state, void* u,
                         float* u_scales, void* v, float* v_scales);
int cfo_lowrank_decompress(int factor_bits, const void* u, const float* u_scales, const void* v,
                           const float* v_scales, float* ahat, int64_t m, int64_t n, int rank);
int cfo_topk_compress(int k, int dtype, const void* a, float* ahat, float* err, uint8_t* idx,
                      uint16_t* vals, int64_t numel);
int cfo_topk_decompress(int k, const uint8_t* idx, const uint16_t* vals, float* ahat, int64_t numel);

enum { BF16 = 0, F32 = 1, OK = 0, EARG = -1 };

static int failures = 0;

static void expect(int got, int want, const char* what, int line) {
    if (got != want) {
        fprintf(stderr, "line %d: %s returned %d, expected %d\n", line, what, got, want);
        ++failures;
    }
}
#define EXPECT(call, want) expect((call), (want), #call, __LINE__)

/* splitmix64: a fixed, seedable stream of 64-bit words. */
static uint64_t mix_state = 0x9E3779B97F4A7C15ull;
static uint64_t next64(void) {
    uint64_t z = (mix_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
/* Uniform in [-1, 1) with 24 random bits. */
static float uniform(void) { return (float)((int32_t)(next64() >> 40) - (1 << 23)) / (float)(1 << 23); }

static void* xalloc(size_t bytes) {
    void* p = malloc(bytes ? bytes : 1);
    if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
    return p;
}

/* An activation of numel elements in the given dtype, exactly sized. */
static void* activation(int dtype, int64_t numel) {
    if (dtype == F32) {
        float* a = (float*)xalloc(sizeof(float) * (size_t)numel);
        for (int64_t i = 0; i < numel; ++i) a[i] = 3.0f * uniform();
        return a;
    }
    uint16_t* a = (uint16_t*)xalloc(sizeof(uint16_t) * (size_t)numel);
    for (int64_t i = 0; i < numel; ++i) {
        float f = 3.0f * uniform();
        uint32_t u;
        memcpy(&u, &f, 4);
        a[i] = (uint16_t)(u >> 16);
    }
    return a;
}

static void quantizers(int bits, int dtype, int64_t numel) {
    const int64_t ngroups = numel / 128;
    void* a0 = activation(dtype, numel);
    void* a1 = activation(dtype, numel);
    float* ahat = (float*)xalloc(sizeof(float) * (size_t)numel);
    float* rx = (float*)xalloc(sizeof(float) * (size_t)numel);
    float* err = (float*)xalloc(sizeof(float) * (size_t)numel);
    uint8_t* codes = (uint8_t*)xalloc((size_t)(numel * bits / 8));
    float* scales = (float*)xalloc(sizeof(float) * (size_t)ngroups);

    EXPECT(cfo_init_state(dtype, a0, ahat, err, numel), OK);
    EXPECT(cfo_init_state(dtype, a0, rx, NULL, numel), OK);
    /* Zero residual: the activation equals the reconstruction. */
    EXPECT(cfo_compress(bits, dtype, a0, ahat, err, codes, scales, numel), OK);
    EXPECT(cfo_decompress(bits, codes, scales, rx, numel), OK);
    for (int step = 0; step < 3; ++step) {
        EXPECT(cfo_compress(bits, dtype, step & 1 ? a0 : a1, ahat, err, codes, scales, numel), OK);
        EXPECT(cfo_decompress(bits, codes, scales, rx, numel), OK);
    }
    EXPECT(cfo_compress_explicit_ef(bits, dtype, a1, a0, ahat, err, codes, scales, numel), OK);
    EXPECT(cfo_compress_noef(bits, dtype, a1, a0, ahat, codes, scales, numel), OK);
    EXPECT(cfo_quantize_naive(bits, dtype, a1, rx, codes, scales, numel), OK);

    /* Argument checks return before touching any buffer. */
    EXPECT(cfo_compress(bits, dtype, a0, ahat, err, codes, scales, numel - 1), EARG);
    EXPECT(cfo_compress(3, dtype, a0, ahat, err, codes, scales, numel), EARG);
    EXPECT(cfo_compress(bits, 7, a0, ahat, err, codes, scales, numel), EARG);
    EXPECT(cfo_compress(bits, dtype, a0, ahat, NULL, codes, scales, numel), EARG);
    EXPECT(cfo_decompress(bits, NULL, scales, rx, numel), EARG);
    EXPECT(cfo_init_state(dtype, a0, ahat, err, -128), EARG);
    /* Empty calls do nothing and succeed. */
    EXPECT(cfo_compress(bits, dtype, a0, ahat, err, codes, scales, 0), OK);
    EXPECT(cfo_decompress(bits, codes, scales, rx, 0), OK);

    free(a0); free(a1); free(ahat); free(rx); free(err); free(codes); free(scales);
}

static void int4(int64_t rows, int k, int zero_column) {
    float* x = (float*)xalloc(sizeof(float) * (size_t)(rows * k));
    for (int64_t i = 0; i < rows * k; ++i) x[i] = (i % k == zero_column) ? 0.0f : uniform();
    uint8_t* packed = (uint8_t*)xalloc((size_t)(rows * k / 2));
    float* scales = (float*)xalloc(sizeof(float) * (size_t)k);
    float* back = (float*)xalloc(sizeof(float) * (size_t)(rows * k));
    EXPECT(cfo_int4_quantize(x, rows, k, packed, scales), OK);
    EXPECT(cfo_int4_dequantize(packed, scales, rows, k, back), OK);
    EXPECT(cfo_int4_quantize(x, rows, k + 1, packed, scales), EARG);
    free(x); free(packed); free(scales); free(back);
}

static size_t factor_bytes(int factor_bits, int64_t rows, int rank) {
    if (factor_bits == 4) return (size_t)(rows * rank / 2);
    return (size_t)(rows * rank) * (size_t)(factor_bits / 8);
}

static void lowrank(int dtype, int64_t m, int64_t n, int rank, int iters, int factor_bits,
                    int zero_residual) {
    const int64_t numel = m * n;
    void* a = activation(dtype, numel);
    float* ahat = (float*)xalloc(sizeof(float) * (size_t)numel);
    float* rx = (float*)xalloc(sizeof(float) * (size_t)numel);
    float* err = (float*)xalloc(sizeof(float) * (size_t)numel);
    float* q = (float*)xalloc(sizeof(float) * (size_t)(n * rank));
    void* u = xalloc(factor_bytes(factor_bits, m, rank));
    void* v = xalloc(factor_bytes(factor_bits, n, rank));
    float* us = factor_bits == 4 ? (float*)xalloc(sizeof(float) * (size_t)rank) : NULL;
    float* vs = factor_bits == 4 ? (float*)xalloc(sizeof(float) * (size_t)rank) : NULL;
    for (int64_t i = 0; i < n * rank; ++i) q[i] = uniform();

    if (zero_residual) {
        EXPECT(cfo_init_state(dtype, a, ahat, err, numel), OK);
        EXPECT(cfo_init_state(dtype, a, rx, NULL, numel), OK);
    } else {
        for (int64_t i = 0; i < numel; ++i) ahat[i] = rx[i] = 0.5f * uniform();
    }
    for (int step = 0; step < 2; ++step) {
        EXPECT(cfo_lowrank_compress(dtype, a, ahat, err, m, n, rank, iters, factor_bits, q, u, us, v,
                                    vs),
               OK);
        EXPECT(cfo_lowrank_decompress(factor_bits, u, us, v, vs, rx, m, n, rank), OK);
    }
    EXPECT(cfo_lowrank_compress(dtype, a, ahat, err, m, n, (int)(m < n ? m : n) + 1, iters,
                                factor_bits, q, u, us, v, vs),
           EARG);
    EXPECT(cfo_lowrank_compress(dtype, a, ahat, err, m, n, rank, 0, factor_bits, q, u, us, v, vs),
           EARG);
    EXPECT(cfo_lowrank_decompress(8, u, us, v, vs, rx, m, n, rank), EARG);
    free(a); free(ahat); free(rx); free(err); free(q); free(u); free(v); free(us); free(vs);
}

/* Residual patterns for top-k: 0 random, 1 all equal, 2 signed zeros and ties. */
static void topk(int k, int dtype, int64_t numel, int pattern) {
    const int64_t ngroups = numel / 128;
    float* a = (float*)xalloc(sizeof(float) * (size_t)numel);
    for (int64_t i = 0; i < numel; ++i) {
        if (pattern == 1) a[i] = 0.25f;
        else if (pattern == 2) a[i] = (i % 3 == 0) ? -0.0f : (i % 3 == 1 ? 0.0f : 0.5f);
        else a[i] = uniform();
    }
    void* act = a;
    uint16_t* a16 = NULL;
    if (dtype == BF16) {
        a16 = (uint16_t*)xalloc(sizeof(uint16_t) * (size_t)numel);
        for (int64_t i = 0; i < numel; ++i) {
            uint32_t w;
            memcpy(&w, &a[i], 4);
            a16[i] = (uint16_t)(w >> 16);
        }
        act = a16;
    }
    float* ahat = (float*)xalloc(sizeof(float) * (size_t)numel);
    float* rx = (float*)xalloc(sizeof(float) * (size_t)numel);
    float* err = (float*)xalloc(sizeof(float) * (size_t)numel);
    uint8_t* idx = (uint8_t*)xalloc((size_t)(ngroups * k));
    uint16_t* vals = (uint16_t*)xalloc(sizeof(uint16_t) * (size_t)(ngroups * k));
    for (int64_t i = 0; i < numel; ++i) ahat[i] = rx[i] = 0.0f;

    for (int step = 0; step < 2; ++step) {
        EXPECT(cfo_topk_compress(k, dtype, act, ahat, err, idx, vals, numel), OK);
        EXPECT(cfo_topk_decompress(k, idx, vals, rx, numel), OK);
    }
    /* A receiver masks index bytes to their group, whatever arrives. */
    memset(idx, 0xFF, (size_t)(ngroups * k));
    EXPECT(cfo_topk_decompress(k, idx, vals, rx, numel), OK);
    EXPECT(cfo_topk_compress(0, dtype, act, ahat, err, idx, vals, numel), EARG);
    EXPECT(cfo_topk_compress(129, dtype, act, ahat, err, idx, vals, numel), EARG);
    EXPECT(cfo_topk_decompress(k, idx, vals, rx, numel + 64), EARG);
    free(a); free(a16); free(ahat); free(rx); free(err); free(idx); free(vals);
}

int main(void) {
    for (int bits = 1; bits <= 2; ++bits)
        for (int dtype = 0; dtype <= 1; ++dtype) {
            quantizers(bits, dtype, 128);
            quantizers(bits, dtype, 5 * 128);
        }
    int4(1, 2, -1);
    int4(7, 4, 1);
    int4(33, 32, 31);
    /* dtype, m, n, rank, iterations, factor bits, zero residual */
    lowrank(BF16, 8, 16, 2, 2, 4, 0);
    lowrank(F32, 16, 8, 3, 1, 32, 0);
    lowrank(F32, 8, 8, 8, 2, 16, 0);   /* full rank */
    lowrank(BF16, 4, 12, 1, 3, 32, 0); /* rank 1 */
    lowrank(BF16, 12, 4, 4, 2, 4, 0);  /* rank = n */
    lowrank(F32, 8, 16, 4, 2, 4, 1);   /* zero residual: every column dead */
    lowrank(BF16, 6, 10, 3, 2, 16, 1);
    for (int dtype = 0; dtype <= 1; ++dtype) {
        const int ks[] = {1, 6, 12, 127, 128};
        for (int i = 0; i < 5; ++i)
            for (int pattern = 0; pattern < 3; ++pattern) topk(ks[i], dtype, 3 * 128, pattern);
    }
    if (failures) {
        fprintf(stderr, "%d unexpected return codes\n", failures);
        return 1;
    }
    printf("ok\n");
    return 0;
}
