/*
 * Memory, undefined-behaviour and data-race check of the seeded input
 * generator (test infrastructure).
 *
 * Draws trajectories of ragged shapes (rows not a multiple of the generator's
 * 64-row tasks, a channel count with no power-of-two factor, several slots)
 * into buffers of exactly the documented size, once on one thread and once on
 * a pool of threads, and checks that the two are bit-identical.  Built twice by
 * tests/test_sanitizers.py: with AddressSanitizer and UBSan, and with
 * ThreadSanitizer, which reports any unsynchronised access between the pool's
 * workers.  Prints "ok" and exits 0 on success.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int cfgen_normals(uint64_t seed, int64_t kind, int64_t slot, int64_t step, int64_t count, float* out);
int cfgen_channel_scales(uint64_t seed, int64_t slot, int64_t n, double sigma, double outlier_frac,
                         double outlier_mult, float* c);
int cfgen_start(uint64_t seed, int64_t slot0, int64_t nslots, int64_t m, int64_t n, const float* c,
                float* state, uint16_t* out16, float* out32, int threads);
int cfgen_advance(uint64_t seed, int64_t slot0, int64_t nslots, int64_t step, int64_t m, int64_t n,
                  const float* c, double drift, float* state, uint16_t* out16, float* out32,
                  int threads);
int cfgen_to_bf16(const float* in, uint16_t* out, int64_t count);

static void* xalloc(size_t bytes) {
    void* p = malloc(bytes ? bytes : 1);
    if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
    return p;
}

static int failures = 0;
#define CHECK(cond)                                                        \
    do {                                                                   \
        if (!(cond)) { fprintf(stderr, "line %d: %s\n", __LINE__, #cond); ++failures; } \
    } while (0)

/* One trajectory of `steps` steps; returns the final fp32 state and bf16 copy. */
static void trajectory(int64_t nslots, int64_t m, int64_t n, int steps, int threads, float** state_out,
                       uint16_t** bf16_out) {
    const int64_t numel = nslots * m * n;
    float* c = (float*)xalloc(sizeof(float) * (size_t)(nslots * n));
    for (int64_t s = 0; s < nslots; ++s)
        CHECK(cfgen_channel_scales(7, 2 + s, n, 0.5, 0.01 * (double)(s + 1), 20.0, c + s * n) == 0);
    float* state = (float*)xalloc(sizeof(float) * (size_t)numel);
    uint16_t* out16 = (uint16_t*)xalloc(sizeof(uint16_t) * (size_t)numel);
    float* out32 = (float*)xalloc(sizeof(float) * (size_t)numel);
    CHECK(cfgen_start(7, 2, nslots, m, n, c, state, out16, out32, threads) == 0);
    for (int t = 1; t <= steps; ++t)
        CHECK(cfgen_advance(7, 2, nslots, t, m, n, c, 0.05, state, out16, out32, threads) == 0);
    CHECK(memcmp(state, out32, sizeof(float) * (size_t)numel) == 0);
    free(c);
    free(out32);
    *state_out = state;
    *bf16_out = out16;
}

int main(void) {
    const int64_t shapes[][3] = {{1, 1, 1}, {3, 130, 37}, {2, 64, 128}, {1, 200, 96}};
    for (int i = 0; i < 4; ++i) {
        const int64_t nslots = shapes[i][0], m = shapes[i][1], n = shapes[i][2];
        const int64_t numel = nslots * m * n;
        float *s1, *s4;
        uint16_t *b1, *b4;
        trajectory(nslots, m, n, 3, 1, &s1, &b1);
        trajectory(nslots, m, n, 3, 4, &s4, &b4);
        CHECK(memcmp(s1, s4, sizeof(float) * (size_t)numel) == 0);
        CHECK(memcmp(b1, b4, sizeof(uint16_t) * (size_t)numel) == 0);
        uint16_t* conv = (uint16_t*)xalloc(sizeof(uint16_t) * (size_t)numel);
        CHECK(cfgen_to_bf16(s1, conv, numel) == 0);
        CHECK(memcmp(conv, b1, sizeof(uint16_t) * (size_t)numel) == 0);
        free(s1); free(s4); free(b1); free(b4); free(conv);
    }
    /* Normal streams whose length is not a multiple of the internal batch. */
    float* z = (float*)xalloc(sizeof(float) * 1025);
    CHECK(cfgen_normals(1, 0, 0, 0, 1025, z) == 0);
    CHECK(cfgen_normals(1, 0, 0, 0, 0, z) == 0);
    free(z);
    /* Argument checks. */
    CHECK(cfgen_advance(7, 0, 1, 0, 4, 4, NULL, 0.05, NULL, NULL, NULL, 1) != 0);
    CHECK(cfgen_start(7, 0, 0, 4, 4, NULL, NULL, NULL, NULL, 1) != 0);
    CHECK(cfgen_channel_scales(7, 0, 0, 0.5, 0.01, 20.0, NULL) != 0);
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("ok\n");
    return 0;
}
