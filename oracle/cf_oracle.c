/*
 * cf_oracle.c - CPU oracle for CompactFusion step-wise residual compression with
 * sender-side error feedback.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow reference that the GPU
 * library is checked against.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it; the product path never does.  It
 * shares no code, header or table with the GPU library.
 *
 * Source: "Accelerating Parallel Diffusion Model Serving with Residual
 * Compression" (atlas.scime.ai summary of the CompactFusion paper):
 *   - Approach: the sender transmits the compressed difference between the
 *     current activation and the previous *reconstructed* activation, keeps
 *     sender-side error feedback so quantization error does not accumulate, and
 *     offers a low-rank variant whose factors are INT4-quantized;
 *   - Measured-effects table: Compact-1bit / Compact-2bit variants, warmup
 *     steps, rank 32 with INT4 factors, 2 vs 10 subspace iterations;
 *   - Experimental setup, "Builds on": error feedback from gradient compression
 *     and PowerSGD-style subspace iteration.
 * The pages fix neither group size, scale rule, code layout nor precision; the
 * readings taken here are:
 *   - groups of 128 contiguous elements; 1-bit: code = (r < 0), scale = mean|r|
 *     taken exactly and rounded once to fp32 (to nearest, ties to even), which
 *     leaves no summation order to choose;
 *     2-bit: scale s = max|r| / 1.5, levels {-1.5, -0.5, 0.5, 1.5} * s chosen
 *     by round-to-nearest with ties to the inner level, code bit0 = sign,
 *     bit1 = magnitude; codes packed LSB-first, 8 or 4 per byte;
 *   - error feedback carried in the reconstruction: r = a - Ahat_{t-1},
 *     Ahat_t = Ahat_{t-1} + d, e_t = a - Ahat_t (equal in exact arithmetic to
 *     the explicit form r = (A_t - A_{t-1}) + e_{t-1}, e_t = r - d, which is
 *     kept below as a test-only mode);
 *   - the 1/2-bit path computes in fp32 because fp32 decides the codes; the
 *     low-rank linear algebra (projections, Householder QR, reconstruction
 *     sums) runs in fp64 and rounds to fp32 where a value is stored;
 *   - low rank: P = orth(r Q) (thin Householder QR, diag(R) >= 0, columns with
 *     |R_jj| <= 1e-5 ||Y||_F set to zero: the residual is fp32, so a column of Y
 *     that small relative to the whole sits at the level of fp32 rounding noise,
 *     and counts as rank-deficient), Q = r^T P, repeated `iters` times;
 *     INT4 factors use per-column absmax scales s = max|x| / 7 and codes
 *     rint(x / s) clamped to [-7, 7], two's-complement nibbles, low nibble
 *     first along the rank index; 16-bit factors (the table's "Pure Lowrank")
 *     are the round-to-nearest-even bf16 of each fp32 factor element;
 *   - top-k sparsity (named only as a compressor family): per group of 128 the
 *     k residuals of largest |r| (ties to the lower index), sent as index bytes
 *     and bf16 values in increasing index order, with the same error feedback.
 * Built with -O2 -ffp-contract=off and no fast-math, so every fp32 operation
 * rounds once, in the order written.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define CFO_BF16 0
#define CFO_F32 1
#define CFO_GROUP 128

#define CFO_OK 0
#define CFO_EARG (-1)
#define CFO_ENOMEM (-2)

/* Activation element i widened to fp32 (bf16 -> fp32 is exact). */
static float act(int dtype, const void* a, int64_t i) {
    if (dtype == CFO_F32) return ((const float*)a)[i];
    uint32_t bits = (uint32_t)((const uint16_t*)a)[i] << 16;
    float f;
    memcpy(&f, &bits, 4);
    return f;
}

/* Round-to-nearest-even bf16 of a finite float, and its exact widening. */
static uint16_t bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

static float bf16_widen(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static int check_common(int bits, int dtype, int64_t numel) {
    if (bits != 1 && bits != 2) return CFO_EARG;
    if (dtype != CFO_BF16 && dtype != CFO_F32) return CFO_EARG;
    if (numel < 0 || numel % CFO_GROUP != 0) return CFO_EARG;
    return CFO_OK;
}

/* ---------------------------------------------------------------------------
 * One group of 128 residuals: scale, packed codes, and the dequantized values.
 * The dequantized values are produced by decoding the codes just written, so the
 * sender and the receiver use one and the same expression.
 * ------------------------------------------------------------------------- */

/* 1-bit scale: the mean of |r| over the group, taken exactly and rounded once to
 * fp32 (to nearest, ties to even).
 * Every finite fp32 value is a whole number of units of 2^-149, so the sum of the
 * 128 magnitudes is a whole number N of those units, below 2^285.  N is held in
 * nine 32-bit words, least significant first; the mean is N * 2^-156. */
#define CFO_SUM_WORDS 9

static int sum_bit(const uint32_t* N, int b) { return (int)((N[b >> 5] >> (b & 31)) & 1u); }

static float scale_1bit(const float* r) {
    uint32_t N[CFO_SUM_WORDS] = {0};
    for (int i = 0; i < CFO_GROUP; ++i) {
        float x = fabsf(r[i]);
        uint32_t u;
        memcpy(&u, &x, 4);
        uint32_t expo = u >> 23, mant = u & 0x7FFFFFu;
        /* normal: (mant + 2^23) * 2^(expo - 150);  subnormal: mant * 2^-149 */
        uint64_t units = expo ? (uint64_t)(mant | 0x800000u) : mant;
        int shift = expo ? (int)expo - 1 : 0; /* x = units * 2^(shift - 149) */
        /* add units << shift to N, word by word, carrying upwards */
        int w = shift / 32;
        uint64_t add = units << (shift % 32); /* below 2^55: words w and w + 1 */
        uint64_t carry = 0;
        for (int j = w; j < CFO_SUM_WORDS; ++j) {
            uint64_t t = (uint64_t)N[j] + (add & 0xFFFFFFFFu) + carry;
            N[j] = (uint32_t)t;
            carry = t >> 32;
            add >>= 32;
        }
    }
    int top = -1; /* highest set bit of N */
    for (int b = 32 * CFO_SUM_WORDS - 1; b >= 0 && top < 0; --b)
        if (sum_bit(N, b)) top = b;
    if (top < 0) return 0.0f;
    /* N * 2^-156 as q * 2^(low - 156): keep 24 significant bits, or fewer when the
     * mean is subnormal (its last bit is worth 2^-149, bit 7 of N). */
    int low = top - 23 > 7 ? top - 23 : 7;
    uint32_t q = 0;
    for (int b = top; b >= low; --b) q = (q << 1) | (uint32_t)sum_bit(N, b);
    int half = sum_bit(N, low - 1), rest = 0;
    for (int b = low - 2; b >= 0; --b) rest |= sum_bit(N, b);
    if (half && (rest || (q & 1u))) q += 1; /* to nearest, ties to even */
    return ldexpf((float)q, low - 156);
}

/* 2-bit scale: largest |r| mapped onto the outer level 1.5 s. */
static float scale_2bit(const float* r) {
    float M = 0.0f;
    for (int i = 0; i < CFO_GROUP; ++i) {
        float x = fabsf(r[i]);
        if (x > M) M = x;
    }
    return M / 1.5f;
}

/* Decoded value of code c (bits wide) for a group scale s. */
static float dequant(int bits, unsigned c, float s) {
    if (bits == 1) return (c & 1u) ? -s : s;
    float lvl = (c & 2u) ? 1.5f * s : 0.5f * s;
    return (c & 1u) ? -lvl : lvl;
}

static unsigned code_at(int bits, const uint8_t* gcodes, int i) {
    if (bits == 1) return (gcodes[i >> 3] >> (i & 7)) & 1u;
    return (gcodes[i >> 2] >> (2 * (i & 3))) & 3u;
}

/* Quantize one group: writes bits*16 bytes of codes, the scale, and d[128]. */
static void quantize_group(int bits, const float* r, uint8_t* gcodes, float* scale, float* d) {
    float s = bits == 1 ? scale_1bit(r) : scale_2bit(r);
    memset(gcodes, 0, (size_t)bits * 16);
    for (int i = 0; i < CFO_GROUP; ++i) {
        unsigned c;
        if (bits == 1) {
            c = r[i] < 0.0f ? 1u : 0u;
            gcodes[i >> 3] |= (uint8_t)(c << (i & 7));
        } else {
            unsigned sign = r[i] < 0.0f ? 1u : 0u;
            unsigned mag = fabsf(r[i]) > s ? 1u : 0u;
            c = sign | (mag << 1);
            gcodes[i >> 2] |= (uint8_t)(c << (2 * (i & 3)));
        }
    }
    for (int i = 0; i < CFO_GROUP; ++i) d[i] = dequant(bits, code_at(bits, gcodes, i), s);
    *scale = s;
}

/* ---------------------------------------------------------------------------
 * Warmup / initialisation: the first W steps send the activation itself, and
 * both sides take it as their reconstruction (measured-effects table: the rows
 * with one and with two warmup steps).
 * ------------------------------------------------------------------------- */
int cfo_init_state(int dtype, const void* a, float* ahat, float* err, int64_t numel) {
    if (!a || !ahat || numel < 0 || (dtype != CFO_BF16 && dtype != CFO_F32)) return CFO_EARG;
    for (int64_t i = 0; i < numel; ++i) {
        ahat[i] = act(dtype, a, i);
        if (err) err[i] = 0.0f;
    }
    return CFO_OK;
}

/* ---------------------------------------------------------------------------
 * Sender, 1/2-bit (Approach: residual against the previous reconstruction,
 * with error feedback).  Per group: r = a - Ahat, quantize, Ahat += d,
 * e = a - Ahat.  Codes: numel*bits/8 bytes; scales: numel/128 floats.
 * ------------------------------------------------------------------------- */
int cfo_compress(int bits, int dtype, const void* a, float* ahat, float* err, uint8_t* codes,
                 float* scales, int64_t numel) {
    if (check_common(bits, dtype, numel) || !a || !ahat || !err || !codes || !scales) return CFO_EARG;
    float r[CFO_GROUP], d[CFO_GROUP];
    for (int64_t g = 0; g < numel / CFO_GROUP; ++g) {
        int64_t base = g * CFO_GROUP;
        for (int i = 0; i < CFO_GROUP; ++i) r[i] = act(dtype, a, base + i) - ahat[base + i];
        quantize_group(bits, r, codes + g * 16 * bits, &scales[g], d);
        for (int i = 0; i < CFO_GROUP; ++i) {
            ahat[base + i] = ahat[base + i] + d[i];
            err[base + i] = act(dtype, a, base + i) - ahat[base + i];
        }
    }
    return CFO_OK;
}

/* Receiver: the same decoded values added to its mirror of the reconstruction. */
int cfo_decompress(int bits, const uint8_t* codes, const float* scales, float* ahat, int64_t numel) {
    if (check_common(bits, CFO_F32, numel) || !codes || !scales || !ahat) return CFO_EARG;
    for (int64_t g = 0; g < numel / CFO_GROUP; ++g) {
        const uint8_t* gc = codes + g * 16 * bits;
        for (int i = 0; i < CFO_GROUP; ++i) {
            int64_t k = g * CFO_GROUP + i;
            ahat[k] = ahat[k] + dequant(bits, code_at(bits, gc, i), scales[g]);
        }
    }
    return CFO_OK;
}

/* ---------------------------------------------------------------------------
 * Test-only modes (ablations on the pages: without error feedback; naive
 * quantization of the full activation).
 * ------------------------------------------------------------------------- */

/* Explicit error-feedback form: r = (a - a_prev) + e_prev; Ahat += d; e = r - d. */
int cfo_compress_explicit_ef(int bits, int dtype, const void* a, const void* a_prev, float* ahat,
                             float* err, uint8_t* codes, float* scales, int64_t numel) {
    if (check_common(bits, dtype, numel) || !a || !a_prev || !ahat || !err || !codes || !scales)
        return CFO_EARG;
    float r[CFO_GROUP], d[CFO_GROUP];
    for (int64_t g = 0; g < numel / CFO_GROUP; ++g) {
        int64_t base = g * CFO_GROUP;
        for (int i = 0; i < CFO_GROUP; ++i)
            r[i] = (act(dtype, a, base + i) - act(dtype, a_prev, base + i)) + err[base + i];
        quantize_group(bits, r, codes + g * 16 * bits, &scales[g], d);
        for (int i = 0; i < CFO_GROUP; ++i) {
            ahat[base + i] = ahat[base + i] + d[i];
            err[base + i] = r[i] - d[i];
        }
    }
    return CFO_OK;
}

/* No error feedback: r = a - a_prev (the raw step delta); the receiver adds d. */
int cfo_compress_noef(int bits, int dtype, const void* a, const void* a_prev, float* ahat,
                      uint8_t* codes, float* scales, int64_t numel) {
    if (check_common(bits, dtype, numel) || !a || !a_prev || !ahat || !codes || !scales)
        return CFO_EARG;
    float r[CFO_GROUP], d[CFO_GROUP];
    for (int64_t g = 0; g < numel / CFO_GROUP; ++g) {
        int64_t base = g * CFO_GROUP;
        for (int i = 0; i < CFO_GROUP; ++i)
            r[i] = act(dtype, a, base + i) - act(dtype, a_prev, base + i);
        quantize_group(bits, r, codes + g * 16 * bits, &scales[g], d);
        for (int i = 0; i < CFO_GROUP; ++i) ahat[base + i] = ahat[base + i] + d[i];
    }
    return CFO_OK;
}

/* Naive: quantize the activation itself; out = decoded activation. */
int cfo_quantize_naive(int bits, int dtype, const void* a, float* out, uint8_t* codes, float* scales,
                       int64_t numel) {
    if (check_common(bits, dtype, numel) || !a || !out || !codes || !scales) return CFO_EARG;
    float r[CFO_GROUP];
    for (int64_t g = 0; g < numel / CFO_GROUP; ++g) {
        int64_t base = g * CFO_GROUP;
        for (int i = 0; i < CFO_GROUP; ++i) r[i] = act(dtype, a, base + i);
        quantize_group(bits, r, codes + g * 16 * bits, &scales[g], out + base);
    }
    return CFO_OK;
}

/* ---------------------------------------------------------------------------
 * INT4 factor quantization (Approach: low-rank compression with INT4
 * quantization).  x is rows x k row-major fp32; per column j:
 * s_j = max_i |x_ij| / 7, c = rint(x / s_j) clamped to [-7, 7] (0 if s_j = 0);
 * packed two's-complement nibbles, element (i, j) at byte (i*k + j) / 2, low
 * nibble for even j.
 * ------------------------------------------------------------------------- */
int cfo_int4_quantize(const float* x, int64_t rows, int k, uint8_t* packed, float* scales) {
    if (!x || !packed || !scales || rows <= 0 || k <= 0 || (k & 1)) return CFO_EARG;
    for (int j = 0; j < k; ++j) {
        float M = 0.0f;
        for (int64_t i = 0; i < rows; ++i) {
            float v = fabsf(x[i * k + j]);
            if (v > M) M = v;
        }
        scales[j] = M / 7.0f;
    }
    memset(packed, 0, (size_t)(rows * k / 2));
    for (int64_t i = 0; i < rows; ++i)
        for (int j = 0; j < k; ++j) {
            float s = scales[j];
            int c = 0;
            if (s > 0.0f) {
                float q = rintf(x[i * k + j] / s);
                if (q > 7.0f) q = 7.0f;
                if (q < -7.0f) q = -7.0f;
                c = (int)q;
            }
            uint8_t nib = (uint8_t)(c & 0xF);
            packed[(i * k + j) / 2] |= (uint8_t)((j & 1) ? nib << 4 : nib);
        }
    return CFO_OK;
}

int cfo_int4_dequantize(const uint8_t* packed, const float* scales, int64_t rows, int k, float* x) {
    if (!x || !packed || !scales || rows <= 0 || k <= 0 || (k & 1)) return CFO_EARG;
    for (int64_t i = 0; i < rows; ++i)
        for (int j = 0; j < k; ++j) {
            uint8_t byte = packed[(i * k + j) / 2];
            int nib = (j & 1) ? (byte >> 4) : (byte & 0xF);
            int c = nib >= 8 ? nib - 16 : nib;
            x[i * k + j] = (float)c * scales[j];
        }
    return CFO_OK;
}

/* ---------------------------------------------------------------------------
 * Low-rank variant (Approach; "Builds on": PowerSGD-style subspace iteration).
 * ------------------------------------------------------------------------- */

/* Thin Householder QR of Y (m x k, row-major, fp64): P (m x k) with
 * orthonormal columns spanning Y's, signs chosen so diag(R) >= 0, and columns
 * whose |R_jj| <= 1e-5 ||Y||_F set to zero.  alive[j] reports which survive. */
static int householder_orth(const double* Y, int64_t m, int k, double* P, int* alive) {
    double* A = (double*)malloc(sizeof(double) * (size_t)(m * k));
    double* V = (double*)calloc((size_t)(m * k), sizeof(double)); /* reflector j in column j */
    double* beta = (double*)calloc((size_t)k, sizeof(double));
    double* rdiag = (double*)calloc((size_t)k, sizeof(double));
    if (!A || !V || !beta || !rdiag) { free(A); free(V); free(beta); free(rdiag); return CFO_ENOMEM; }
    memcpy(A, Y, sizeof(double) * (size_t)(m * k));
    double fro = 0.0;
    for (int64_t i = 0; i < m * k; ++i) fro += Y[i] * Y[i];
    fro = sqrt(fro);
    int steps = (int)(k < m ? k : m);
    for (int j = 0; j < steps; ++j) {
        double nx = 0.0;
        for (int64_t i = j; i < m; ++i) nx += A[i * k + j] * A[i * k + j];
        nx = sqrt(nx);
        if (nx == 0.0) { rdiag[j] = 0.0; beta[j] = 0.0; continue; }
        double x0 = A[(int64_t)j * k + j];
        double alpha = x0 >= 0.0 ? -nx : nx; /* reflect onto -sign(x0) e1: no cancellation */
        for (int64_t i = j; i < m; ++i) V[i * k + j] = A[i * k + j];
        V[(int64_t)j * k + j] = x0 - alpha;
        double vv = 0.0;
        for (int64_t i = j; i < m; ++i) vv += V[i * k + j] * V[i * k + j];
        beta[j] = 2.0 / vv;
        for (int c = j; c < k; ++c) {
            double dot = 0.0;
            for (int64_t i = j; i < m; ++i) dot += V[i * k + j] * A[i * k + c];
            double f = beta[j] * dot;
            for (int64_t i = j; i < m; ++i) A[i * k + c] -= f * V[i * k + j];
        }
        rdiag[j] = alpha;
    }
    /* Form the thin factor: P = H_0 H_1 ... H_{k-1} [I_k; 0]. */
    memset(P, 0, sizeof(double) * (size_t)(m * k));
    for (int j = 0; j < steps; ++j) P[(int64_t)j * k + j] = 1.0;
    for (int j = steps - 1; j >= 0; --j) {
        if (beta[j] == 0.0) continue;
        for (int c = 0; c < k; ++c) {
            double dot = 0.0;
            for (int64_t i = j; i < m; ++i) dot += V[i * k + j] * P[i * k + c];
            double f = beta[j] * dot;
            for (int64_t i = j; i < m; ++i) P[i * k + c] -= f * V[i * k + j];
        }
    }
    for (int j = 0; j < k; ++j) {
        double rj = j < steps ? rdiag[j] : 0.0;
        alive[j] = fabs(rj) > 1e-5 * fro;
        double sgn = rj < 0.0 ? -1.0 : 1.0;
        for (int64_t i = 0; i < m; ++i) P[i * k + j] = alive[j] ? sgn * P[i * k + j] : 0.0;
    }
    free(A); free(V); free(beta); free(rdiag);
    return CFO_OK;
}

/*
 * Sender, low rank.  a: m x n activation; ahat, err: m x n fp32;
 * q_state: n x rank fp32 (in: start basis, out: last unquantized Q);
 * factor_bits 4: u = m*rank/2 bytes, v = n*rank/2 bytes of nibbles, scales
 * rank floats each; factor_bits 16: u, v bf16 bits (m x rank, n x rank);
 * factor_bits 32: u, v fp32 (m x rank, n x rank); scales unused unless 4.
 * Steps: r = a - Ahat; repeat iters times { Y = r Q; P = orth(Y); Q = r^T P;
 * round P, Q to fp32 }; quantize factors; R = P^ Q^^T; Ahat += R; e = a - Ahat.
 * A column that the QR guard zeroes keeps its previous start vector in q_state.
 */
int cfo_lowrank_compress(int dtype, const void* a, float* ahat, float* err, int64_t m, int64_t n,
                         int rank, int iters, int factor_bits, float* q_state, void* u,
                         float* u_scales, void* v, float* v_scales) {
    if (!a || !ahat || !err || !q_state || !u || !v) return CFO_EARG;
    if (dtype != CFO_BF16 && dtype != CFO_F32) return CFO_EARG;
    if (m <= 0 || n <= 0 || rank < 1 || rank > (m < n ? m : n) || iters < 1) return CFO_EARG;
    if (factor_bits != 4 && factor_bits != 16 && factor_bits != 32) return CFO_EARG;
    if (factor_bits == 4 && ((rank & 1) || !u_scales || !v_scales)) return CFO_EARG;
    const int k = rank;
    int rc = CFO_ENOMEM;
    float* r = (float*)malloc(sizeof(float) * (size_t)(m * n));
    double* Q = (double*)malloc(sizeof(double) * (size_t)(n * k));
    double* Y = (double*)malloc(sizeof(double) * (size_t)(m * k));
    double* P = (double*)malloc(sizeof(double) * (size_t)(m * k));
    float* Pf = (float*)malloc(sizeof(float) * (size_t)(m * k));
    float* Qf = (float*)malloc(sizeof(float) * (size_t)(n * k));
    float* Uh = (float*)malloc(sizeof(float) * (size_t)(m * k));
    float* Vh = (float*)malloc(sizeof(float) * (size_t)(n * k));
    int* alive = (int*)malloc(sizeof(int) * (size_t)k);
    if (!r || !Q || !Y || !P || !Pf || !Qf || !Uh || !Vh || !alive) goto done;

    for (int64_t i = 0; i < m * n; ++i) r[i] = act(dtype, a, i) - ahat[i];
    for (int64_t i = 0; i < n * k; ++i) Q[i] = (double)q_state[i];

    for (int it = 0; it < iters; ++it) {
        for (int64_t i = 0; i < m; ++i)
            for (int j = 0; j < k; ++j) {
                double s = 0.0;
                for (int64_t l = 0; l < n; ++l) s += (double)r[i * n + l] * Q[l * k + j];
                Y[i * k + j] = s;
            }
        if (householder_orth(Y, m, k, P, alive)) goto done;
        /* Q[l][j] = sum_i r[i][l] P[i][j], each sum taken in increasing i. */
        for (int64_t i = 0; i < n * k; ++i) Q[i] = 0.0;
        for (int64_t i = 0; i < m; ++i)
            for (int64_t l = 0; l < n; ++l) {
                double ril = (double)r[i * n + l];
                for (int j = 0; j < k; ++j) Q[l * k + j] += ril * P[i * k + j];
            }
        for (int64_t i = 0; i < m * k; ++i) { Pf[i] = (float)P[i]; P[i] = (double)Pf[i]; }
        for (int64_t i = 0; i < n * k; ++i) { Qf[i] = (float)Q[i]; Q[i] = (double)Qf[i]; }
    }

    if (factor_bits == 4) {
        if (cfo_int4_quantize(Pf, m, k, (uint8_t*)u, u_scales)) goto done;
        if (cfo_int4_quantize(Qf, n, k, (uint8_t*)v, v_scales)) goto done;
        cfo_int4_dequantize((const uint8_t*)u, u_scales, m, k, Uh);
        cfo_int4_dequantize((const uint8_t*)v, v_scales, n, k, Vh);
    } else if (factor_bits == 16) {
        for (int64_t i = 0; i < m * k; ++i) {
            ((uint16_t*)u)[i] = bf16_rne(Pf[i]);
            Uh[i] = bf16_widen(((uint16_t*)u)[i]);
        }
        for (int64_t i = 0; i < n * k; ++i) {
            ((uint16_t*)v)[i] = bf16_rne(Qf[i]);
            Vh[i] = bf16_widen(((uint16_t*)v)[i]);
        }
    } else {
        memcpy(u, Pf, sizeof(float) * (size_t)(m * k));
        memcpy(v, Qf, sizeof(float) * (size_t)(n * k));
        memcpy(Uh, Pf, sizeof(float) * (size_t)(m * k));
        memcpy(Vh, Qf, sizeof(float) * (size_t)(n * k));
    }
    for (int64_t i = 0; i < m; ++i)
        for (int64_t l = 0; l < n; ++l) {
            double s = 0.0;
            for (int j = 0; j < k; ++j) s += (double)Uh[i * k + j] * (double)Vh[l * k + j];
            ahat[i * n + l] = ahat[i * n + l] + (float)s;
            err[i * n + l] = act(dtype, a, i * n + l) - ahat[i * n + l];
        }
    for (int64_t l = 0; l < n; ++l)
        for (int j = 0; j < k; ++j)
            if (alive[j]) q_state[l * k + j] = Qf[l * k + j];
    rc = CFO_OK;
done:
    free(r); free(Q); free(Y); free(P); free(Pf); free(Qf); free(Uh); free(Vh); free(alive);
    return rc;
}

/* Receiver, low rank: Ahat += U^ V^^T with the same dequantization and sums. */
int cfo_lowrank_decompress(int factor_bits, const void* u, const float* u_scales, const void* v,
                           const float* v_scales, float* ahat, int64_t m, int64_t n, int rank) {
    if (!u || !v || !ahat || m <= 0 || n <= 0 || rank < 1) return CFO_EARG;
    if (factor_bits != 4 && factor_bits != 16 && factor_bits != 32) return CFO_EARG;
    if (factor_bits == 4 && ((rank & 1) || !u_scales || !v_scales)) return CFO_EARG;
    const int k = rank;
    float* Uh = (float*)malloc(sizeof(float) * (size_t)(m * k));
    float* Vh = (float*)malloc(sizeof(float) * (size_t)(n * k));
    if (!Uh || !Vh) { free(Uh); free(Vh); return CFO_ENOMEM; }
    if (factor_bits == 4) {
        cfo_int4_dequantize((const uint8_t*)u, u_scales, m, k, Uh);
        cfo_int4_dequantize((const uint8_t*)v, v_scales, n, k, Vh);
    } else if (factor_bits == 16) {
        for (int64_t i = 0; i < m * k; ++i) Uh[i] = bf16_widen(((const uint16_t*)u)[i]);
        for (int64_t i = 0; i < n * k; ++i) Vh[i] = bf16_widen(((const uint16_t*)v)[i]);
    } else {
        memcpy(Uh, u, sizeof(float) * (size_t)(m * k));
        memcpy(Vh, v, sizeof(float) * (size_t)(n * k));
    }
    for (int64_t i = 0; i < m; ++i)
        for (int64_t l = 0; l < n; ++l) {
            double s = 0.0;
            for (int j = 0; j < k; ++j) s += (double)Uh[i * k + j] * (double)Vh[l * k + j];
            ahat[i * n + l] = ahat[i * n + l] + (float)s;
        }
    free(Uh); free(Vh);
    return CFO_OK;
}

/* ---------------------------------------------------------------------------
 * Top-k sparsification of the residual (Limitations: quantization and
 * sparsity are the fast compressor families the low-rank variant is compared
 * with; the pages define no sparsity rule, so this reading is taken).  Per
 * group of 128: keep the k residuals of largest |r|, ordered by the bit pattern
 * of |r| (the magnitude order for non-NaN values), equal magnitudes going to
 * the lower index; the kept entries are written in increasing index order as
 * one index byte (0..127) and the round-to-nearest-even bf16 of r.  Error
 * feedback as for the quantizers: Ahat += widened value at the kept indices,
 * e = a - Ahat everywhere (so the dropped residuals stay in e).
 * Payload per group: k index bytes at idx[g*k ..], k bf16 values at vals[g*k ..].
 * ------------------------------------------------------------------------- */
static uint32_t mag_key(float r) {
    float m = fabsf(r);
    uint32_t u;
    memcpy(&u, &m, 4);
    return u;
}

static const float* g_sort_r; /* the group being sorted (comparators take no context) */

static int by_magnitude(const void* x, const void* y) {
    int i = *(const int*)x, j = *(const int*)y;
    uint32_t ki = mag_key(g_sort_r[i]), kj = mag_key(g_sort_r[j]);
    if (ki != kj) return ki > kj ? -1 : 1;
    return i < j ? -1 : (i > j);
}

static int by_index(const void* x, const void* y) {
    int i = *(const int*)x, j = *(const int*)y;
    return i < j ? -1 : (i > j);
}

int cfo_topk_compress(int k, int dtype, const void* a, float* ahat, float* err, uint8_t* idx,
                      uint16_t* vals, int64_t numel) {
    if (k < 1 || k > CFO_GROUP || check_common(1, dtype, numel) || !a || !ahat || !err || !idx ||
        !vals)
        return CFO_EARG;
    float r[CFO_GROUP];
    int order[CFO_GROUP];
    for (int64_t g = 0; g < numel / CFO_GROUP; ++g) {
        int64_t base = g * CFO_GROUP;
        for (int i = 0; i < CFO_GROUP; ++i) {
            r[i] = act(dtype, a, base + i) - ahat[base + i];
            order[i] = i;
        }
        g_sort_r = r;
        qsort(order, CFO_GROUP, sizeof(int), by_magnitude);
        qsort(order, (size_t)k, sizeof(int), by_index);
        for (int j = 0; j < k; ++j) {
            int i = order[j];
            uint16_t h = bf16_rne(r[i]);
            idx[g * k + j] = (uint8_t)i;
            vals[g * k + j] = h;
            ahat[base + i] = ahat[base + i] + bf16_widen(h);
        }
        for (int i = 0; i < CFO_GROUP; ++i) err[base + i] = act(dtype, a, base + i) - ahat[base + i];
    }
    return CFO_OK;
}

/* Receiver: the same widened values added at the sent indices (low 7 bits of
 * each index byte, so any payload stays inside its group). */
int cfo_topk_decompress(int k, const uint8_t* idx, const uint16_t* vals, float* ahat, int64_t numel) {
    if (k < 1 || k > CFO_GROUP || check_common(1, CFO_F32, numel) || !idx || !vals || !ahat)
        return CFO_EARG;
    for (int64_t g = 0; g < numel / CFO_GROUP; ++g)
        for (int j = 0; j < k; ++j) {
            int64_t e = g * CFO_GROUP + (idx[g * k + j] & 127);
            ahat[e] = ahat[e] + bf16_widen(vals[g * k + j]);
        }
    return CFO_OK;
}
