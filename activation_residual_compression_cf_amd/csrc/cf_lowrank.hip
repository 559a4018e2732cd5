// cf_lowrank.hip - Compact-Lowrank: rank-k subspace iteration on the residual with
// INT4 factors, error feedback, and the receiver-side reconstruction, for gfx950.
//
// Method: "Accelerating Parallel Diffusion Model Serving with Residual
// Compression" (CompactFusion summary): section Approach (low-rank compression of
// the step-wise residual with INT4 quantization for extreme ratios, sender-side
// error feedback), Key results (rank 32 with INT4 factors, about 100x), the
// measured-effects table (2 vs 10 subspace iterations) and Experimental setup,
// "Builds on" (PowerSGD-style subspace iteration).
//
// Per tensor (m x n, row-major), with Q the n x k start basis:
//   r = a - Ahat                                   (fp32, kept in the workspace)
//   repeat iters times:  Y = r Q;  P = orth(Y);  Q = r^T P
//   U^ = int4(P), V^ = int4(Q)  (per-column absmax / 7, round half even, [-7, 7])
//   Ahat = Ahat + U^ V^^T;   e = a - Ahat;   q_state = Q (warm start)
// orth(Y) is the thin Q factor with diag(R) >= 0, computed as Cholesky QR with the
// Gram matrix, the factorisation and the triangular solve in fp64 (fp32 Cholesky QR
// loses the factor when kappa(Y)^2 approaches 1/eps_fp32, which warm-started
// iterates on outlier-channel residuals reach).  A column whose Cholesky pivot falls
// to <= 1e-10 trace(Y^T Y) (|R_jj| <= 1e-5 ||Y||_F) is rank deficient: its P column
// is zero and its start vector is kept in q_state.
//
// Kernels (each launch covers every tensor of the batch):
//   k_lr_prep       q_state -> Q^T (rank padded to a multiple of 16 with zeros)
//   k_lr_project    Y partials = r Q over column segments; the first pass also forms
//                   and stores r.  fp32 MFMA 16x16x4: a lane's float4 of r supplies
//                   4 k-slices, Q^T float4s the matching B operands.
//   k_lr_orth       one workgroup per tensor: Y = sum of partials (fixed order), fp64
//                   Gram, Cholesky with the rank guard, P = Y R^-1.
//   k_lr_backproject Q^T = P^T r, MFMA; the four waves of a workgroup split the rows
//                   and their partials are summed in LDS in a fixed order.
//   k_lr_quantize   INT4 (or fp32) factors, scales, and the q_state update.
//   k_lr_reconstruct Ahat += U^ V^^T (MFMA, factors dequantized on the fly from the
//                   payload) and e = a - Ahat; the receiver runs the same kernel
//                   without e, so both sides produce identical bits.
// Every reduction has a fixed order; there are no atomics.

#include "cf_internal.h"

namespace cf {
namespace {

typedef float vf4 __attribute__((ext_vector_type(4)));
typedef unsigned vu2 __attribute__((ext_vector_type(2)));

constexpr int kSegCols = 768;   // columns per projection segment
constexpr int kProjRows = 256;  // rows per projection workgroup (4 waves x 64)
constexpr int kBackCols = 128;  // columns per back-projection workgroup
constexpr int kRecRows = 64;    // reconstruction workgroup: 64 rows x 256 columns
constexpr int kRecCols = 256;

__device__ __forceinline__ vf4 mfma4(float a, float b, vf4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ vf4 ld4(const float* p) { return *reinterpret_cast<const vf4*>(p); }
__device__ __forceinline__ vf4 ld4_nt(const float* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const vf4*>(p));
}
__device__ __forceinline__ void st4_nt(float* p, vf4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<vf4*>(p));
}
__device__ __forceinline__ vf4 act4(const uint16_t* a, int64_t off) {
    const vu2 w = __builtin_nontemporal_load(reinterpret_cast<const vu2*>(a + off));
    return vf4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
               __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u)};
}
__device__ __forceinline__ vf4 act4(const float* a, int64_t off) { return ld4_nt(a + off); }

// The hardware hands workgroup w to XCD w % 8.  Renumber so that each XCD walks a
// contiguous range of logical workgroups (consecutive tiles of the same tensors),
// keeping each tensor's small operands (Q^T, P) in one XCD's L2.  `total` is a
// multiple of 8.
__device__ __forceinline__ int64_t xcd_remap(int64_t w, int64_t total) {
    return (w & 7) * (total >> 3) + (w >> 3);
}

// ---------------------------------------------------------------- prep ----
__global__ __launch_bounds__(256) void k_lr_prep(const float* __restrict__ q_state, float* __restrict__ qt,
                                                  int64_t n, int k, int kp, int64_t batch) {
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;  // over batch*kp*n
    if (idx >= batch * kp * n) return;
    const int64_t c = idx % n;
    const int kk = static_cast<int>((idx / n) % kp);
    const int64_t b = idx / (n * kp);
    qt[idx] = kk < k ? q_state[(b * n + c) * k + kk] : 0.0f;
}

// ------------------------------------------------------------- project ----
// Workgroup: 4 waves, 64 rows each (4 M-tiles of 16), one column segment.
// Ypart[b][s][row][kp] = sum over the segment's columns of r[row][c] Q[c][kk].
template <bool FIRST, typename ActT, int KT>
__global__ __launch_bounds__(256) void k_lr_project(const ActT* __restrict__ a, const float* __restrict__ ahat,
                                                     float* __restrict__ r, const float* __restrict__ qt,
                                                     float* __restrict__ ypart, int64_t m, int64_t n,
                                                     int64_t batch, int64_t nseg, int64_t total) {
    constexpr int kp = 16 * KT;
    const int64_t lw = xcd_remap(blockIdx.x, total);
    const int64_t rblocks = (m + kProjRows - 1) / kProjRows;
    if (lw >= batch * rblocks * nseg) return;  // padding workgroups of the remap
    const int64_t b = lw / (rblocks * nseg);
    const int64_t rb = (lw / nseg) % rblocks;
    const int64_t s = lw % nseg;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int64_t row0 = rb * kProjRows + wave * 64;
    const int64_t c_begin = s * kSegCols;
    const int64_t c_end = c_begin + kSegCols < n ? c_begin + kSegCols : n;
    const int64_t mn = m * n;

    bool mt_ok[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) mt_ok[mt] = row0 + 16 * mt < m;

    vf4 acc[4][KT];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int t = 0; t < KT; ++t) acc[mt][t] = vf4{0.f, 0.f, 0.f, 0.f};

    const float* qtb = qt + b * kp * n;
    for (int64_t c = c_begin; c < c_end; c += 16) {
        const int64_t col = c + 4 * lg;
        vf4 rv[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const int64_t off = b * mn + (row0 + 16 * mt + li) * n + col;
            if (mt_ok[mt]) {
                if constexpr (FIRST) {
                    rv[mt] = act4(a, off) - ld4_nt(ahat + off);
                    st4_nt(r + off, rv[mt]);
                } else {
                    rv[mt] = ld4(r + off);
                }
            } else {
                rv[mt] = vf4{0.f, 0.f, 0.f, 0.f};
            }
        }
        vf4 qv[KT];
#pragma unroll
        for (int t = 0; t < KT; ++t) qv[t] = ld4(qtb + (16 * t + li) * n + col);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int t = 0; t < KT; ++t) acc[mt][t] = mfma4(rv[mt][i], qv[t][i], acc[mt][t]);
    }
    // acc[mt][t] lane: rows row0 + 16 mt + 4 lg + v, column 16 t + li
    float* yp = ypart + ((b * nseg + s) * m) * kp;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        if (!mt_ok[mt]) continue;
#pragma unroll
        for (int t = 0; t < KT; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) yp[(row0 + 16 * mt + 4 * lg + v) * kp + 16 * t + li] = acc[mt][t][v];
    }
}

// ---------------------------------------------------------------- orth ----
// One workgroup (256 threads) per tensor.  Y rows are staged through LDS as fp64
// in chunks of 16 rows; thread (ti, tj) of a 16 x 16 grid owns the KT x KT block of
// the Gram matrix G = Y^T Y at rows ti*KT.., columns tj*KT.. .  The Cholesky factor
// L overwrites G's lower triangle; Li = L^-1; P = Y (L^T)^-1 = Y Li^T.
template <int KT>
__global__ __launch_bounds__(256) void k_lr_orth(const float* __restrict__ ypart, float* __restrict__ p,
                                                  int* __restrict__ alive, int64_t m, int64_t nseg, int k) {
    constexpr int kp = 16 * KT;
    constexpr int CH = 16;
    __shared__ double ys[CH][kp + 1];
    __shared__ double G[kp][kp + 1];
    __shared__ double Li[kp][kp + 1];
    __shared__ int dead[kp];
    const int tid = threadIdx.x;
    const int64_t b = blockIdx.x;
    const float* yb = ypart + b * nseg * m * kp;
    const int ti = tid >> 4, tj = tid & 15;

    // Y[row][kk]: the segment partials summed in segment order (fp32), widened.
    auto yval = [&](int64_t row, int kk) -> double {
        float s = yb[row * kp + kk];
        for (int64_t q = 1; q < nseg; ++q) s = s + yb[(q * m + row) * kp + kk];
        return static_cast<double>(s);
    };

    double g[KT][KT];
#pragma unroll
    for (int i = 0; i < KT; ++i)
#pragma unroll
        for (int j = 0; j < KT; ++j) g[i][j] = 0.0;
    for (int64_t r0 = 0; r0 < m; r0 += CH) {
        for (int e = tid; e < CH * kp; e += 256) {
            const int rr = e / kp, kk = e % kp;
            ys[rr][kk] = (r0 + rr < m) ? yval(r0 + rr, kk) : 0.0;
        }
        __syncthreads();
        for (int rr = 0; rr < CH; ++rr) {
            double yi[KT], yj[KT];
#pragma unroll
            for (int i = 0; i < KT; ++i) yi[i] = ys[rr][ti * KT + i];
#pragma unroll
            for (int j = 0; j < KT; ++j) yj[j] = ys[rr][tj * KT + j];
#pragma unroll
            for (int i = 0; i < KT; ++i)
#pragma unroll
                for (int j = 0; j < KT; ++j) g[i][j] = fma(yi[i], yj[j], g[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < KT; ++i)
#pragma unroll
        for (int j = 0; j < KT; ++j) G[ti * KT + i][tj * KT + j] = g[i][j];
    __syncthreads();

    double tr = 0.0;
    for (int j = 0; j < kp; ++j) tr += G[j][j];
    const double thresh = 1e-10 * tr;
    __syncthreads();  // every trace read precedes the in-place factorisation
    // Cholesky, column by column, in place in the lower triangle of G.
    for (int j = 0; j < kp; ++j) {
        if (tid == 0) {
            double d = G[j][j];
            for (int q = 0; q < j; ++q) d -= G[j][q] * G[j][q];
            const bool ok = j < k && d > thresh;
            G[j][j] = ok ? sqrt(d) : 0.0;
            dead[j] = ok ? 0 : 1;
        }
        __syncthreads();
        const bool ok = dead[j] == 0;
        for (int i = j + 1 + tid; i < kp; i += 256) {
            double v = G[i][j];
            for (int q = 0; q < j; ++q) v -= G[i][q] * G[j][q];
            G[i][j] = ok ? v / G[j][j] : 0.0;
        }
        __syncthreads();
    }
    // Li = L^-1, column c by thread c (forward substitution; dead rows give 0).
    if (tid < kp) {
        const int c = tid;
        for (int i = 0; i < kp; ++i) {
            double x = 0.0;
            if (i >= c && dead[i] == 0) {
                double v = (i == c) ? 1.0 : 0.0;
                for (int q = c; q < i; ++q) v -= G[i][q] * Li[q][c];
                x = v / G[i][i];
            }
            Li[i][c] = x;
        }
    }
    __syncthreads();
    if (tid < kp) alive[b * kp + tid] = dead[tid] ? 0 : 1;

    // P[row][j] = sum_{i <= j} Y[row][i] Li[j][i], with Y rows staged in LDS again.
    float* pb = p + b * m * kp;
    for (int64_t r0 = 0; r0 < m; r0 += CH) {
        for (int e = tid; e < CH * kp; e += 256) {
            const int rr = e / kp, kk = e % kp;
            ys[rr][kk] = (r0 + rr < m) ? yval(r0 + rr, kk) : 0.0;
        }
        __syncthreads();
        for (int e = tid; e < CH * kp; e += 256) {
            const int rr = e / kp, j = e % kp;
            double acc = 0.0;
            for (int i = 0; i <= j; ++i) acc = fma(ys[rr][i], Li[j][i], acc);
            if (r0 + rr < m) pb[(r0 + rr) * kp + j] = static_cast<float>(acc);
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------- backproject ----
// Workgroup: 4 waves over the same 128 columns; wave w takes the 4-row steps
// w, w + 4, w + 8, ...  Lane: rows row + lg, columns c0 + 64 h + 4 li .. + 3.
template <int KT>
__global__ __launch_bounds__(256) void k_lr_backproject(const float* __restrict__ r, const float* __restrict__ p,
                                                         float* __restrict__ qt, int64_t m, int64_t n,
                                                         int64_t batch, int64_t total) {
    constexpr int kp = 16 * KT;
    __shared__ float red[kp][kBackCols + 4];
    const int64_t cblocks = (n + kBackCols - 1) / kBackCols;
    const int64_t lw = xcd_remap(blockIdx.x, total);
    if (lw >= batch * cblocks) return;
    const int64_t b = lw / cblocks;
    const int64_t c0 = (lw % cblocks) * kBackCols;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int64_t mn = m * n;
    const float* rb = r + b * mn;
    const float* pb = p + b * m * kp;

    bool h_ok[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) h_ok[h] = c0 + 64 * h + 4 * li < n;

    vf4 acc[2][4][KT];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int t = 0; t < KT; ++t) acc[h][i][t] = vf4{0.f, 0.f, 0.f, 0.f};

    for (int64_t row = 4 * wave; row < m; row += 16) {
        const int64_t rr = row + lg;
        vf4 rv[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
            rv[h] = h_ok[h] ? ld4(rb + rr * n + c0 + 64 * h + 4 * li) : vf4{0.f, 0.f, 0.f, 0.f};
        float pv[KT];
#pragma unroll
        for (int t = 0; t < KT; ++t) pv[t] = pb[rr * kp + 16 * t + li];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int t = 0; t < KT; ++t) acc[h][i][t] = mfma4(pv[t], rv[h][i], acc[h][i][t]);
    }
    // acc[h][i][t] lane: Q^T row 16 t + 4 lg + v, column c0 + 64 h + 4 li + i.
    // Sum the four waves' partials in LDS, in wave order.
    for (int w = 0; w < 4; ++w) {
        if (wave == w) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int t = 0; t < KT; ++t)
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            float& dst = red[16 * t + 4 * lg + v][64 * h + 4 * li + i];
                            dst = (w == 0) ? acc[h][i][t][v] : dst + acc[h][i][t][v];
                        }
        }
        __syncthreads();
    }
    float* qtb = qt + b * kp * n;
    for (int e = threadIdx.x; e < kp * kBackCols; e += 256) {
        const int kk = e / kBackCols, cc = e % kBackCols;
        if (c0 + cc < n) qtb[kk * n + c0 + cc] = red[kk][cc];
    }
}

// ------------------------------------------------------------ quantize ----
// blockIdx.x = 2 b + f: f = 0 quantizes U = P (m rows, row-major m x kp),
// f = 1 quantizes V = Q (n rows, stored transposed as Q^T kp x n) and updates
// q_state.  Per column: s = max|x| / 7, c = rint(x / s) in [-7, 7] (0 if s = 0).
template <int KT>
__global__ __launch_bounds__(256) void k_lr_quantize(const float* __restrict__ p, const float* __restrict__ qt,
                                                      const int* __restrict__ alive, int64_t m, int64_t n, int k,
                                                      int factor_bits, float* __restrict__ q_state,
                                                      void* __restrict__ u, float* __restrict__ u_scales,
                                                      void* __restrict__ v, float* __restrict__ v_scales) {
    constexpr int kp = 16 * KT;
    constexpr int RPT = 256 / kp;  // threads per column in the max reduction
    __shared__ float part[256];
    __shared__ float sc[kp];
    const int64_t b = blockIdx.x >> 1;
    const int f = blockIdx.x & 1;
    const int64_t rows = f ? n : m;
    const float* x = f ? qt + b * kp * n : p + b * m * kp;
    // element (row, kk) of the factor
    auto at = [&](int64_t row, int kk) -> float { return f ? x[kk * n + row] : x[row * kp + kk]; };
    const int tid = threadIdx.x;

    if (factor_bits == 4) {
        const int kk = tid % kp;
        float mx = 0.0f;
        for (int64_t row = tid / kp; row < rows; row += RPT) mx = fmaxf(mx, fabsf(at(row, kk)));
        part[tid] = mx;
        __syncthreads();
        if (tid < kp) {
            float mm = part[tid];
            for (int q = 1; q < RPT; ++q) mm = fmaxf(mm, part[q * kp + tid]);
            const float s = mm / 7.0f;
            sc[tid] = s;
            if (tid < k) (f ? v_scales : u_scales)[b * k + tid] = s;
        }
        __syncthreads();
        uint8_t* out = static_cast<uint8_t*>(f ? v : u) + b * rows * k / 2;
        const int64_t nbytes = rows * k / 2;
        for (int64_t e = tid; e < nbytes; e += 256) {
            const int64_t row = (2 * e) / k;
            const int kk0 = static_cast<int>((2 * e) % k);
            uint32_t byte = 0;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const float s = sc[kk0 + h];
                int c = 0;
                if (s > 0.0f) {
                    float q = rintf(at(row, kk0 + h) / s);
                    q = fminf(fmaxf(q, -7.0f), 7.0f);
                    c = static_cast<int>(q);
                }
                byte |= (static_cast<uint32_t>(c) & 0xFu) << (4 * h);
            }
            out[e] = static_cast<uint8_t>(byte);
        }
    } else {
        float* out = static_cast<float*>(f ? v : u) + b * rows * k;
        for (int64_t e = tid; e < rows * k; e += 256) out[e] = at(e / k, static_cast<int>(e % k));
    }
    if (f) {
        float* qs = q_state + b * n * k;
        const int* al = alive + b * kp;
        for (int64_t e = tid; e < n * k; e += 256) {
            const int kk = static_cast<int>(e % k);
            if (al[kk]) qs[e] = at(e / k, kk);
        }
    }
}

// --------------------------------------------------------- reconstruct ----
// Workgroup: 4 waves side by side, each a 64 x 64 tile (4 x 4 MFMA tiles).
// C'[i][j] = sum_kk V^[col i][kk] U^[row j][kk] = R^[row j][col i], so lane l holds
// R^[row0 + 16 jt + li][col0 + 16 it + 4 lg .. + 3] after the k loop.
template <int FB>
__device__ __forceinline__ float factor_at(const void* f, const float* scales, int64_t row, int k, int kk) {
    if (kk >= k) return 0.0f;
    if constexpr (FB == 4) {
        const uint8_t byte = static_cast<const uint8_t*>(f)[(row * k + kk) >> 1];
        const int nib = (kk & 1) ? (byte >> 4) : (byte & 0xF);
        const int c = nib >= 8 ? nib - 16 : nib;
        return static_cast<float>(c) * scales[kk];
    } else {
        return static_cast<const float*>(f)[row * k + kk];
    }
}

template <bool HAS_E, typename ActT, int FB>
__global__ __launch_bounds__(256) void k_lr_reconstruct(const ActT* __restrict__ a, float* __restrict__ ahat,
                                                         float* __restrict__ err, const void* __restrict__ u,
                                                         const float* __restrict__ u_scales,
                                                         const void* __restrict__ v,
                                                         const float* __restrict__ v_scales, int64_t m,
                                                         int64_t n, int k, int64_t batch, int64_t total) {
    const int64_t rblocks = (m + kRecRows - 1) / kRecRows;
    const int64_t cblocks = (n + kRecCols - 1) / kRecCols;
    const int64_t lw = xcd_remap(blockIdx.x, total);
    if (lw >= batch * rblocks * cblocks) return;
    const int64_t b = lw / (rblocks * cblocks);
    const int64_t row0 = ((lw / cblocks) % rblocks) * kRecRows;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int64_t col0 = (lw % cblocks) * kRecCols + 64 * wave;
    if (col0 >= n) return;  // uniform per wave

    const int64_t usz = FB == 4 ? m * k / 2 : m * k * 4;  // bytes per tensor
    const int64_t vsz = FB == 4 ? n * k / 2 : n * k * 4;
    const void* ub = static_cast<const uint8_t*>(u) + b * usz;
    const void* vb = static_cast<const uint8_t*>(v) + b * vsz;
    const float* usb = FB == 4 ? u_scales + b * k : nullptr;
    const float* vsb = FB == 4 ? v_scales + b * k : nullptr;

    bool jt_ok[4], it_ok[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        jt_ok[q] = row0 + 16 * q < m;
        it_ok[q] = col0 + 16 * q < n;
    }
    vf4 acc[4][4];
#pragma unroll
    for (int it = 0; it < 4; ++it)
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) acc[it][jt] = vf4{0.f, 0.f, 0.f, 0.f};

    for (int s = 0; 4 * s < k; ++s) {
        const int kk = 4 * s + lg;
        float bu[4], av[4];
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) bu[jt] = jt_ok[jt] ? factor_at<FB>(ub, usb, row0 + 16 * jt + li, k, kk) : 0.0f;
#pragma unroll
        for (int it = 0; it < 4; ++it) av[it] = it_ok[it] ? factor_at<FB>(vb, vsb, col0 + 16 * it + li, k, kk) : 0.0f;
#pragma unroll
        for (int it = 0; it < 4; ++it)
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) acc[it][jt] = mfma4(av[it], bu[jt], acc[it][jt]);
    }

    const int64_t mn = m * n;
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
        if (!jt_ok[jt]) continue;
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            if (!it_ok[it]) continue;
            const int64_t off = b * mn + (row0 + 16 * jt + li) * n + col0 + 16 * it + 4 * lg;
            const vf4 hn = ld4_nt(ahat + off) + acc[it][jt];
            st4_nt(ahat + off, hn);
            if constexpr (HAS_E) st4_nt(err + off, act4(a, off) - hn);
        }
    }
}

// ------------------------------------------------------------- launchers --
int64_t round8(int64_t x) { return (x + 7) & ~int64_t(7); }

template <typename K>
hipError_t go(K kernel, int64_t blocks, void** args, hipStream_t stream) {
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(static_cast<unsigned>(blocks)), dim3(256),
                           args, 0, stream);
}

template <typename ActT, int KT>
hipError_t run_lowrank(const ActT* a, float* ahat, float* err, int64_t m, int64_t n, int k, int iters,
                       int factor_bits, int64_t batch, float* q_state, void* u, float* u_scales, void* v,
                       float* v_scales, const LowrankWorkspace& ws, hipStream_t stream) {
    int kp = 16 * KT;
    int64_t nseg = (n + kSegCols - 1) / kSegCols;
    hipError_t e;
    {
        int64_t cnt = batch * kp * n;
        void* args[] = {&q_state, (void*)&ws.qt, &n, &k, &kp, &batch};
        if ((e = go(&k_lr_prep, (cnt + 255) / 256, args, stream)) != hipSuccess) return e;
    }
    const int64_t rblocks = (m + kProjRows - 1) / kProjRows;
    int64_t ptotal = round8(batch * rblocks * nseg);
    int64_t btotal = round8(batch * ((n + kBackCols - 1) / kBackCols));
    for (int it = 0; it < iters; ++it) {
        void* pargs[] = {&a, &ahat, (void*)&ws.r, (void*)&ws.qt, (void*)&ws.ypart, &m, &n, &batch, &nseg, &ptotal};
        e = it == 0 ? go(&k_lr_project<true, ActT, KT>, ptotal, pargs, stream)
                    : go(&k_lr_project<false, ActT, KT>, ptotal, pargs, stream);
        if (e != hipSuccess) return e;
        void* oargs[] = {(void*)&ws.ypart, (void*)&ws.p, (void*)&ws.alive, &m, &nseg, &k};
        if ((e = go(&k_lr_orth<KT>, batch, oargs, stream)) != hipSuccess) return e;
        void* bargs[] = {(void*)&ws.r, (void*)&ws.p, (void*)&ws.qt, &m, &n, &batch, &btotal};
        if ((e = go(&k_lr_backproject<KT>, btotal, bargs, stream)) != hipSuccess) return e;
    }
    {
        void* qargs[] = {(void*)&ws.p, (void*)&ws.qt, (void*)&ws.alive, &m, &n, &k, &factor_bits,
                         &q_state, &u, &u_scales, &v, &v_scales};
        if ((e = go(&k_lr_quantize<KT>, 2 * batch, qargs, stream)) != hipSuccess) return e;
    }
    int64_t rtotal = round8(batch * ((m + kRecRows - 1) / kRecRows) * ((n + kRecCols - 1) / kRecCols));
    const void* uc = u;
    const void* vc = v;
    const float* usc = u_scales;
    const float* vsc = v_scales;
    void* rargs[] = {&a, &ahat, &err, &uc, &usc, &vc, &vsc, &m, &n, &k, &batch, &rtotal};
    return factor_bits == 4 ? go(&k_lr_reconstruct<true, ActT, 4>, rtotal, rargs, stream)
                            : go(&k_lr_reconstruct<true, ActT, 32>, rtotal, rargs, stream);
}

template <typename ActT>
hipError_t dispatch_rank(const ActT* a, float* ahat, float* err, int64_t m, int64_t n, int k, int iters,
                         int factor_bits, int64_t batch, float* q_state, void* u, float* u_scales, void* v,
                         float* v_scales, const LowrankWorkspace& ws, hipStream_t stream) {
    switch ((k + 15) / 16) {
        case 1: return run_lowrank<ActT, 1>(a, ahat, err, m, n, k, iters, factor_bits, batch, q_state, u, u_scales, v, v_scales, ws, stream);
        case 2: return run_lowrank<ActT, 2>(a, ahat, err, m, n, k, iters, factor_bits, batch, q_state, u, u_scales, v, v_scales, ws, stream);
        case 3: return run_lowrank<ActT, 3>(a, ahat, err, m, n, k, iters, factor_bits, batch, q_state, u, u_scales, v, v_scales, ws, stream);
        default: return run_lowrank<ActT, 4>(a, ahat, err, m, n, k, iters, factor_bits, batch, q_state, u, u_scales, v, v_scales, ws, stream);
    }
}

}  // namespace

LowrankWorkspace carve_lowrank_workspace(void* base, int64_t m, int64_t n, int rank, int64_t batch, size_t* bytes) {
    const int64_t kp = (rank + 15) / 16 * 16;
    const int64_t nseg = (n + kSegCols - 1) / kSegCols;
    auto up = [](int64_t x) { return (x + 255) & ~int64_t(255); };
    const int64_t sz_r = up(batch * m * n * 4);
    const int64_t sz_qt = up(batch * kp * n * 4);
    const int64_t sz_y = up(batch * nseg * m * kp * 4);
    const int64_t sz_p = up(batch * m * kp * 4);
    const int64_t sz_al = up(batch * kp * 4);
    if (bytes) *bytes = static_cast<size_t>(sz_r + sz_qt + sz_y + sz_p + sz_al);
    LowrankWorkspace ws{};
    if (base) {
        char* c = static_cast<char*>(base);
        ws.r = reinterpret_cast<float*>(c);
        ws.qt = reinterpret_cast<float*>(c + sz_r);
        ws.ypart = reinterpret_cast<float*>(c + sz_r + sz_qt);
        ws.p = reinterpret_cast<float*>(c + sz_r + sz_qt + sz_y);
        ws.alive = reinterpret_cast<int*>(c + sz_r + sz_qt + sz_y + sz_p);
    }
    return ws;
}

hipError_t launch_lowrank_compress(int a_dtype, const void* a, float* ahat, float* err, int64_t m, int64_t n,
                                   int rank, int iters, int factor_bits, int64_t batch, float* q_state, void* u,
                                   float* u_scales, void* v, float* v_scales, void* workspace,
                                   hipStream_t stream) {
    const LowrankWorkspace ws = carve_lowrank_workspace(workspace, m, n, rank, batch, nullptr);
    if (a_dtype == 0)
        return dispatch_rank(static_cast<const uint16_t*>(a), ahat, err, m, n, rank, iters, factor_bits, batch,
                             q_state, u, u_scales, v, v_scales, ws, stream);
    return dispatch_rank(static_cast<const float*>(a), ahat, err, m, n, rank, iters, factor_bits, batch, q_state,
                         u, u_scales, v, v_scales, ws, stream);
}

hipError_t launch_lowrank_decompress(int factor_bits, const void* u, const float* u_scales, const void* v,
                                     const float* v_scales, float* ahat, int64_t m, int64_t n, int rank,
                                     int64_t batch, hipStream_t stream) {
    int64_t rtotal = round8(batch * ((m + kRecRows - 1) / kRecRows) * ((n + kRecCols - 1) / kRecCols));
    const uint16_t* a = nullptr;
    float* err = nullptr;
    int k = rank;
    void* args[] = {&a, &ahat, &err, &u, &u_scales, &v, &v_scales, &m, &n, &k, &batch, &rtotal};
    return factor_bits == 4 ? go(&k_lr_reconstruct<false, uint16_t, 4>, rtotal, args, stream)
                            : go(&k_lr_reconstruct<false, uint16_t, 32>, rtotal, args, stream);
}

}  // namespace cf
