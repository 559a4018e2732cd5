// cf_lowrank.hip - Compact-Lowrank: rank-k subspace iteration on the residual with
// INT4 factors, error feedback, and the receiver-side reconstruction, for gfx950.
//
// Method: "Accelerating Parallel Diffusion Model Serving with Residual
// Compression" (CompactFusion summary): section Approach (the low-rank variant
// factors the step's residual and quantizes both factors to INT4; the sender's error
// feedback is the same as for the quantizers), Key results (the compression ratio
// reached at rank 32), the measured-effects table (2 against 10 subspace iterations)
// and Experimental setup, "Builds on" (subspace iteration as in PowerSGD).
//
// Per tensor (m x n, row-major), with Q the n x k start basis:
//   r = a - Ahat                                   (fp32, kept in the workspace)
//   repeat iters times:  Y = r Q;  P = orth(Y);  Q = r^T P
//   U^ = int4(P), V^ = int4(Q)  (per-column absmax / 7, round half even, [-7, 7]),
//   or the bf16 of P and Q (16-bit factors), or P and Q themselves (fp32)
//   Ahat = Ahat + U^ V^^T;   e = a - Ahat;   q_state = Q (warm start)
// orth(Y) is the thin Q factor with diag(R) >= 0, computed as Cholesky QR with the
// Gram matrix, the factorisation and the triangular solve in fp64 (fp32 Cholesky QR
// loses the factor when kappa(Y)^2 approaches 1/eps_fp32, which warm-started
// iterates on outlier-channel residuals reach).  A column whose Cholesky pivot falls
// to <= 1e-10 trace(Y^T Y) (|R_jj| <= 1e-5 ||Y||_F) is rank deficient: its P column
// is zero and its start vector is kept in q_state.
//
// Kernels (each launch covers every tensor of the batch):
//   k_lr_project    Y partials = r Q over column segments; the first pass also forms
//                   and stores r, and reads Q from q_state (rank padded to a multiple of
//                   16 with zeros).  fp32 MFMA 16x16x4: a lane's float4 of r supplies
//                   4 k-slices, Q^T float4s the matching B operands.
//   k_lr_gram, k_lr_solve  orth: Y = sum of partials (fixed order), fp64 Gram; then
//                   Cholesky with the rank guard and P = Y R^-1; the last solve also
//                   writes U's column maxima for the quantizer.
//   k_lr_backproject Q^T = P^T r, MFMA; each wave of a workgroup owns 64 of its 256
//                   columns over every row; the last one also writes V's column maxima.
//   k_lr_backfore   every iteration but the last, for m <= 1024 and padded rank <= 32:
//                   Q = r^T P and the next Y = r Q in one pass over r.
//   k_lr_pack       INT4 (or bf16 / fp32) factors, scales, q_state update.
//   k_lr_reconstruct Ahat += U^ V^^T (MFMA, factors dequantized on the fly from the
//                   payload) and e = a - Ahat; the receiver runs the same kernel
//                   without e, so both sides produce identical bits.
//   k_lr_reconstruct_v the same on the vector unit for INT4 factors of rank <= 8 when n
//                   is a multiple of 256 (sender and receiver alike).
// Every reduction has a fixed order; there are no atomics.

#include "cf_internal.h"
#include "cf_vec.h"

namespace cf {
namespace {

constexpr int kSegCols = 512;   // columns per projection segment
// Rows per projection workgroup: the first pass streams a and Ahat and writes r, and it
// runs fastest in short workgroups (4 stages of 16 rows); the re-projection re-reads its
// Q operands from L2 at every workgroup's start and keeps 16 stages.
template <bool FIRST>
constexpr int proj_rows() { return FIRST ? 64 : 256; }
constexpr int kBackCols = 256;  // columns per back-projection workgroup
constexpr int kRecRows = 32;    // reconstruction workgroup: 32 rows x 256 columns
constexpr int kRecCols = 256;

__device__ __forceinline__ vf4 mfma4(float a, float b, vf4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
typedef double vd4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ vd4 mfma_f64(double a, double b, vd4 c) {
    return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ vf4 ld4(const float* p) { return *reinterpret_cast<const vf4*>(p); }

// r in the workspace is strip-major: per tensor, strip s holds columns 16 s .. 16 s + 15 of
// every row, row after row (m x 16 floats, contiguous).  Every pass over r then moves 1 KB
// runs (16 rows of one strip) per wave instruction, and the fused pass reads whole strips.
__device__ __forceinline__ int64_t strip_off(int64_t m, int64_t row, int64_t col) {
    return (col >> 4) * (m << 4) + (row << 4) + (col & 15);
}

// Activation loads kept raw until use, so a prefetch does not wait for its data.
template <typename ActT>
struct RawAct;
template <>
struct RawAct<uint16_t> {
    using T = vu2;
    static __device__ __forceinline__ vu2 load(const uint16_t* a, int64_t off) {
        return __builtin_nontemporal_load(reinterpret_cast<const vu2*>(a + off));
    }
    static __device__ __forceinline__ vu2 zero() { return vu2{0u, 0u}; }
    static __device__ __forceinline__ vf4 cvt(vu2 w) {
        return vf4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                   __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u)};
    }
};
template <>
struct RawAct<float> {
    using T = vf4;
    static __device__ __forceinline__ vf4 load(const float* a, int64_t off) { return ld_nt(a + off); }
    static __device__ __forceinline__ vf4 zero() { return vf4{0.f, 0.f, 0.f, 0.f}; }
    static __device__ __forceinline__ vf4 cvt(vf4 w) { return w; }
};

// The hardware hands workgroup w to XCD w % 8.  Renumber so that each XCD walks a
// contiguous range of logical workgroups (consecutive tiles of the same tensors),
// keeping each tensor's small operands (Q^T, P) in one XCD's L2.  `total` is a
// multiple of 8.
__device__ __forceinline__ int64_t xcd_remap(int64_t w, int64_t total) {
    return (w & 7) * (total >> 3) + (w >> 3);
}

// ------------------------------------------------------------- project ----
// Workgroup: 4 waves over columns [c0, c0 + 512) and rows [r0, r0 + proj_rows) (64 rows
// in the first pass, 256 after), in stages of 16 rows.  Wave w owns columns
// c0 + 128 w .. + 127 and keeps the matching Q^T float4 operands (8 column groups x KT
// tiles) in registers for the whole kernel.  Per stage the 16 x 512 slab of r is formed (first pass: a - Ahat, also
// stored to the workspace) or read, one instruction per 256 consecutive columns
// of a row, and staged in LDS; each wave multiplies its 128 columns (MFMA, a lane's
// float4 of r supplying 4 k-slices), the four partial Y tiles are summed in LDS in
// wave order, and the 16 x kp result goes to Ypart[b][segment][row][kp].
// The first pass takes its Q operands from q_state itself (n x k per tensor, row-major;
// rank indices k .. kp - 1 read as 0), later passes from Q^T (kp x n) in the workspace.
template <bool FIRST, typename ActT, int KT>
__global__ __launch_bounds__(256) void k_lr_project(const ActT* __restrict__ a, const float* __restrict__ ahat,
                                                     float* __restrict__ r, const float* __restrict__ qt,
                                                     float* __restrict__ ypart, int64_t m, int64_t n,
                                                     int64_t batch, int64_t nseg, int64_t total, int k) {
    constexpr int kp = 16 * KT;
    constexpr int kStage = 16;
    __shared__ float slab[kStage][kSegCols + 4];
    __shared__ float red[4][kStage][kp + 1];
    const int64_t lw = xcd_remap(blockIdx.x, total);
    constexpr int kProjRows = proj_rows<FIRST>();
    const int64_t rblocks = (m + kProjRows - 1) / kProjRows;
    if (lw >= batch * rblocks * nseg) return;  // uniform per workgroup
    const int64_t b = lw / (rblocks * nseg);
    const int64_t rb = (lw / nseg) % rblocks;
    const int64_t sgi = lw % nseg;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    const int li = lane & 15, lg = lane >> 4;
    const int64_t c0 = sgi * kSegCols;
    const int64_t mn = m * n;

    // Q^T operands: column group g covers columns c0 + 128 w + 16 g .. + 15;
    // lane: Q^T[16 t + li][c0 + 128 w + 16 g + 4 lg .. + 3].
    vf4 qv[8][KT];
    if constexpr (FIRST) {
        const float* qsb = qt + b * n * k;  // q_state
#pragma unroll
        for (int g = 0; g < 8; ++g) {
            const int64_t col = c0 + 128 * wave + 16 * g + 4 * lg;
#pragma unroll
            for (int t = 0; t < KT; ++t) {
                const int kk = 16 * t + li;
                const bool ok = col < n && kk < k;  // n is a multiple of 16: col .. col + 3 < n
#pragma unroll
                for (int i = 0; i < 4; ++i) qv[g][t][i] = ok ? qsb[(col + i) * k + kk] : 0.0f;
            }
        }
    } else {
        const float* qtb = qt + b * kp * n;
#pragma unroll
        for (int g = 0; g < 8; ++g) {
            const int64_t col = c0 + 128 * wave + 16 * g + 4 * lg;
#pragma unroll
            for (int t = 0; t < KT; ++t)
                qv[g][t] = col < n ? ld4(qtb + (16 * t + li) * n + col) : vf4{0.f, 0.f, 0.f, 0.f};
        }
    }

    const int64_t rend = (rb + 1) * kProjRows < m ? (rb + 1) * kProjRows : m;
    // staging.  First pass (a and Ahat, row-major): wave w forms rows sr + 4 w + q, lane l
    // columns c0 + 256 h + 4 l.  Later passes (r, strip-major): instruction (q, h) of wave w
    // reads strip 4 (2 q + h) + w of the segment, lane l row sr + l / 4, columns 4 (l % 4)
    // of the strip, one 1 KB run.
    using RA = RawAct<ActT>;
    typename RA::T pa[4][2];
    vf4 ph[4][2];
    auto fetch = [&](int64_t sr) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                if constexpr (FIRST) {
                    const int64_t col = c0 + 256 * h + 4 * lane;
                    const int64_t off = b * mn + (sr + 4 * wave + q) * n + col;
                    const bool ok = col < n;
                    pa[q][h] = ok ? RA::load(a, off) : RA::zero();
                    ph[q][h] = ok ? ld_nt(ahat + off) : vf4{0.f, 0.f, 0.f, 0.f};
                } else {
                    const int64_t scol = c0 + 16 * (4 * (2 * q + h) + wave);
                    ph[q][h] = scol < n ? ld_nt(r + b * mn + strip_off(m, sr + (lane >> 2), scol + 4 * (lane & 3)))
                                        : vf4{0.f, 0.f, 0.f, 0.f};
                }
            }
    };
    int64_t sr = rb * kProjRows;
    if (sr < rend) fetch(sr);
    for (; sr < rend; sr += kStage) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                if constexpr (FIRST) {
                    *reinterpret_cast<vf4*>(&slab[4 * wave + q][256 * h + 4 * lane]) = RA::cvt(pa[q][h]) - ph[q][h];
                } else {
                    const int st = 4 * (2 * q + h) + wave;
                    *reinterpret_cast<vf4*>(&slab[lane >> 2][16 * st + 4 * (lane & 3)]) = ph[q][h];
                }
            }
        __syncthreads();
        if constexpr (FIRST) {
            // r to the workspace, strip-major: instruction i of wave w stores strip 4 i + w of
            // the segment (its 16 rows of 16 columns, one 1 KB run)
#pragma unroll
            for (int i = 0; i < kSegCols / 64; ++i) {
                const int st = 4 * i + wave;
                const int sst = 4 * i + wave_s;  // the same strip, in scalar registers
                if (c0 + 16 * st < n)
                    st_stream_run(r + b * mn + strip_off(m, sr, c0 + 16 * sst),
                                  *reinterpret_cast<const vf4*>(&slab[lane >> 2][16 * st + 4 * (lane & 3)]));
            }
        }
        if (sr + kStage < rend) fetch(sr + kStage);  // next stage's loads overlap the MFMAs
        vf4 acc[KT];
#pragma unroll
        for (int t = 0; t < KT; ++t) acc[t] = vf4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int g = 0; g < 8; ++g) {
            const vf4 rv = *reinterpret_cast<const vf4*>(&slab[li][128 * wave + 16 * g + 4 * lg]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int t = 0; t < KT; ++t) acc[t] = mfma4(rv[i], qv[g][t][i], acc[t]);
        }
        // acc[t] lane: rows 4 lg + v of the stage, Y column 16 t + li
#pragma unroll
        for (int t = 0; t < KT; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) red[wave][4 * lg + v][16 * t + li] = acc[t][v];
        __syncthreads();
        float* yp = ypart + ((b * nseg + sgi) * m + sr) * kp;
        for (int e = threadIdx.x; e < kStage * kp; e += 256) {
            const int rr = e / kp, kk = e % kp;
            yp[rr * kp + kk] = ((red[0][rr][kk] + red[1][rr][kk]) + red[2][rr][kk]) + red[3][rr][kk];
        }
        // No barrier here: the next stage writes the slab, whose reads all ended before
        // the barrier above, and writes red only after its first barrier, which every
        // wave reaches after its own reads of red.
    }
}

// ---------------------------------------------------------------- orth ----
// orth(Y) in two launches:
//   k_lr_gram   (batch x row blocks) Y = sum of the tensor's partials in order (fp32,
//               written to `p` for the solve), and the fp64 Gram
//               contribution Y_blk^T Y_blk of the block's rows (fp64 MFMA);
//   k_lr_solve  (batch x blocks of 256 rows) G = sum of the block Grams in block
//               order; right-looking Cholesky G = L L^T in LDS with the rank guard
//               (pivot <= 1e-10 trace(G) -> dead column), the same in every workgroup
//               of a tensor; then P[row] = Y[row] L^-T by forward substitution in
//               fp64, in place over Y.
constexpr int64_t gram_rows(int64_t kt) { return kt == 1 ? 256 : (kt == 2 ? 128 : 64); }  // rows per Gram block
template <int KT>
struct GramShape {
    static constexpr int kp = 16 * KT;
    static constexpr int rows = static_cast<int>(gram_rows(KT));
};

template <int KT>
// The partials of Y: nwg == 0, those of a projection, nseg column segments per tensor
// (Ypart[b][segment]); else those of a fused pass over nwg equal ranges of the batch's
// list of `strips`-strip tensors (Ypart[2 w + 1] when tensor b is the second of workgroup
// w's range, else Ypart[2 w]).
__global__ __launch_bounds__(256) void k_lr_gram(const float* __restrict__ ypart, float* __restrict__ p,
                                                  double* __restrict__ gpart, int64_t m, int64_t nseg,
                                                  int64_t batch, int64_t nwg, int64_t strips) {
    constexpr int kp = GramShape<KT>::kp;
    constexpr int GR = GramShape<KT>::rows;
    __shared__ double ys[GR][kp + 1];
    const int64_t gblocks = (m + GR - 1) / GR;
    const int64_t b = blockIdx.x / gblocks;
    const int64_t blk = blockIdx.x % gblocks;
    const int64_t r0 = blk * GR;
    const int tid = threadIdx.x;
    // partial 0 at y0, partial q >= 1 at y1 + (q - 1) ystep
    const int64_t mk = m * kp;
    const float *y0, *y1;
    int64_t ystep;
    if (nwg == 0) {
        y0 = ypart + b * nseg * mk;
        y1 = y0 + mk;
        ystep = mk;
    } else {
        // the workgroups whose ranges hold the tensor's first and last strip: workgroup w
        // starts at strip floor(w L / nwg), so strip x lies in floor(((x + 1) nwg - 1) / L)
        const int64_t nlist = batch * strips, x0 = b * strips;
        const int64_t wlo = ((x0 + 1) * nwg - 1) / nlist;
        const int64_t whi = ((x0 + strips) * nwg - 1) / nlist;
        const int64_t second = wlo * nlist / nwg < x0 ? 1 : 0;  // wlo's range began in tensor b - 1
        nseg = whi - wlo + 1;
        y0 = ypart + (2 * wlo + second) * mk;
        y1 = ypart + 2 * (wlo + 1) * mk;
        ystep = 2 * mk;
    }
    float* pb = p + b * m * kp;
    // Y = sum of the partials in order.  The loads of kSegBatch partials are issued
    // together (indices past the last partial re-read it and are not added), so a thread
    // waits for one batch at a time, not for every partial.
    constexpr int kEPT = GR * kp / 256;
    constexpr int kSegBatch = 3;
    float ysum[kEPT];
    for (int64_t q0 = 0; q0 < nseg; q0 += kSegBatch) {
        float v[kSegBatch][kEPT];
#pragma unroll
        for (int qq = 0; qq < kSegBatch; ++qq) {
            const int64_t q = q0 + qq < nseg ? q0 + qq : nseg - 1;
#pragma unroll
            for (int j = 0; j < kEPT; ++j) {
                const int e = tid + 256 * j;
                const int64_t row = r0 + e / kp < m ? r0 + e / kp : m - 1;
                v[qq][j] = (q == 0 ? y0 : y1 + (q - 1) * ystep)[row * kp + e % kp];
            }
        }
#pragma unroll
        for (int qq = 0; qq < kSegBatch; ++qq) {
            if (q0 + qq >= nseg) break;  // uniform; no memory operation below
#pragma unroll
            for (int j = 0; j < kEPT; ++j) ysum[j] = q0 + qq == 0 ? v[qq][j] : ysum[j] + v[qq][j];
        }
    }
#pragma unroll
    for (int j = 0; j < kEPT; ++j) {
        const int e = tid + 256 * j;
        const int rr = e / kp, kk = e % kp;
        const bool in = r0 + rr < m;
        if (in) pb[(r0 + rr) * kp + kk] = ysum[j];
        ys[rr][kk] = in ? static_cast<double>(ysum[j]) : 0.0;
    }
    __syncthreads();
    // G_blk = Y_blk^T Y_blk on the fp64 MFMA 16x16x4, tile by tile, 4 rows of the
    // block per instruction.  Lane l = i + 16 s holds A[i][s] = Y[4t + s][16 ta + i] and
    // B[s][i] = Y[4t + s][16 tb + i]; the result D[s + 4 v][i] sits in lane l, item v.
    const int wave = tid >> 6, lane = tid & 63, li = lane & 15, lg = lane >> 4;
    double* gp = gpart + (b * gblocks + blk) * kp * kp;
    if constexpr (KT == 1) {
        // one tile: each wave takes a quarter of the rows; partials summed in wave order
        __shared__ double red[4][16][17];
        vd4 acc = vd4{0.0, 0.0, 0.0, 0.0};
        for (int t = wave * (GR / 16); t < (wave + 1) * (GR / 16); ++t) {
            const double y = ys[4 * t + lg][li];
            acc = mfma_f64(y, y, acc);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) red[wave][lg + 4 * v][li] = acc[v];
        __syncthreads();
        const int i = tid >> 4, j = tid & 15;
        gp[i * kp + j] = ((red[0][i][j] + red[1][i][j]) + red[2][i][j]) + red[3][i][j];
    } else {
        for (int tile = wave; tile < KT * KT; tile += 4) {
            const int ta = tile / KT, tb = tile % KT;
            vd4 acc = vd4{0.0, 0.0, 0.0, 0.0};
            for (int t = 0; t < GR / 4; ++t)
                acc = mfma_f64(ys[4 * t + lg][16 * ta + li], ys[4 * t + lg][16 * tb + li], acc);
#pragma unroll
            for (int v = 0; v < 4; ++v) gp[(16 * ta + lg + 4 * v) * kp + 16 * tb + li] = acc[v];
        }
    }
}

// Threads of a factorisation (every solve workgroup factorises its tensor's Gram).
constexpr int kCholThreads = 256;

// G = sum of the tensor's block Grams in block order, then the right-looking Cholesky
// G = L L^T with the rank guard (pivot <= 1e-10 trace(G) -> dead column), in LDS.  The
// whole workgroup (kCholThreads threads) takes part; L is complete when it returns.
template <int KT>
__device__ __forceinline__ void chol_factor(const double* __restrict__ gb, int64_t gblocks, int k,
                                            double (*G)[16 * KT + 1], double (*L)[16 * KT + 1]) {
    constexpr int kp = 16 * KT;
    const int tid = threadIdx.x;
    // The loads of kBlkBatch blocks are issued together (indices past the last block
    // re-read it and are not added).
    constexpr int kEPT = (kp * kp + kCholThreads - 1) / kCholThreads;
    constexpr int kBlkBatch = KT == 4 ? 4 : 8;
    double gs[kEPT];
    for (int64_t q0 = 0; q0 < gblocks; q0 += kBlkBatch) {
        double v[kBlkBatch][kEPT];
#pragma unroll
        for (int qq = 0; qq < kBlkBatch; ++qq) {
            const int64_t q = q0 + qq < gblocks ? q0 + qq : gblocks - 1;
#pragma unroll
            for (int j = 0; j < kEPT; ++j) {
                const int e = tid + kCholThreads * j;
                v[qq][j] = gb[q * kp * kp + (e < kp * kp ? e : 0)];
            }
        }
#pragma unroll
        for (int qq = 0; qq < kBlkBatch; ++qq) {
            if (q0 + qq >= gblocks) break;  // uniform; no memory operation below
#pragma unroll
            for (int j = 0; j < kEPT; ++j) gs[j] = q0 + qq == 0 ? v[qq][j] : gs[j] + v[qq][j];
        }
    }
#pragma unroll
    for (int j = 0; j < kEPT; ++j) {
        const int e = tid + kCholThreads * j;
        if (e < kp * kp) G[e / kp][e % kp] = gs[j];
    }
    __syncthreads();
    double tr = 0.0;
    for (int j = 0; j < kp; ++j) tr += G[j][j];
    const double thresh = 1e-10 * tr;
    __syncthreads();  // every trace read precedes the in-place factorisation
    // One barrier per column.  Every thread reads the pivot d = G[j][j].  Column j of L
    // goes to its own array, and the trailing lower triangle is updated from the
    // unscaled column, G[i][l] -= G[i][j] G[l][j] / d for j < l <= i: the phase reads
    // column j and writes only columns right of it.  One reciprocal square root per
    // column gives the pivot sqrt(d) = d / sqrt(d), the column scale 1 / sqrt(d) and
    // 1 / d, which keeps the phase's dependent chain short.
    static_assert(kp * kp % kCholThreads == 0, "the update covers whole rounds of the workgroup");
    for (int j = 0; j < kp; ++j) {
        const double d = G[j][j];
        const bool dj = !(j < k && d > thresh);
        const double rs = dj ? 0.0 : rsqrt(d);
        const double inv_d = rs * rs;
        for (int i = j + tid; i < kp; i += kCholThreads) L[i][j] = i == j ? d * rs : G[i][j] * rs;
#pragma unroll
        for (int q = 0; q < kp * kp / kCholThreads; ++q) {
            const int e = tid + kCholThreads * q;
            const int i = e / kp, l = e % kp;
            if (l > j && l <= i) G[i][l] -= G[i][j] * G[l][j] * inv_d;
        }
        __syncthreads();
    }
}

// orth's second launch, per tensor and block of 256 rows: the factorisation of the
// tensor's Gram (chol_factor; each of the tensor's workgroups computes the same L, in
// the same order, so one launch replaces a per-tensor factorisation and the solve that
// waited for it), then P[row] = Y[row] L^-T by forward substitution,
// p_j = (y_j - sum_{i<j} L[j][i] p_i) / L[j][j], in fp64, one row per thread, in place
// over Y.  A dead column has 1/L[j][j] = 0 and zeros below it in L, so its p_j is 0 and
// it feeds nothing later; the tensor's first workgroup writes the alive flags.  Every
// lane reads the same factor address in the substitution (a broadcast).
// In the last iteration (cmax not null) the workgroup also writes the INT4 quantizer's
// column maxima of its 256 rows of P = U: cmax[b][block][kk] = max |P[row][kk]| (rows
// past m count as 0), nblk the blocks of U and V per tensor.
template <int KT>
__global__ __launch_bounds__(256) void k_lr_solve(float* __restrict__ p, const double* __restrict__ gpart,
                                                   int* __restrict__ alive, int64_t gblocks, int k,
                                                   int64_t m, int64_t batch, float* __restrict__ cmax,
                                                   int64_t nblk) {
    static_assert(kCholThreads == 256, "the factorisation runs on the solve's workgroup");
    constexpr int kp = 16 * KT;
    __shared__ double G[kp][kp + 1];  // Gram, updated in place; then the substitution's factor
    __shared__ double L[kp][kp + 1];
    __shared__ float cm[4][kp];
    const int64_t rblocks = (m + 255) / 256;
    const int64_t b = blockIdx.x / rblocks;
    const int64_t blk = blockIdx.x % rblocks;
    const int64_t row = blk * 256 + threadIdx.x;
    const bool in = row < m;
    // this thread's row of Y, loaded before the factorisation so its latency is hidden
    float* pr = p + (b * m + (in ? row : m - 1)) * kp;
    vf4 yv[kp / 4];
#pragma unroll
    for (int i = 0; i < kp; i += 4) yv[i / 4] = ld4(pr + i);
    chol_factor<KT>(gpart + b * gblocks * kp * kp, gblocks, k, G, L);
    // The factor of the substitution: L below the diagonal, 1 / L[j][j] on it (0 for a
    // dead column, whose pivot is 0), zeros above; G is no longer read.
    double* lb = &G[0][0];
    for (int e = threadIdx.x; e < kp * kp; e += 256) {
        const int j = e / kp, i = e % kp;
        lb[e] = i < j ? L[j][i] : (i == j && L[j][j] > 0.0 ? 1.0 / L[j][j] : 0.0);
    }
    if (blk == 0 && threadIdx.x < kp) alive[b * kp + threadIdx.x] = L[threadIdx.x][threadIdx.x] > 0.0 ? 1 : 0;
    __syncthreads();
    float pf[kp];
    if (in) {
        double x[kp];
#pragma unroll
        for (int i = 0; i < kp; i += 4) {
            const vf4 v = yv[i / 4];
            x[i] = v[0]; x[i + 1] = v[1]; x[i + 2] = v[2]; x[i + 3] = v[3];
        }
#pragma unroll
        for (int j = 0; j < kp; ++j) {
            double acc = x[j];
#pragma unroll
            for (int i = 0; i < j; ++i) acc = fma(-lb[j * kp + i], x[i], acc);
            x[j] = acc * lb[j * kp + j];
        }
#pragma unroll
        for (int j = 0; j < kp; ++j) pf[j] = static_cast<float>(x[j]);
#pragma unroll
        for (int j = 0; j < kp; j += 4) *reinterpret_cast<vf4*>(pr + j) = vf4{pf[j], pf[j + 1], pf[j + 2], pf[j + 3]};
    }
    if (cmax) {  // uniform per launch
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
        for (int kk = 0; kk < kp; ++kk) {
            float v = in ? fabsf(pf[kk]) : 0.0f;
#pragma unroll
            for (int mask = 32; mask >= 1; mask >>= 1) v = fmaxf(v, __shfl_xor(v, mask, 64));
            if (lane == 0) cm[wave][kk] = v;
        }
        __syncthreads();
        if (threadIdx.x < kp) {
            const int kk = threadIdx.x;
            cmax[(b * nblk + blk) * kp + kk] = fmaxf(fmaxf(cm[0][kk], cm[1][kk]), fmaxf(cm[2][kk], cm[3][kk]));
        }
    }
}

// ---------------------------------------------------------- backproject ----
// Workgroup: 4 waves over columns [c0, c0 + 256) and every row, in stages of 16
// rows.  Per stage the 16 x 256 slab of r (one instruction per row) and the 16 x kp
// block of P are staged in LDS; wave w owns columns c0 + 64 w .. + 63 and
// accumulates Q^T[kk][col] = sum_rows P[row][kk] r[row][col] with MFMA (4 rows per
// k-slice; a lane's float4 of r gives 4 column sets).  No cross-wave reduction.
// In the last iteration (cmax not null) the workgroup also writes the INT4 quantizer's
// column maxima of its 256 rows of Q = V: cmax[b][mb + block][kk] = max over its columns
// of |Q^T[kk][col]|, nblk the blocks of U and V per tensor, mb those of U.
template <int KT>
__global__ __launch_bounds__(256) void k_lr_backproject(const float* r, const float* p,
                                                         float* __restrict__ qt, int64_t m, int64_t n,
                                                         int64_t batch, int64_t total, float* __restrict__ cmax,
                                                         int64_t nblk, int64_t mb) {
    constexpr int kp = 16 * KT;
    constexpr int kStage = 16;
    __shared__ float slab[2][kStage][kBackCols + 4];
    __shared__ float ps[2][kStage][kp + 1];
    const int64_t cblocks = (n + kBackCols - 1) / kBackCols;
    const int64_t lw = xcd_remap(blockIdx.x, total);
    if (lw >= batch * cblocks) return;  // uniform per workgroup
    const int64_t b = lw / cblocks;
    const int64_t c0 = (lw % cblocks) * kBackCols;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int64_t mn = m * n;
    const float* rb = r + b * mn;
    const float* pb = p + b * m * kp;

    vf4 acc[4][KT];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int t = 0; t < KT; ++t) acc[i][t] = vf4{0.f, 0.f, 0.f, 0.f};

    const int64_t nst = m / kStage;
    // Two register buffers and two LDS buffers, addressed by name (the loop is unrolled
    // by two).  While a stage's MFMAs run on one LDS buffer, the wave waits for the next
    // stage's loads and writes them into the other, so each stage needs one barrier and
    // the multiply overlaps the wait.  Every load is unconditional (stages past the end
    // reload the last one and are never used).
    vf4 rq[2][4];
    float pq[2][KT];
    // r is strip-major: instruction q of wave w reads strip 4 q + w of the workgroup's 16, lane
    // l row sr + l / 4 and columns 4 (l % 4) of the strip, one 1 KB run.  A strip past n
    // loads a valid one, whose products only reach output columns that are never stored.
    auto fetch = [&](vf4 (&rx)[4], float (&px)[KT], int64_t st) {
        const int64_t sr = (st < nst ? st : nst - 1) * kStage;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t scol = c0 + 16 * (4 * q + wave) < n ? c0 + 16 * (4 * q + wave) : n - 16;
            rx[q] = ld_nt(rb + strip_off(m, sr + (lane >> 2), scol + 4 * (lane & 3)));
        }
#pragma unroll
        for (int j = 0; j < KT; ++j) {  // kStage * kp = 256 KT values, KT per thread
            const int e = threadIdx.x + 256 * j;
            px[j] = pb[(sr + e / kp) * kp + e % kp];
        }
    };
    auto put = [&](float (&sl)[kStage][kBackCols + 4], float (&pp)[kStage][kp + 1], const vf4 (&rx)[4],
                   const float (&px)[KT]) {
#pragma unroll
        for (int q = 0; q < 4; ++q) *reinterpret_cast<vf4*>(&sl[lane >> 2][16 * (4 * q + wave) + 4 * (lane & 3)]) = rx[q];
#pragma unroll
        for (int j = 0; j < KT; ++j) {
            const int e = threadIdx.x + 256 * j;
            pp[e / kp][e % kp] = px[j];
        }
    };
    auto mult = [&](float (&sl)[kStage][kBackCols + 4], float (&pp)[kStage][kp + 1]) {
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            const vf4 rv = *reinterpret_cast<const vf4*>(&sl[4 * rg + lg][64 * wave + 4 * li]);
            float pv[KT];
#pragma unroll
            for (int t = 0; t < KT; ++t) pv[t] = pp[4 * rg + lg][16 * t + li];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int t = 0; t < KT; ++t) acc[i][t] = mfma4(pv[t], rv[i], acc[i][t]);
        }
    };
    fetch(rq[0], pq[0], 0);
    fetch(rq[1], pq[1], 1);
    put(slab[0], ps[0], rq[0], pq[0]);
    fetch(rq[0], pq[0], 2);
    __syncthreads();
    for (int64_t st = 0; st < nst; st += 2) {
        // stage st is in LDS buffer 0, stage st + 1 in rq[1], stage st + 2 in rq[0]
        mult(slab[0], ps[0]);
        put(slab[1], ps[1], rq[1], pq[1]);
        fetch(rq[1], pq[1], st + 3);
        __syncthreads();
        if (st + 1 >= nst) break;
        mult(slab[1], ps[1]);
        put(slab[0], ps[0], rq[0], pq[0]);
        fetch(rq[0], pq[0], st + 4);
        __syncthreads();
    }
    // acc[i][t] lane: Q^T row 16 t + 4 lg + v, column c0 + 64 w + 4 li + i
    float* qtb = qt + b * kp * n;
    const int64_t wc = c0 + 64 * wave + 4 * li;
    if (wc < n) {
#pragma unroll
        for (int t = 0; t < KT; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const vf4 o = vf4{acc[0][t][v], acc[1][t][v], acc[2][t][v], acc[3][t][v]};
                *reinterpret_cast<vf4*>(qtb + (16 * t + 4 * lg + v) * n + wc) = o;
            }
    }
    if (cmax) {  // uniform per launch
        // per row kk: this lane's 4 columns (none past n), then the 16 lanes of the row
        // group (lane bits 0..3), then the 4 waves
        __shared__ float cm[4][kp];
#pragma unroll
        for (int t = 0; t < KT; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                float x = wc < n ? fmaxf(fmaxf(fabsf(acc[0][t][v]), fabsf(acc[1][t][v])),
                                         fmaxf(fabsf(acc[2][t][v]), fabsf(acc[3][t][v])))
                                 : 0.0f;
#pragma unroll
                for (int mask = 8; mask >= 1; mask >>= 1) x = fmaxf(x, __shfl_xor(x, mask, 64));
                if (li == 0) cm[wave][16 * t + 4 * lg + v] = x;
            }
        __syncthreads();
        if (threadIdx.x < kp) {
            const int kk = threadIdx.x;
            cmax[(b * nblk + mb + c0 / 256) * kp + kk] =
                fmaxf(fmaxf(cm[0][kk], cm[1][kk]), fmaxf(cm[2][kk], cm[3][kk]));
        }
    }
}

// ------------------------------------------------------------ fused pass ----
// Iterations after the first: Q = r^T P (the back-projection) and the next Y = r Q (the
// projection) in one pass over r, which the two passes would otherwise read twice.  With r
// strip-major a strip (16 columns of one tensor over all m rows) is one contiguous block,
// and each 16 x 16 row tile of it is 1 KiB.
// The batch's strips, tensor after tensor, are one list (strip g of the list is at
// r + g m 16, since each tensor's strips follow the last tensor's), cut into nwg equal ranges
// of consecutive strips: workgroup w takes strips [w L / nwg, (w + 1) L / nwg) of the L in
// the list.  nwg fills the chip in whole rounds of workgroups (fused_wgs), whatever the
// batch, and nwg >= batch keeps a range within two tensors.
// Workgroup: 8 waves.  Wave w owns the row tiles T = w + 8 jt (jt < RT) of every strip: it
// loads them (one 1 KiB run per instruction) into registers a strip ahead, copies them into
// its own part of the LDS slot once it is done with the strip before, and is the only wave
// that reads them, so the slot needs no barrier.  Per strip:
//   A  Q^T[kk][c] = sum over rows of P[row][kk] r[row][c]: MFMA 16x16x4 with P^T as the A
//      operand (in registers for the whole workgroup) and 4 rows of a tile as B;
//   the waves' partial Q^T tiles are summed in LDS in wave order (two barriers);
//   B  Y[row][kk] += sum over the strip's columns of r[row][c] Q^T[kk][c]: a lane's float4
//      of a row gives 4 k-slices, Q^T from LDS; the accumulators stay in registers over all
//      of the workgroup's strips.
// Each wave writes its rows of the Y partial of the range's first tensor to Ypart[2 w] and,
// if the range runs into the next tensor, of that tensor to Ypart[2 w + 1] (the P operands
// are reloaded there); the orthonormalisation sums a tensor's partials in workgroup order.
// Used for m <= 1024 and padded rank <= 32; RT = 2, 4 or 8 tiles per wave covers m <= 256,
// 512 or 1024.  Tiles past the last row tile of the tensor re-read that tile: their P rows
// are zero, so they add exact zeros to Q^T, and their Y rows are not stored.
constexpr int kFusedWaves = 8;
constexpr int kFusedMaxRows = 1024;
// Workgroups of the fused pass resident on one CU, from their registers (8 waves each;
// RT = 8: 250-254 VGPRs, 2 waves per SIMD; RT = 4: 144-148, 3; RT = 2: 88-94, 5) and LDS
// (26-86 KB), times the 256 CUs of an MI355X: one round of workgroups.  When the batch
// runs as two halves on two streams (`shared`), a half's round is 7/8 of the chip: a pass
// that takes every CU holds off the other stream's kernels until it ends, and the halves
// then stop overlapping (FLUX shard, two halves: 224 workgroups a pass run r32/q2 at
// 2.23-2.24 ms and r8/q10 at 4.13-4.18 ms; 232 or 256 run r8/q10 at 4.27-4.40 ms).
constexpr int64_t kCUs = 256;
constexpr int64_t fused_round(int64_t m, bool shared) { return kCUs * (m <= 256 ? 2 : 1) * (shared ? 7 : 8) / 8; }
// Workgroups of one fused pass: whole rounds (the ranges are equal, so every workgroup of a
// round ends at about the same time and no round runs part-empty), at least one per tensor,
// and, where the batch is too small to fill a round, ranges of at least kp strips, so that a
// range's Y partial (m kp floats, written once and read once) stays within 1/16 of the
// r it reads (16 m floats per strip).
constexpr int64_t fused_wgs(int64_t m, int64_t n, int64_t kp, int64_t batch, bool shared) {
    const int64_t round = fused_round(m, shared);
    const int64_t full = (batch + round - 1) / round * round;
    const int64_t cap = (batch * (n >> 4) + kp - 1) / kp;
    return full <= cap ? full : (cap > batch ? cap : batch);
}

template <int KT, int RT>
__global__ __launch_bounds__(64 * kFusedWaves) void k_lr_backfore(const float* __restrict__ r,
                                                                   const float* __restrict__ p,
                                                                   float* __restrict__ ypart, int64_t m, int64_t n,
                                                                   int64_t batch, int64_t nwg, int64_t total) {
    constexpr int kp = 16 * KT;
    constexpr int kTile = 256;  // floats of one 16 x 16 tile
    __shared__ float slot[kFusedWaves * RT * kTile];  // wave w's tile jt at (w RT + jt) kTile
    __shared__ float red[kFusedWaves][KT][16][17];
    __shared__ float qs[kp][20];
    const int64_t lw = xcd_remap(blockIdx.x, total);
    if (lw >= nwg) return;  // uniform per workgroup
    const int64_t S = n >> 4, nlist = batch * S;  // strips per tensor, in the list
    const int64_t g0 = lw * nlist / nwg, g1 = (lw + 1) * nlist / nwg;
    const int64_t b0 = g0 / S;  // the range's first tensor
    const int ns = static_cast<int>(g1 - g0);
    // strips of the first tensor (== ns when the range stays in it)
    const int jb = static_cast<int>(((b0 + 1) * S < g1 ? (b0 + 1) * S : g1) - g0);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, li = lane & 15, lg = lane >> 4;
    const int mt = static_cast<int>(m >> 4);
    const float* rs = r + g0 * (m << 4);  // the range's first strip

    // this lane's 16 bytes of tile jt inside a strip
    // (unsigned: a uniform base plus a zero-extended 32-bit offset is one load with a scalar
    // base, so the addresses take no 64-bit vector registers)
    unsigned toff[RT];
#pragma unroll
    for (int jt = 0; jt < RT; ++jt) {
        const int T = wave + kFusedWaves * jt;
        toff[jt] = static_cast<unsigned>((T < mt ? T : mt - 1) * kTile + 4 * lane);
    }
    // Strip j into the registers, and the registers into this wave's part of the slot.
    // Strips loaded ahead: two at rank <= 16, one at rank 17..32 (whose registers are full).
    // In the steady loops below every strip loads one (`sure`: the strip exists), so the
    // compiler counts the loads in flight exactly and waits only for the strip it copies;
    // a load skipped on some path would make it wait for every load at every strip.  Near
    // the range's end nothing past the range is loaded (its copy would never be read).
    constexpr int kDepth = KT == 1 ? 2 : 1;
    vf4 stage[kDepth][RT];
    auto fetch = [&](int j, vf4 (&st)[RT], bool sure) __attribute__((always_inline)) {
        if (!sure && j >= ns) return;  // uniform per workgroup
        const float* src = rs + j * (m << 4);
#pragma unroll
        for (int jt = 0; jt < RT; ++jt) st[jt] = ld_nt(src + toff[jt]);
    };
    float* ws = slot + wave * RT * kTile;
    auto put = [&](const vf4 (&st)[RT]) __attribute__((always_inline)) {
#pragma unroll
        for (int jt = 0; jt < RT; ++jt) *reinterpret_cast<vf4*>(ws + jt * kTile + 4 * lane) = st[jt];
    };

    // P^T operands of A for tensor b, and Y's accumulators set to zero.  Lane:
    // P[16 T + 4 c + lg][16 t + li] for tile jt, chunk c.
    float pv[RT][4][KT];
    vf4 acc[RT][KT];
    auto begin_tensor = [&](int64_t b) __attribute__((always_inline)) {
        const float* pb = p + b * m * kp;
#pragma unroll
        for (int jt = 0; jt < RT; ++jt) {
            const int T = wave + kFusedWaves * jt;
#pragma unroll
            for (int t = 0; t < KT; ++t) acc[jt][t] = vf4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int t = 0; t < KT; ++t)
                    pv[jt][c][t] = T < mt ? pb[(16 * T + 4 * c + lg) * kp + 16 * t + li] : 0.0f;
        }
    };
    // acc[jt][t] lane: Y rows 16 T + 4 lg + v, column 16 t + li
    auto store_y = [&](int seg) __attribute__((always_inline)) {
        float* yp = ypart + (2 * lw + seg) * m * kp;
#pragma unroll
        for (int jt = 0; jt < RT; ++jt) {
            const int T = wave + kFusedWaves * jt;
            if (T < mt)
#pragma unroll
                for (int t = 0; t < KT; ++t)
#pragma unroll
                    for (int v = 0; v < 4; ++v) yp[(16 * T + 4 * lg + v) * kp + 16 * t + li] = acc[jt][t][v];
        }
    };
    begin_tensor(b0);
    fetch(0, stage[0], true);
    put(stage[0]);
#pragma unroll
    for (int d = 0; d < kDepth; ++d) fetch(1 + d < ns ? 1 + d : ns - 1, stage[d], true);  // the copy past ns is unread
    // The change to the next tensor: Y of the first goes out, the new P operands come in,
    // and the wave waits for them right here (a load still in flight where two paths meet
    // would make the compiler wait for every load at every strip).
    auto next_tensor = [&]() __attribute__((always_inline)) {
        store_y(0);
        begin_tensor(b0 + 1);
#pragma unroll
        for (int jt = 0; jt < RT; ++jt)
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int t = 0; t < KT; ++t) asm volatile("" ::"v"(pv[jt][c][t]));
    };
    auto strip = [&](int j, vf4 (&st)[RT], bool sure) __attribute__((always_inline)) {
        // A: this wave's partial Q^T of the strip (two accumulator sets per tile column)
        vf4 qa[2][KT];
#pragma unroll
        for (int t = 0; t < KT; ++t) qa[0][t] = qa[1][t] = vf4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int jt = 0; jt < RT; ++jt) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float bv = ws[jt * kTile + (4 * c + lg) * 16 + li];
#pragma unroll
                for (int t = 0; t < KT; ++t) qa[c & 1][t] = mfma4(pv[jt][c][t], bv, qa[c & 1][t]);
            }
        }
        // qa lane: Q^T rows 16 t + 4 lg + v, strip column li
#pragma unroll
        for (int t = 0; t < KT; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) red[wave][t][4 * lg + v][li] = qa[0][t][v] + qa[1][t][v];
        __syncthreads();
        if (tid < kp * 16) {  // the waves' partials summed in wave order
            const int kk = tid >> 4, cc = tid & 15;
            float q = red[0][kk >> 4][kk & 15][cc];
#pragma unroll
            for (int w = 1; w < kFusedWaves; ++w) q = q + red[w][kk >> 4][kk & 15][cc];
            qs[kk][cc] = q;
        }
        __syncthreads();
        // B: lane's B operand for k-slice i is Q^T[16 t + li][4 lg + i]; its A operand
        // r[16 T + li][4 lg + i]
        vf4 qb[KT];
#pragma unroll
        for (int t = 0; t < KT; ++t) qb[t] = *reinterpret_cast<const vf4*>(&qs[16 * t + li][4 * lg]);
#pragma unroll
        for (int jt = 0; jt < RT; ++jt) {
            const vf4 rv = *reinterpret_cast<const vf4*>(ws + jt * kTile + li * 16 + 4 * lg);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int t = 0; t < KT; ++t) acc[jt][t] = mfma4(rv[i], qb[t][i], acc[jt][t]);
        }
        // The wave is done with its part of the slot: strip j + 1 goes in, and the loads of
        // strip j + 2 start.  (The next writes of red and qs follow the next strip's barriers,
        // which every wave reaches only after its reads of them above.)
        put(st);
        fetch(j + 1 + kDepth, st, sure);
    };
    // The range's strips, one tensor at a time.  The change of tensor sits outside the strip
    // loops: a branch inside them, even one never taken, costs the loops register copies and
    // scalar work at every strip.
    if constexpr (kDepth == 2) {
        // strips [j, j1) of a tensor start with strip j + 1 in stage[0] and j + 2 in stage[1]
        int j = 0, j1 = jb;
        for (;;) {
            for (; j + 1 < j1 && j + 4 < ns; j += 2) {
                strip(j, stage[0], true);
                strip(j + 1, stage[1], true);
            }
            for (; j + 1 < j1; j += 2) {
                strip(j, stage[0], false);
                strip(j + 1, stage[1], false);
            }
            const bool odd = j < j1;  // uniform per workgroup
            if (odd) strip(j++, stage[0], false);
            if (j1 == ns) break;
            next_tensor();
            if (odd) {  // one strip past the pairs: the next strip's copy is in stage[1]
#pragma unroll
                for (int jt = 0; jt < RT; ++jt) {
                    const vf4 x = stage[0][jt];
                    stage[0][jt] = stage[1][jt];
                    stage[1][jt] = x;
                }
            }
            j1 = ns;
        }
    } else {  // (as one loop over the tensors, the rank 17..32 body spills)
        int j = 0;
        for (; j < jb && j + 2 < ns; ++j) strip(j, stage[0], true);
        for (; j < jb; ++j) strip(j, stage[0], false);
        if (jb < ns) {
            next_tensor();
            for (; j + 2 < ns; ++j) strip(j, stage[0], true);
            for (; j < ns; ++j) strip(j, stage[0], false);
        }
    }
    store_y(jb < ns ? 1 : 0);
}

// ------------------------------------------------------------ quantize ----
// Factor f of tensor b: f = 0 is U = P (m rows, row-major m x kp), f = 1 is V = Q
// (n rows, stored transposed as Q^T kp x n).  Row blocks of 256 rows: blocks
// [0, mb) cover U, [mb, mb + nb) cover V, for each tensor.
// The last solve (U) and back-projection (V) leave max |x| per block and column in cmax.
// k_lr_pack:   s = (max over the factor's blocks) / 7; one row per thread:
//              c = rint(x / s) clamped to [-7, 7] (0 if s = 0), nibbles packed low
//              first along the rank index (or the fp32 factor copied); V's rows
//              also refresh q_state where the column is alive.
// The block's factor rows r0 .. r0 + nr - 1 into blk, rows past nr zero.  P rows are
// kp consecutive floats, so the block is one contiguous span, read with coalesced
// 16-byte loads; Q^T holds the factor transposed, so each rank index is a contiguous
// run of the block's rows.  Either way every global access of a wave is one span.
template <int kp>
__device__ __forceinline__ void stage_factor_block(const float* x, int f, int64_t n, int64_t r0, int nr,
                                                   float (*blk)[kp + 1]) {
    const int t = threadIdx.x;
    if (f) {
#pragma unroll
        for (int kk = 0; kk < kp; ++kk) blk[t][kk] = t < nr ? x[kk * n + r0 + t] : 0.0f;
    } else {
#pragma unroll
        for (int i = 0; i < kp / 4; ++i) {
            const int e = 4 * (t + 256 * i);
            const int r = e / kp, c = e % kp;
            const vf4 v = r < nr ? ld4(x + r0 * kp + e) : vf4{0.f, 0.f, 0.f, 0.f};
            blk[r][c] = v[0];
            blk[r][c + 1] = v[1];
            blk[r][c + 2] = v[2];
            blk[r][c + 3] = v[3];
        }
    }
}

template <int KT>
__global__ __launch_bounds__(256) void k_lr_pack(const float* __restrict__ p, const float* __restrict__ qt,
                                                  const float* __restrict__ cmax, const int* __restrict__ alive,
                                                  int64_t m, int64_t n, int k, int factor_bits,
                                                  float* __restrict__ q_state, void* __restrict__ u,
                                                  float* __restrict__ u_scales, void* __restrict__ v,
                                                  float* __restrict__ v_scales) {
    constexpr int kp = 16 * KT;
    constexpr int TPC = 256 / kp;  // threads per column when reducing the block maxima
    __shared__ float blk[256][kp + 1];
    __shared__ float sc[kp];
    __shared__ float part[kp][TPC];
    __shared__ int sal[kp];
    const int t = threadIdx.x;
    const int64_t mb = (m + 255) / 256, nb = (n + 255) / 256;
    const int64_t b = blockIdx.x / (mb + nb);
    const int64_t bi = blockIdx.x % (mb + nb);
    const int f = bi >= mb;
    const int64_t fblk = f ? bi - mb : bi;
    const int64_t r0 = fblk * 256;
    const int64_t rows = f ? n : m;
    const int nr = static_cast<int>(rows - r0 < 256 ? rows - r0 : 256);
    stage_factor_block<kp>(f ? qt + b * kp * n : p + b * m * kp, f, n, r0, nr, blk);
    if (t < kp) sal[t] = alive[b * kp + t];
    if (factor_bits == 4 && t < kp * TPC) {
        const int kk = t % kp, slot = t / kp;
        const float* cm = cmax + (b * (mb + nb) + (f ? mb : 0)) * kp + kk;
        float mm = 0.0f;
        for (int64_t q = slot; q < (f ? nb : mb); q += TPC) mm = fmaxf(mm, cm[q * kp]);
        part[kk][slot] = mm;
    }
    __syncthreads();
    if (factor_bits == 4 && t < kp) {
        float mm = part[t][0];
        for (int q = 1; q < TPC; ++q) mm = fmaxf(mm, part[t][q]);
        const float s = mm / 7.0f;
        sc[t] = s;
        if (fblk == 0 && t < k) (f ? v_scales : u_scales)[b * k + t] = s;
    }
    __syncthreads();
    const int64_t row = r0 + t;
    if (factor_bits == 4 && t < nr) {
        uint32_t words[kp / 8];
#pragma unroll
        for (int w = 0; w < kp / 8; ++w) words[w] = 0;
#pragma unroll
        for (int kk = 0; kk < kp; ++kk) {
            const float s = sc[kk];
            int c = 0;
            if (kk < k && s > 0.0f) {
                float q = rintf(blk[t][kk] / s);
                q = fminf(fmaxf(q, -7.0f), 7.0f);
                c = static_cast<int>(q);
            }
            words[kk / 8] |= (static_cast<uint32_t>(c) & 0xFu) << (4 * (kk % 8));
        }
        // the row's k/2 bytes start at a 16-byte boundary when k % 32 == 0 (one
        // 16-byte store per 32 codes), at a 4-byte boundary when k % 8 == 0
        uint8_t* out = static_cast<uint8_t*>(f ? v : u) + (b * rows + row) * k / 2;
        if ((k & 31) == 0 && (reinterpret_cast<uintptr_t>(u) & 15) == 0 &&
            (reinterpret_cast<uintptr_t>(v) & 15) == 0) {
#pragma unroll
            for (int w = 0; w < kp / 8; w += 4)
                if (8 * w < k)
                    *reinterpret_cast<uint4*>(out + 4 * w) = make_uint4(words[w], words[w + 1], words[w + 2], words[w + 3]);
        } else if ((k & 7) == 0) {
#pragma unroll
            for (int w = 0; w < kp / 8; ++w)
                if (8 * w < k) reinterpret_cast<uint32_t*>(out)[w] = words[w];
        } else {
            for (int q = 0; q < k / 2; ++q) out[q] = static_cast<uint8_t>(words[q / 4] >> (8 * (q % 4)));
        }
    } else if (factor_bits == 16 && t < nr) {
        // round-to-nearest-even bf16 of each element; 8-byte stores when k % 4 == 0
        uint16_t* out = static_cast<uint16_t*>(f ? v : u) + (b * rows + row) * k;
        if ((k & 3) == 0 && (reinterpret_cast<uintptr_t>(f ? v : u) & 7) == 0) {
#pragma unroll
            for (int kk = 0; kk < kp; kk += 4) {
                if (kk >= k) break;
                const uint32_t lo = bf16_rne(blk[t][kk]) | (bf16_rne(blk[t][kk + 1]) << 16);
                const uint32_t hi = bf16_rne(blk[t][kk + 2]) | (bf16_rne(blk[t][kk + 3]) << 16);
                *reinterpret_cast<uint2*>(out + kk) = make_uint2(lo, hi);
            }
        } else {
            for (int kk = 0; kk < k; ++kk) out[kk] = static_cast<uint16_t>(bf16_rne(blk[t][kk]));
        }
    } else if (factor_bits == 32 && t < nr) {
        float* out = static_cast<float*>(f ? v : u) + (b * rows + row) * k;
        if ((k & 3) == 0 && (reinterpret_cast<uintptr_t>(f ? v : u) & 15) == 0) {
#pragma unroll
            for (int kk = 0; kk < kp; kk += 4) {
                if (kk >= k) break;
                *reinterpret_cast<vf4*>(out + kk) = vf4{blk[t][kk], blk[t][kk + 1], blk[t][kk + 2], blk[t][kk + 3]};
            }
        } else {
            for (int kk = 0; kk < k; ++kk) out[kk] = blk[t][kk];
        }
    }
    if (f) {
        // q_state rows r0 .. r0 + nr - 1 (one contiguous span of nr * k floats) = Q where
        // the column is alive, else their previous value; written by the whole
        // workgroup in 16-byte pieces when the layout allows (k % 4 == 0, aligned base)
        float* qs = q_state + (b * n + r0) * k;
        const int cnt = nr * k;
        if ((k & 3) == 0 && (reinterpret_cast<uintptr_t>(q_state) & 15) == 0) {
            for (int e = 4 * t; e < cnt; e += 1024) {
                const int r = e / k, c = e % k;
                vf4 o = vf4{blk[r][c], blk[r][c + 1], blk[r][c + 2], blk[r][c + 3]};
                if (!(sal[c] && sal[c + 1] && sal[c + 2] && sal[c + 3])) {
                    const vf4 old = ld4(qs + e);
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (!sal[c + j]) o[j] = old[j];
                }
                *reinterpret_cast<vf4*>(qs + e) = o;
            }
        } else {
            for (int e = t; e < cnt; e += 256) {
                const int r = e / k, c = e % k;
                if (sal[c]) qs[e] = blk[r][c];
            }
        }
    }
}

// --------------------------------------------------------- reconstruct ----
// Workgroup: 4 waves over columns [c0, c0 + kRecCols) and rows [r0, r0 + kRecRows),
// in stages of 16 rows.  Wave w owns columns c0 + 64 w .. + 63 (4 MFMA tiles) and keeps
// their V^ operands in registers.  Per stage the MFMAs give
// C'[i][j] = sum_kk V^[col i][kk] U^[row j][kk] = R^[row j][col i]  (lane l holds
// R^[row0 + li][col + 4 lg .. + 3]); the 16 x 256 tile goes to LDS, then every wave
// streams 4 whole rows: one load/store instruction covers 256 consecutive columns.
template <int FB>
__device__ __forceinline__ float factor_at(const void* f, const float* scales, int64_t row, int k, int kk) {
    if (kk >= k) return 0.0f;
    if constexpr (FB == 4) {
        const uint8_t byte = static_cast<const uint8_t*>(f)[(row * k + kk) >> 1];
        const int nib = (kk & 1) ? (byte >> 4) : (byte & 0xF);
        const int c = nib >= 8 ? nib - 16 : nib;
        return static_cast<float>(c) * scales[kk];
    } else if constexpr (FB == 16) {
        return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(f)[row * k + kk]) << 16);
    } else {
        return static_cast<const float*>(f)[row * k + kk];
    }
}

// The same value, written so that a batch of them issues every load before any is
// used: the index is clamped into range and the value is multiplied by 1 or 0
// afterwards.  (A select on the loaded value would be turned back into a branch
// around the load; the product cannot be, and a dropped entry becomes +-0, which
// leaves every sum it enters unchanged because the sums start at +0.)
template <int FB>
__device__ __forceinline__ float factor_sel(const void* f, const float* scales, int64_t row, int k, int kk,
                                            bool keep) {
    const int kc = kk < k ? kk : k - 1;
    float x;
    if constexpr (FB == 4) {
        const uint8_t byte = static_cast<const uint8_t*>(f)[(row * k + kc) >> 1];
        const int nib = (kc & 1) ? (byte >> 4) : (byte & 0xF);
        x = static_cast<float>(nib >= 8 ? nib - 16 : nib) * scales[kc];
    } else if constexpr (FB == 16) {
        x = __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(f)[row * k + kc]) << 16);
    } else {
        x = static_cast<const float*>(f)[row * k + kc];
    }
    return x * (keep && kk < k ? 1.0f : 0.0f);
}

template <bool HAS_E, typename ActT, int FB, int KS>
__global__ __launch_bounds__(256) void k_lr_reconstruct(const ActT* __restrict__ a, float* __restrict__ ahat,
                                                         float* __restrict__ err, const void* __restrict__ u,
                                                         const float* __restrict__ u_scales,
                                                         const void* __restrict__ v,
                                                         const float* __restrict__ v_scales, int64_t m,
                                                         int64_t n, int k, int64_t batch, int64_t total) {
    constexpr int kStage = 16;
    constexpr int kNS = kRecRows / kStage;
    __shared__ float tile[kStage][kRecCols + 4];
    __shared__ float uh[kRecRows][4 * KS + 1];  // dequantized U^ rows of this workgroup
    const int64_t rblocks = (m + kRecRows - 1) / kRecRows;
    const int64_t cblocks = (n + kRecCols - 1) / kRecCols;
    // Tiles in hardware order: unlike the projections, whose many workgroups per tensor
    // re-read the same small operands, the reconstruction streams faster when
    // consecutive tiles go to different XCDs (measured 3% over per-XCD ranges).
    const int64_t lw = static_cast<int64_t>(blockIdx.x);
    if (lw >= batch * rblocks * cblocks) return;  // uniform per workgroup
    const int64_t b = lw / (rblocks * cblocks);
    const int64_t r0 = ((lw / cblocks) % rblocks) * kRecRows;
    const int64_t c0 = (lw % cblocks) * kRecCols;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    const int li = lane & 15, lg = lane >> 4;

    const int64_t usz = m * k * FB / 8;  // bytes per tensor
    const int64_t vsz = n * k * FB / 8;
    const void* ub = static_cast<const uint8_t*>(u) + b * usz;
    const void* vb = static_cast<const uint8_t*>(v) + b * vsz;
    const float* usb = FB == 4 ? u_scales + b * k : nullptr;
    const float* vsb = FB == 4 ? v_scales + b * k : nullptr;
    const int64_t nrows = r0 + kRecRows < m ? kRecRows : m - r0;  // multiple of 16
    const int nst = static_cast<int>(nrows / kStage);

    // U^ rows of this workgroup (KS / 2 values per thread, into uh) and the V^ operands
    // of this wave's 4 column tiles (k-slice s: V^[col][4 s + lg]); rows and columns past
    // the tensor read as 0.
    constexpr int kUPT = kRecRows * 4 * KS / 256;
    const int64_t wc0 = c0 + 64 * wave;
    float av[4][KS];
    auto setup_operands = [&]() {
        if constexpr (FB == 4) {
            // INT4: the workgroup's code bytes (its 256 columns of V, its 32 rows of U; each
            // a contiguous, 4-byte aligned span) and both scale vectors are staged in LDS by
            // a few dword loads per thread, and the nibbles are taken from there.  Per-lane
            // byte loads of the operands would outnumber the streaming loads several times.
            constexpr int kVW = kRecCols * 4 * KS / 8;  // dwords of V codes for 4 KS >= k
            constexpr int kUW = kRecRows * 4 * KS / 8;
            __shared__ uint32_t vcode[kVW];
            __shared__ uint32_t ucode[kUW];
            __shared__ float vsc[4 * KS], usc[4 * KS];
            const int64_t ncols = c0 + kRecCols <= n ? kRecCols : n - c0;  // multiple of 16
            const int vwords = static_cast<int>(ncols * k / 8), uwords = static_cast<int>(nrows * k / 8);
            const uint32_t* vsrc = reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(vb) + c0 * k / 2);
            const uint32_t* usrc = reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(ub) + r0 * k / 2);
            uint32_t vw[(kVW + 255) / 256], uw[(kUW + 255) / 256];
    #pragma unroll
            for (int j = 0; j < (kVW + 255) / 256; ++j) {
                const int e = threadIdx.x + 256 * j;
                vw[j] = vsrc[e < vwords ? e : vwords - 1];
            }
    #pragma unroll
            for (int j = 0; j < (kUW + 255) / 256; ++j) {
                const int e = threadIdx.x + 256 * j;
                uw[j] = usrc[e < uwords ? e : uwords - 1];
            }
            const int ks = threadIdx.x < 4 * KS ? threadIdx.x : 0;
            const float vs_ = vsb[ks < k ? ks : k - 1], us_ = usb[ks < k ? ks : k - 1];
    #pragma unroll
            for (int j = 0; j < (kVW + 255) / 256; ++j)
                if (threadIdx.x + 256 * j < kVW) vcode[threadIdx.x + 256 * j] = vw[j];
    #pragma unroll
            for (int j = 0; j < (kUW + 255) / 256; ++j)
                if (threadIdx.x + 256 * j < kUW) ucode[threadIdx.x + 256 * j] = uw[j];
            if (threadIdx.x < 4 * KS) {
                vsc[threadIdx.x] = threadIdx.x < k ? vs_ : 0.0f;
                usc[threadIdx.x] = threadIdx.x < k ? us_ : 0.0f;
            }
            __syncthreads();
            const uint8_t* vbytes = reinterpret_cast<const uint8_t*>(vcode);
            const uint8_t* ubytes = reinterpret_cast<const uint8_t*>(ucode);
            auto nib = [](uint8_t byte, int kk) {
                const int c = (kk & 1) ? (byte >> 4) : (byte & 0xF);
                return static_cast<float>(c >= 8 ? c - 16 : c);
            };
    #pragma unroll
            for (int j = 0; j < kUPT; ++j) {
                const int e = threadIdx.x + 256 * j;
                const int rr = e / (4 * KS), kk = e % (4 * KS);
                const bool keep = rr < nrows && kk < k;
                const float x = nib(ubytes[(keep ? rr * k + kk : 0) >> 1], kk) * usc[kk];
                uh[rr][kk] = keep ? x : 0.0f;
            }
    #pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int cc = 64 * wave + 16 * it + li;  // column within the workgroup
    #pragma unroll
                for (int s = 0; s < KS; ++s) {
                    const int kk = 4 * s + lg;
                    const bool keep = cc < ncols && kk < k;
                    const float x = nib(vbytes[(keep ? cc * k + kk : 0) >> 1], kk) * vsc[kk];
                    av[it][s] = keep ? x : 0.0f;
                }
            }
        } else {
            // 16-bit and fp32 factors: batches of per-lane loads issued together.
            float uvals[kUPT];
    #pragma unroll
            for (int j = 0; j < kUPT; ++j) {
                const int e = threadIdx.x + 256 * j;
                const int rr = e / (4 * KS), kk = e % (4 * KS);
                uvals[j] = factor_sel<FB>(ub, usb, r0 + (rr < nrows ? rr : nrows - 1), k, kk, rr < nrows);
            }
    #pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int64_t col = wc0 + 16 * it + li;
    #pragma unroll
                for (int s = 0; s < KS; ++s)
                    av[it][s] = factor_sel<FB>(vb, vsb, col < n ? col : n - 1, k, 4 * s + lg, col < n);
            }
    #pragma unroll
            for (int j = 0; j < kUPT; ++j) {
                const int e = threadIdx.x + 256 * j;
                uh[e / (4 * KS)][e % (4 * KS)] = uvals[j];
            }
        }
    };

    const int64_t mn = m * n;
    const int64_t col = c0 + 4 * lane;  // streaming column of this lane
    const bool cok = col < n;
    using RA = RawAct<ActT>;
    vf4 hq[4];
    typename RA::T xq[4];
    auto load_stage = [&](int st) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t off = b * mn + (r0 + kStage * st + 4 * wave + q) * n + col;
            hq[q] = cok ? ld_nt(ahat + off) : vf4{0.f, 0.f, 0.f, 0.f};
            if constexpr (HAS_E) xq[q] = cok ? RA::load(a, off) : RA::zero();
        }
    };
    if (nrows == kRecRows && c0 + kRecCols <= n) {
        // Whole tile: the stages run as straight-line code with loads two stages ahead
        // and no branch around any memory operation, so each stage waits for exactly
        // its own loads and never for the stores before them.
        vf4 hb[2][4];
        typename RA::T xb[2][4];
        auto fill = [&](vf4 (&h)[4], typename RA::T (&x)[4], int st) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t off = b * mn + (r0 + kStage * st + 4 * wave + q) * n + col;
                h[q] = ld_nt(ahat + off);
                if constexpr (HAS_E) x[q] = RA::load(a, off);
            }
        };
        fill(hb[0], xb[0], 0);
        fill(hb[1], xb[1], 1);
        setup_operands();  // its factor loads overlap the streaming loads above
        __syncthreads();   // uh is complete
#pragma unroll
        for (int st = 0; st < kNS; ++st) {
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                vf4 acc = vf4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < KS; ++s) acc = mfma4(av[it][s], uh[kStage * st + li][4 * s + lg], acc);
                *reinterpret_cast<vf4*>(&tile[li][64 * wave + 16 * it + 4 * lg]) = acc;
            }
            __syncthreads();
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int rr = 4 * wave + q;
                // the row's run of 256 columns, its address in scalar registers
                const int64_t run = b * mn + (r0 + kStage * st + 4 * wave_s + q) * n + c0;
                const vf4 hn = hb[st & 1][q] + *reinterpret_cast<const vf4*>(&tile[rr][4 * lane]);
                st_stream_run(ahat + run, hn);
                if constexpr (HAS_E) st_stream_run(err + run, RA::cvt(xb[st & 1][q]) - hn);
            }
            if (st + 2 < kNS) fill(hb[st & 1], xb[st & 1], st + 2);
            __syncthreads();
        }
        return;
    }
    setup_operands();
    load_stage(0);
    __syncthreads();  // uh is complete
    for (int st = 0; st < nst; ++st) {
        vf4 acc[4];
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            acc[it] = vf4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s) acc[it] = mfma4(av[it][s], uh[kStage * st + li][4 * s + lg], acc[it]);
            *reinterpret_cast<vf4*>(&tile[li][64 * wave + 16 * it + 4 * lg]) = acc[it];
        }
        __syncthreads();
        vf4 hc[4];
        typename RA::T xc[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            hc[q] = hq[q];
            if constexpr (HAS_E) xc[q] = xq[q];
        }
        if (st + 1 < nst) load_stage(st + 1);  // next stage's loads overlap this stage's stores
        if (cok) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int rr = 4 * wave + q;
                const int64_t off = b * mn + (r0 + kStage * st + rr) * n + col;
                const vf4 hn = hc[q] + *reinterpret_cast<const vf4*>(&tile[rr][4 * lane]);
                st_nt(ahat + off, hn);
                if constexpr (HAS_E) st_nt(err + off, RA::cvt(xc[q]) - hn);
            }
        }
        __syncthreads();
    }
}

// Reconstruction with INT4 factors of rank K <= 8 when every row is a whole number of
// 256-element runs (n % 256 == 0): one-wave blocks over kRvRows rows x 256 columns, in
// runs per XCD like the element-wise senders, so each load and store instruction is one
// 1 KiB run of state.  R^[row][col] = sum over kk of U^[row][kk] V^[col][kk] on the
// vector unit (2 K flops per element, one fused multiply-add per term, kk in order).
// Lane l dequantizes V^ rows col .. col + 3 (K / 2 dwords of codes) once for the wave's
// rows; each U^ row is shared by the wave's lanes.  Sender and receiver both take this
// kernel for such calls, so their results stay identical.
// Measured on the FLUX batch at rank 8 against the 32-row MFMA kernel (three interleaved
// runs each): 2 rows per wave, r8/q10 step 3.955 against 3.967 ms and the receiver 0.444
// against 0.455 ms; 1 row, 3.936 and 0.457 ms (the dequantization per element costs the
// receiver, whose stream is shorter); 4 rows, 3.966 and 0.448 ms.
constexpr int kRvRows = 2;  // rows per wave of k_lr_reconstruct_v
template <bool HAS_E, typename ActT, int K>
__global__ __launch_bounds__(64) void k_lr_reconstruct_v(const ActT* __restrict__ a, float* __restrict__ ahat,
                                                          float* __restrict__ err, const void* __restrict__ u,
                                                          const float* __restrict__ u_scales,
                                                          const void* __restrict__ v,
                                                          const float* __restrict__ v_scales, int64_t m,
                                                          int64_t n, int k, int64_t batch, int64_t total) {
    static_assert(K % 2 == 0 && K <= 8, "even rank up to 8");
    constexpr int R = kRvRows;
    const uint32_t tile = run_order_block<kRunWaves>();
    if (tile >= total) return;  // total: tiles of R rows x 256 columns in the batch, below 2^31
    const int lane = threadIdx.x & 63;
    // the tile's first row of the batch and its column block, in 32-bit arithmetic (uniform)
    const uint32_t tpr = static_cast<uint32_t>(n >> 8);
    const uint32_t rgrp = tile / tpr;
    const uint32_t rg0 = rgrp * R;  // first row of the batch; the R rows lie in one tensor
    const uint32_t b = rg0 / static_cast<uint32_t>(m);
    const int64_t c0 = static_cast<int64_t>(tile - rgrp * tpr) * 256;
    const int64_t col = c0 + 4 * lane;
    using RA = RawAct<ActT>;
    typename RA::T xr[R];
    vf4 h[R];
#pragma unroll
    for (int q = 0; q < R; ++q) {
        const int64_t off = static_cast<int64_t>(rg0 + q) * n + col;
        xr[q] = HAS_E ? RA::load(a, off) : RA::zero();
        h[q] = ld_nt(ahat + off);
    }
    const uint8_t* ub = static_cast<const uint8_t*>(u) + static_cast<int64_t>(rg0) * (K / 2);  // U rows of the batch
    const uint32_t* vw = reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(v) +
                                                           static_cast<int64_t>(b) * (n * K / 2) + col * (K / 2));
    uint8_t ubyte[R][K / 2];
    uint32_t w[K / 2];
#pragma unroll
    for (int d = 0; d < K / 2; ++d) {
        w[d] = vw[d];
#pragma unroll
        for (int q = 0; q < R; ++q) ubyte[q][d] = ub[q * (K / 2) + d];
    }
    auto sext = [](uint32_t c) { return static_cast<float>(static_cast<int>(c ^ 8u) - 8); };
    // V^[col + c][kk], shared by the R rows
    float vx[4][K];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int kk = 0; kk < K; ++kk) {
            const int ni = c * K + kk;  // nibble of V^[col + c][kk] within the lane's dwords
            vx[c][kk] = sext((w[ni >> 3] >> (4 * (ni & 7))) & 0xFu) * v_scales[b * K + kk];
        }
#pragma unroll
    for (int q = 0; q < R; ++q) {
        float us[K];
#pragma unroll
        for (int kk = 0; kk < K; ++kk)
            us[kk] = sext((kk & 1) ? (ubyte[q][kk >> 1] >> 4) : (ubyte[q][kk >> 1] & 0xFu)) * u_scales[b * K + kk];
        vf4 rh;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            float acc = 0.0f;
#pragma unroll
            for (int kk = 0; kk < K; ++kk) acc = fmaf(us[kk], vx[c][kk], acc);
            rh[c] = acc;
        }
        const vf4 hn = h[q] + rh;
        const int64_t run = static_cast<int64_t>(rg0 + q) * n + c0;
        st_stream_run(ahat + run, hn);
        if constexpr (HAS_E) st_stream_run(err + run, RA::cvt(xr[q]) - hn);
    }
}

// ------------------------------------------------------------- launchers --
int64_t round8(int64_t x) { return (x + 7) & ~int64_t(7); }

// Workgroup counts of every launch of one call; the launches and the argument check
// share this computation.  Every workgroup has 256 threads (kCholThreads for the
// factorisation, one workgroup per tensor).
struct LowrankGrids {
    int64_t kp, nseg, fwgs, gblocks;  // fwgs: workgroups (strip ranges) of a fused pass
    int64_t project_first, project, gram, solve, backproject, backfore, quant, reconstruct;
    bool fused;  // iterations after the first run the fused pass
};

LowrankGrids lowrank_grids(int64_t m, int64_t n, int rank, int64_t batch, bool shared = false) {
    LowrankGrids g;
    g.kp = (rank + 15) / 16 * 16;
    g.nseg = (n + kSegCols - 1) / kSegCols;
    g.gblocks = (m + gram_rows(g.kp / 16) - 1) / gram_rows(g.kp / 16);
    g.project_first = round8(batch * ((m + proj_rows<true>() - 1) / proj_rows<true>()) * g.nseg);
    g.project = round8(batch * ((m + proj_rows<false>() - 1) / proj_rows<false>()) * g.nseg);
    g.gram = batch * g.gblocks;
    g.solve = batch * ((m + 255) / 256);
    g.backproject = round8(batch * ((n + kBackCols - 1) / kBackCols));
    g.fused = g.kp <= 32 && m <= kFusedMaxRows;
    g.fwgs = fused_wgs(m, n, g.kp, batch, shared);
    g.backfore = round8(g.fwgs);
    g.quant = batch * ((m + 255) / 256 + (n + 255) / 256);
    g.reconstruct = round8(batch * ((m + kRecRows - 1) / kRecRows) * ((n + kRecCols - 1) / kRecCols));
    return g;
}

template <typename K>
hipError_t go(K kernel, int64_t blocks, void** args, hipStream_t stream) {
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(static_cast<unsigned>(blocks)), dim3(256),
                           args, 0, stream);
}

// k-slices of the reconstruction: ceil(k / 4), instantiated for the rank buckets.
template <bool HAS_E, typename ActT, int FB>
hipError_t launch_reconstruct_fb(int k, int64_t total, void** args, hipStream_t stream) {
    const int ks = (k + 3) / 4;
    if (ks <= 2) return go(&k_lr_reconstruct<HAS_E, ActT, FB, 2>, total, args, stream);
    if (ks <= 4) return go(&k_lr_reconstruct<HAS_E, ActT, FB, 4>, total, args, stream);
    if (ks <= 8) return go(&k_lr_reconstruct<HAS_E, ActT, FB, 8>, total, args, stream);
    if (ks <= 12) return go(&k_lr_reconstruct<HAS_E, ActT, FB, 12>, total, args, stream);
    return go(&k_lr_reconstruct<HAS_E, ActT, FB, 16>, total, args, stream);
}

// Whether a reconstruction runs on the vector unit (k_lr_reconstruct_v); the sender and
// the receiver take the same decision.
bool reconstruct_on_valu(int factor_bits, int k, int64_t m, int64_t n, int64_t batch) {
    return factor_bits == 4 && k <= 8 && n % 256 == 0 && batch * m * n / 256 < (int64_t(1) << 31);
}

template <bool HAS_E, typename ActT, int K>
hipError_t launch_reconstruct_v(void** args, int64_t tiles, hipStream_t stream) {
    // the last argument, the grid total, is the tile count for this kernel
    void* vargs[12];
    for (int i = 0; i < 11; ++i) vargs[i] = args[i];
    vargs[11] = &tiles;
    return hipLaunchKernel(reinterpret_cast<const void*>(&k_lr_reconstruct_v<HAS_E, ActT, K>),
                           dim3(static_cast<unsigned>(tiles)), dim3(64), vargs, 0, stream);
}

template <bool HAS_E, typename ActT>
hipError_t launch_reconstruct(int factor_bits, int k, int64_t total, void** args, hipStream_t stream) {
    const int64_t m = *static_cast<int64_t*>(args[7]), n = *static_cast<int64_t*>(args[8]);
    const int64_t batch = *static_cast<int64_t*>(args[10]);
    if (reconstruct_on_valu(factor_bits, k, m, n, batch)) {
        const int64_t tiles = batch * m / kRvRows * (n / 256);
        if (k == 2) return launch_reconstruct_v<HAS_E, ActT, 2>(args, tiles, stream);
        if (k == 4) return launch_reconstruct_v<HAS_E, ActT, 4>(args, tiles, stream);
        if (k == 6) return launch_reconstruct_v<HAS_E, ActT, 6>(args, tiles, stream);
        return launch_reconstruct_v<HAS_E, ActT, 8>(args, tiles, stream);
    }
    if (factor_bits == 4) return launch_reconstruct_fb<HAS_E, ActT, 4>(k, total, args, stream);
    if (factor_bits == 16) return launch_reconstruct_fb<HAS_E, ActT, 16>(k, total, args, stream);
    return launch_reconstruct_fb<HAS_E, ActT, 32>(k, total, args, stream);
}

// One call's kernels for `batch` tensors on one stream.  With `after_first` set, that
// event is recorded on the stream right after the first projection.
template <typename ActT, int KT>
hipError_t run_lowrank(const ActT* a, float* ahat, float* err, int64_t m, int64_t n, int k, int iters,
                       int factor_bits, int64_t batch, float* q_state, void* u, float* u_scales, void* v,
                       float* v_scales, const LowrankWorkspace& ws, hipStream_t stream, hipEvent_t after_first) {
    const LowrankGrids grid = lowrank_grids(m, n, k, batch, ws.shared);
    int64_t nseg = grid.nseg;
    hipError_t e;
    int64_t ptotal = grid.project;
    int64_t btotal = grid.backproject;
    int64_t ftotal = grid.backfore;
    int64_t mblk = (m + 255) / 256;               // U blocks of the quantizer per tensor
    int64_t nblk = mblk + (n + 255) / 256;        // U and V blocks
    int64_t fwgs = grid.fwgs;
    int64_t strips = n >> 4;
    int64_t none = 0;
    const bool fused = KT <= 2 && grid.fused;
    int64_t pftotal = grid.project_first;
    void* pfargs[] = {&a, &ahat, (void*)&ws.r, (void*)&q_state, (void*)&ws.ypart, &m, &n, &batch, &nseg, &pftotal, &k};
    if ((e = go(&k_lr_project<true, ActT, KT>, pftotal, pfargs, stream)) != hipSuccess) return e;
    void* pargs[] = {&a, &ahat, (void*)&ws.r, (void*)&ws.qt, (void*)&ws.ypart, &m, &n, &batch, &nseg, &ptotal, &k};
    if (after_first && (e = hipEventRecord(after_first, stream)) != hipSuccess) return e;
    for (int it = 0; it < iters; ++it) {
        // orth of Y: its partials come from the column segments of a projection, or from
        // the strip ranges of a fused pass
        int64_t gblocks = grid.gblocks;
        void* gargs[] = {(void*)&ws.ypart, (void*)&ws.p, (void*)&ws.gpart, &m, &nseg, &batch,
                         it > 0 && fused ? (void*)&fwgs : (void*)&none, &strips};
        if ((e = go(&k_lr_gram<KT>, grid.gram, gargs, stream)) != hipSuccess) return e;
        // the last iteration's solve and back-projection also leave the quantizer's
        // column maxima of U and V in cmax
        float* cmax = it + 1 == iters ? ws.cmax : nullptr;
        void* sargs[] = {(void*)&ws.p, (void*)&ws.gpart, (void*)&ws.alive, &gblocks, &k, &m, &batch,
                         (void*)&cmax, &nblk};
        if ((e = go(&k_lr_solve<KT>, grid.solve, sargs, stream)) != hipSuccess) return e;
        void* bargs[] = {(void*)&ws.r, (void*)&ws.p, (void*)&ws.qt, &m, &n, &batch, &btotal, (void*)&cmax, &nblk, &mblk};
        if (it + 1 == iters) {  // the last Q, the one that is sent
            if ((e = go(&k_lr_backproject<KT>, btotal, bargs, stream)) != hipSuccess) return e;
        } else if (fused) {     // Q of this iteration and Y of the next in one pass
            if constexpr (KT <= 2) {
                void* fargs[] = {(void*)&ws.r, (void*)&ws.p, (void*)&ws.ypart, &m, &n, &batch, &fwgs, &ftotal};
                const void* fk = m <= 256   ? reinterpret_cast<const void*>(&k_lr_backfore<KT, 2>)
                                 : m <= 512 ? reinterpret_cast<const void*>(&k_lr_backfore<KT, 4>)
                                            : reinterpret_cast<const void*>(&k_lr_backfore<KT, 8>);
                if ((e = hipLaunchKernel(fk, dim3(static_cast<unsigned>(ftotal)), dim3(64 * kFusedWaves), fargs, 0,
                                         stream)) != hipSuccess)
                    return e;
            }
        } else {
            if ((e = go(&k_lr_backproject<KT>, btotal, bargs, stream)) != hipSuccess) return e;
            if ((e = go(&k_lr_project<false, ActT, KT>, ptotal, pargs, stream)) != hipSuccess) return e;
        }
    }
    {
        const int64_t qblocks = grid.quant;
        void* qargs[] = {(void*)&ws.p, (void*)&ws.qt, (void*)&ws.cmax, (void*)&ws.alive, &m, &n, &k,
                         &factor_bits, &q_state, &u, &u_scales, &v, &v_scales};
        if ((e = go(&k_lr_pack<KT>, qblocks, qargs, stream)) != hipSuccess) return e;
    }
    int64_t rtotal = grid.reconstruct;
    const void* uc = u;
    const void* vc = v;
    const float* usc = u_scales;
    const float* vsc = v_scales;
    void* rargs[] = {&a, &ahat, &err, &uc, &usc, &vc, &vsc, &m, &n, &k, &batch, &rtotal};
    // without an error buffer the sender's reconstruction is the receiver's: ahat += U^ V^^T
    // (a is neither read nor needed)
    if (!err) return launch_reconstruct<false, ActT>(factor_bits, k, rtotal, rargs, stream);
    return launch_reconstruct<true, ActT>(factor_bits, k, rtotal, rargs, stream);
}

template <typename ActT>
hipError_t dispatch_rank(const ActT* a, float* ahat, float* err, int64_t m, int64_t n, int k, int iters,
                         int factor_bits, int64_t batch, float* q_state, void* u, float* u_scales, void* v,
                         float* v_scales, const LowrankWorkspace& ws, hipStream_t stream, hipEvent_t after_first) {
    switch ((k + 15) / 16) {
        case 1: return run_lowrank<ActT, 1>(a, ahat, err, m, n, k, iters, factor_bits, batch, q_state, u, u_scales, v, v_scales, ws, stream, after_first);
        case 2: return run_lowrank<ActT, 2>(a, ahat, err, m, n, k, iters, factor_bits, batch, q_state, u, u_scales, v, v_scales, ws, stream, after_first);
        case 3: return run_lowrank<ActT, 3>(a, ahat, err, m, n, k, iters, factor_bits, batch, q_state, u, u_scales, v, v_scales, ws, stream, after_first);
        default: return run_lowrank<ActT, 4>(a, ahat, err, m, n, k, iters, factor_bits, batch, q_state, u, u_scales, v, v_scales, ws, stream, after_first);
    }
}

// ------------------------------------------------------- two halves, two streams --
// A large call runs its tensors as two halves: the first on the caller's stream, the
// second on a side stream that starts once the first half's first projection is done.
// The halves then stand about one streaming pass apart, so the latency-bound kernels of
// one (orthonormalisation, factor quantization) run while the other streams r, and the
// ramp and drain of each pass overlaps the other half's work.  The side stream has the
// default priority; the caller's stream waits for it before the call's later work.
// Calls below this size run as one sequence: the event round trips would cost more than
// the overlap gains.  So do calls at rank <= 16, whose orthonormalisation is short and
// whose fused passes run best over the whole batch (FLUX shard, one sequence against two
// halves: r8/q10 4.04-4.07 against 4.08-4.10 ms, r16/q4 2.54 against 2.58; at rank 32 the
// halves win, r32/q2 2.23-2.24 against 2.29, r32/q10 5.47-5.52 against 5.75).
constexpr int64_t kSplitElems = int64_t(1) << 24;

// Tensors in the first half, or 0 for one sequence.
int64_t split_first_half(int64_t m, int64_t n, int rank, int64_t batch) {
    return batch >= 2 && rank > 16 && m * n * batch >= kSplitElems ? (batch + 1) / 2 : 0;
}

// The side stream and the two events of one host thread on one device, made on first use
// (with that device current) and kept for the life of the thread.  One set per thread, so
// calls from several host threads never share an event.
struct SplitSync {
    hipStream_t side = nullptr;
    hipEvent_t first_done = nullptr, second_done = nullptr;
    hipError_t err = hipSuccess;
    bool made = false;
};
constexpr int kMaxSplitDevices = 64;
thread_local SplitSync t_split[kMaxSplitDevices];

hipError_t split_sync(SplitSync** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxSplitDevices) return hipErrorInvalidDevice;
    SplitSync& s = t_split[dev];
    if (!s.made) {
        s.made = true;
        s.err = hipStreamCreateWithFlags(&s.side, hipStreamNonBlocking);
        if (s.err == hipSuccess) s.err = hipEventCreateWithFlags(&s.first_done, hipEventDisableTiming);
        if (s.err == hipSuccess) s.err = hipEventCreateWithFlags(&s.second_done, hipEventDisableTiming);
    }
    *out = &s;
    return s.err;
}

template <typename ActT>
hipError_t run_split(const ActT* a, float* ahat, float* err, int64_t m, int64_t n, int k, int iters, int factor_bits,
                     int64_t batch, float* q_state, void* u, float* u_scales, void* v, float* v_scales,
                     void* workspace, int64_t half, hipStream_t stream) {
    SplitSync* sync = nullptr;
    hipError_t e = split_sync(&sync);
    if (e != hipSuccess) return e;
    size_t bytes_first = 0;
    const LowrankWorkspace ws1 = carve_lowrank_workspace(workspace, m, n, k, half, true, &bytes_first);
    const LowrankWorkspace ws2 =
        carve_lowrank_workspace(static_cast<char*>(workspace) + bytes_first, m, n, k, batch - half, true, nullptr);
    const int64_t mn = m * n, fb8 = factor_bits;  // factor bits per (row, rank) pair
    if ((e = dispatch_rank(a, ahat, err, m, n, k, iters, factor_bits, half, q_state, u, u_scales, v, v_scales, ws1,
                           stream, sync->first_done)) != hipSuccess)
        return e;
    if ((e = hipStreamWaitEvent(sync->side, sync->first_done, 0)) != hipSuccess) return e;
    if ((e = dispatch_rank(a + half * mn, ahat + half * mn, err ? err + half * mn : nullptr, m, n, k, iters,
                           factor_bits, batch - half, q_state + half * n * k,
                           static_cast<char*>(u) + half * m * k * fb8 / 8, u_scales ? u_scales + half * k : nullptr,
                           static_cast<char*>(v) + half * n * k * fb8 / 8, v_scales ? v_scales + half * k : nullptr,
                           ws2, sync->side, nullptr)) != hipSuccess)
        return e;
    if ((e = hipEventRecord(sync->second_done, sync->side)) != hipSuccess) return e;
    return hipStreamWaitEvent(stream, sync->second_done, 0);
}

}  // namespace

size_t lowrank_workspace_total(int64_t m, int64_t n, int rank, int64_t batch) {
    size_t one = 0, two = 0;
    const int64_t half = split_first_half(m, n, rank, batch);
    if (!half) {
        carve_lowrank_workspace(nullptr, m, n, rank, batch, false, &one);
        return one;
    }
    carve_lowrank_workspace(nullptr, m, n, rank, half, true, &one);
    carve_lowrank_workspace(nullptr, m, n, rank, batch - half, true, &two);
    return one + two;
}

LowrankWorkspace carve_lowrank_workspace(void* base, int64_t m, int64_t n, int rank, int64_t batch, bool shared,
                                         size_t* bytes) {
    const int64_t kp = (rank + 15) / 16 * 16;
    const int64_t nseg = (n + kSegCols - 1) / kSegCols;
    const int64_t gblocks = lowrank_grids(m, n, rank, batch, shared).gblocks;
    auto up = [](int64_t x) { return (x + 255) & ~int64_t(255); };
    const int64_t sz_r = up(batch * m * n * 4);
    const int64_t sz_qt = up(batch * kp * n * 4);
    const LowrankGrids g = lowrank_grids(m, n, rank, batch, shared);
    const int64_t sz_y = up((g.fused && 2 * g.fwgs > batch * nseg ? 2 * g.fwgs : batch * nseg) * m * kp * 4);
    const int64_t sz_p = up(batch * m * kp * 4);
    const int64_t sz_al = up(batch * kp * 4);
    const int64_t sz_g = up(batch * gblocks * kp * kp * 8);
    const int64_t sz_c = up(batch * ((m + 255) / 256 + (n + 255) / 256) * kp * 4);
    if (bytes) *bytes = static_cast<size_t>(sz_r + sz_qt + sz_y + sz_p + sz_al + sz_g + sz_c);
    LowrankWorkspace ws{};
    ws.shared = shared;
    if (base) {
        char* c = static_cast<char*>(base);
        ws.r = reinterpret_cast<float*>(c);
        c += sz_r;
        ws.qt = reinterpret_cast<float*>(c);
        c += sz_qt;
        ws.ypart = reinterpret_cast<float*>(c);
        c += sz_y;
        ws.p = reinterpret_cast<float*>(c);
        c += sz_p;
        ws.alive = reinterpret_cast<int*>(c);
        c += sz_al;
        ws.gpart = reinterpret_cast<double*>(c);
        c += sz_g;
        ws.cmax = reinterpret_cast<float*>(c);
    }
    return ws;
}

bool lowrank_launches_fit(int64_t m, int64_t n, int rank, int64_t batch) {
    const LowrankGrids g = lowrank_grids(m, n, rank, batch);
    const int64_t blocks[] = {g.project_first, g.project, g.gram, g.solve, g.backproject, g.quant,
                              g.reconstruct};
    for (int64_t b : blocks)
        if (b * 256 > kMaxDispatchItems) return false;
    return g.backfore * 64 * kFusedWaves <= kMaxDispatchItems;
}

hipError_t launch_lowrank_compress(int a_dtype, const void* a, float* ahat, float* err, int64_t m, int64_t n,
                                   int rank, int iters, int factor_bits, int64_t batch, float* q_state, void* u,
                                   float* u_scales, void* v, float* v_scales, void* workspace,
                                   hipStream_t stream) {
    if (const int64_t half = split_first_half(m, n, rank, batch)) {
        if (a_dtype == 0)
            return run_split(static_cast<const uint16_t*>(a), ahat, err, m, n, rank, iters, factor_bits, batch,
                             q_state, u, u_scales, v, v_scales, workspace, half, stream);
        return run_split(static_cast<const float*>(a), ahat, err, m, n, rank, iters, factor_bits, batch, q_state, u,
                         u_scales, v, v_scales, workspace, half, stream);
    }
    const LowrankWorkspace ws = carve_lowrank_workspace(workspace, m, n, rank, batch, false, nullptr);
    if (a_dtype == 0)
        return dispatch_rank(static_cast<const uint16_t*>(a), ahat, err, m, n, rank, iters, factor_bits, batch,
                             q_state, u, u_scales, v, v_scales, ws, stream, nullptr);
    return dispatch_rank(static_cast<const float*>(a), ahat, err, m, n, rank, iters, factor_bits, batch, q_state,
                         u, u_scales, v, v_scales, ws, stream, nullptr);
}

hipError_t launch_lowrank_decompress(int factor_bits, const void* u, const float* u_scales, const void* v,
                                     const float* v_scales, float* ahat, int64_t m, int64_t n, int rank,
                                     int64_t batch, hipStream_t stream) {
    int64_t rtotal = lowrank_grids(m, n, rank, batch).reconstruct;
    const uint16_t* a = nullptr;
    float* err = nullptr;
    int k = rank;
    void* args[] = {&a, &ahat, &err, &u, &u_scales, &v, &v_scales, &m, &n, &k, &batch, &rtotal};
    return launch_reconstruct<false, uint16_t>(factor_bits, k, rtotal, args, stream);
}

}  // namespace cf
