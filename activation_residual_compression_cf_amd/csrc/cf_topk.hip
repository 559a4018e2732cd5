// cf_topk.hip - per-group top-k sparsification of the residual with error
// feedback, and its receiver-side decode, for gfx950.
//
// Method: "Accelerating Parallel Diffusion Model Serving with Residual
// Compression" (CompactFusion summary): section Approach (residual against the
// previous reconstruction, sender-side error feedback) and Limitations, which
// names sparsity beside quantization as the fast compressor families.  The pages
// give no sparsity rule; the one built here: per group of 128 keep the k
// residuals of largest |r| (equal magnitudes to the lower index), sent in
// increasing index order as one index byte and the round-to-nearest-even bf16 of
// r each; ahat adds the sent values, err = a - ahat.
//
// Work mapping: the same as the quantizers.  A half wave (32 lanes) owns one
// group, lane j holds the 4 consecutive elements 4j .. 4j+3, and each load or
// store instruction covers one contiguous span.  Selection needs no sort and no
// LDS.  The keys are the bit patterns of |r| (their integer order is the
// magnitude order), and the k-th largest key T is found bit by bit from the top:
// a candidate T | 2^b is kept while at least k keys reach it, and the counts come
// from wave ballots, popcounted per half.  The search stops early once exactly k
// keys reach T, which smooth data does after about 15 of the 31 bits.  Keys above
// T are kept, and so are the first k - #(key > T) keys equal to T in index order
// (a ballot prefix count).  The same prefix count over the kept flags gives each
// kept element its output slot.

#include "cf_internal.h"
#include "cf_vec.h"

namespace cf {
namespace {

constexpr uint64_t kLoHalf = 0x00000000ffffffffull;

// Number of lanes in this lane's half wave whose predicate holds.  The two
// popcounts are wave-uniform; only the final select depends on the lane.
__device__ __forceinline__ int half_count(bool pred, bool upper) {
    const uint64_t m = __ballot(pred);
    const int lo = __popc(static_cast<uint32_t>(m));
    const int hi = __popc(static_cast<uint32_t>(m >> 32));
    return upper ? hi : lo;
}

template <typename ActT, int BLOCK>
__global__ __launch_bounds__(BLOCK) void k_topk_compress(const ActT* __restrict__ a, float* __restrict__ ahat,
                                                         float* __restrict__ err, uint8_t* __restrict__ idx,
                                                         uint16_t* __restrict__ vals, int k, int64_t ngroups) {
    constexpr int kWaves = BLOCK / 64;
    const int lane = threadIdx.x & 63;
    const int hl = lane & 31;
    const bool upper = lane >= 32;
    const int64_t tile = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
    if (tile * 2 >= ngroups) return;  // uniform per wave
    const int64_t g = tile * 2 + (upper ? 1 : 0);
    const bool ok = g < ngroups;
    const int64_t gi = ok ? g : ngroups - 1;  // ragged tail: recompute the last group, skip the stores
    const int64_t off = gi * kGroup + hl * 4;

    const vf4 x = load_act4(a, off);
    const vf4 h = ld_nt(ahat + off);
    const vf4 r = x - h;
    uint32_t key[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) key[j] = __float_as_uint(r[j]) & 0x7fffffffu;

    // T: the k-th largest key of the group (or a prefix of it that exactly k keys reach).
    uint32_t T = 0;
    int cntT = kGroup;
    for (int b = 30; b >= 0; --b) {
        if (__all(cntT == k)) break;
        const uint32_t cand = T | (1u << b);
        const int cnt = half_count(key[0] >= cand, upper) + half_count(key[1] >= cand, upper) +
                        half_count(key[2] >= cand, upper) + half_count(key[3] >= cand, upper);
        if (cnt >= k) {
            T = cand;
            cntT = cnt;
        }
    }

    // Keys above T are kept; of the keys equal to T, the lowest-indexed k - #above.
    const uint64_t below = ((1ull << lane) - 1ull) & (upper ? ~kLoHalf : kLoHalf);
    int above = 0, eq_before = 0;
    bool eq[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        above += half_count(key[j] > T, upper);
        eq[j] = key[j] == T;
        eq_before += __popcll(__ballot(eq[j]) & below);
    }
    const int need = k - above;
    bool sel[4];
    int sel_before = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        sel[j] = key[j] > T || (eq[j] && eq_before < need);
        eq_before += eq[j] ? 1 : 0;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) sel_before += __popcll(__ballot(sel[j]) & below);

    vf4 hn = h;
    uint32_t v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v[j] = bf16_rne(r[j]);
        if (sel[j]) hn[j] = h[j] + bf16_widen(v[j]);
    }
    const vf4 e = x - hn;

    if (ok) {
        st_nt(ahat + off, hn);
        st_nt(err + off, e);
        uint8_t* gidx = idx + gi * k;
        uint16_t* gval = vals + gi * k;
        int slot = sel_before;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (sel[j]) {
                gidx[slot] = static_cast<uint8_t>(hl * 4 + j);
                gval[slot] = static_cast<uint16_t>(v[j]);
                ++slot;
            }
        }
    }
}

// Receiver: ahat[g*128 + idx] += widened value, one half wave per group, lane j
// taking entries j, j + 32, ...  Index bytes are masked to 7 bits so any payload
// stays inside its group.
template <int BLOCK>
__global__ __launch_bounds__(BLOCK) void k_topk_decompress(const uint8_t* __restrict__ idx,
                                                           const uint16_t* __restrict__ vals,
                                                           float* __restrict__ ahat, int k, int64_t ngroups) {
    constexpr int kWaves = BLOCK / 64;
    const int lane = threadIdx.x & 63;
    const int hl = lane & 31;
    const int64_t tile = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
    const int64_t g = tile * 2 + (lane >> 5);
    if (g >= ngroups) return;
    for (int j = hl; j < k; j += 32) {
        const int64_t t = g * k + j;
        float* p = ahat + g * kGroup + (idx[t] & 127);
        *p = *p + bf16_widen(vals[t]);
    }
}

template <typename K>
hipError_t launch_pairs(K kernel, int64_t ngroups, int block, void** args, hipStream_t stream) {
    const int64_t tiles = (ngroups + 1) / 2;
    const int64_t blocks = (tiles + block / 64 - 1) / (block / 64);
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(static_cast<unsigned>(blocks)),
                           dim3(block), args, 0, stream);
}

// Calls of at least this many groups take 256-thread blocks, smaller ones 128.
constexpr int64_t kLargeTopk = int64_t(1) << 17;

template <typename ActT>
hipError_t run_topk(const ActT* a, float* ahat, float* err, uint8_t* idx, uint16_t* vals, int k, int64_t ngroups,
                    hipStream_t stream) {
    void* args[] = {&a, &ahat, &err, &idx, &vals, &k, &ngroups};
    if (ngroups >= kLargeTopk) return launch_pairs(&k_topk_compress<ActT, 256>, ngroups, 256, args, stream);
    return launch_pairs(&k_topk_compress<ActT, 128>, ngroups, 128, args, stream);
}

}  // namespace

hipError_t launch_topk_compress(int k, int a_dtype, const void* a, float* ahat, float* err, uint8_t* idx,
                                uint16_t* vals, int64_t numel, hipStream_t stream) {
    const int64_t ng = numel / kGroup;
    if (a_dtype == 0) return run_topk(static_cast<const uint16_t*>(a), ahat, err, idx, vals, k, ng, stream);
    return run_topk(static_cast<const float*>(a), ahat, err, idx, vals, k, ng, stream);
}

hipError_t launch_topk_decompress(int k, const uint8_t* idx, const uint16_t* vals, float* ahat, int64_t numel,
                                  hipStream_t stream) {
    int64_t ng = numel / kGroup;
    void* args[] = {&idx, &vals, &ahat, &k, &ng};
    return launch_pairs(&k_topk_decompress<256>, ng, 256, args, stream);
}

}  // namespace cf
