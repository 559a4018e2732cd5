// cf_quant.hip - fused 1/2-bit residual compression with error feedback, its
// receiver-side decode, and the warmup initialisation, for gfx950.
//
// Method: "Accelerating Parallel Diffusion Model Serving with Residual
// Compression" (CompactFusion summary), section Approach (residual against the
// previous reconstruction, sender-side error feedback) and the measured-effects
// table (Compact-1bit, Compact-2bit, warmup steps).
//
// Work mapping (wave64).  A wave tile is 2*IPS consecutive groups (256*IPS
// elements).  Wave instruction k (0 <= k < IPS) covers elements
// [256k, 256k + 256) of the tile: lane j holds the 4 consecutive elements
// 256k + 4j .. 256k + 4j + 3, so every load and store instruction touches one
// contiguous span (1 KiB of fp32 state, 512 B of bf16 activation) and each half
// wave (32 lanes) owns one whole group of 128 elements.  The group reduction
// (sum or max of |r|) is a 5-step xor butterfly (16, 8, 4, 2, 1) inside the half
// wave; every lane ends with the same value.  Activations and state are read, and
// state written, with non-temporal accesses: each byte is touched once per step,
// so nothing is worth keeping in L2 and the end-of-kernel write-back stays short.
// One pass per element: the activation and reconstruction are read once, the
// reconstruction and error written once, codes and the scale written once per
// group.  No atomics, no inter-block communication.
//
// Launch shape (measured on MI355X): the senders run one instruction per stream per
// tile in one-wave blocks at every call size (2-3% faster than 256-thread blocks on a
// whole FLUX step, 1.5% faster than two instructions per tile in 128-thread blocks on
// one layer's K and V), with their blocks renumbered into runs per XCD
// (run_order_block, cf_vec.h).  The decode of a whole step runs 256-thread blocks, its bf16
// variant one-wave blocks; a small decode call uses two instructions per tile and
// 128-thread blocks, which keeps more bytes in flight per wave when the grid alone
// cannot fill the chip for long.
//
// Numerics: fp32 throughout, built with -ffp-contract=off so that every add and
// multiply rounds once, in the order written; the 2-bit scale uses IEEE division.

#include "cf_internal.h"
#include "cf_vec.h"

namespace cf {
namespace {

// Value held by lane (this lane ^ mask) / (this lane + delta), as 32-bit words.
__device__ __forceinline__ float xor_lane(float v, int mask) { return __shfl_xor(v, mask, 64); }
__device__ __forceinline__ uint32_t down_lane(uint32_t v, int delta) {
    return static_cast<uint32_t>(__shfl_down(static_cast<int>(v), delta, 64));
}

// Decoded value of one code (the expression shared by sender and receiver).
template <int BITS>
__device__ __forceinline__ float dequant(uint32_t c, float s) {
    if constexpr (BITS == 1) {
        return (c & 1u) ? -s : s;
    } else {
        const float lvl = (c & 2u) ? 1.5f * s : 0.5f * s;
        return (c & 1u) ? -lvl : lvl;
    }
}

template <int BITS>
__device__ __forceinline__ vf4 dequant4(uint32_t c, float s) {
    return vf4{dequant<BITS>(c, s), dequant<BITS>(c >> BITS, s), dequant<BITS>(c >> (2 * BITS), s),
               dequant<BITS>(c >> (3 * BITS), s)};
}

// Sender modes.  kEF: r = a - ahat; ahat += d; err = a - ahat (the method).
// kNoEF (ablation without error feedback): r = a - a_prev; ahat += d (the receiver's
// mirror); no err.  kNaive (ablation: the activation itself is quantized): r = a;
// ahat = d; no err.
enum SenderMode { kEF = 0, kNoEF = 1, kNaive = 2 };

template <int BITS, typename ActT, int IPS, int BLOCK, int MODE>
__global__ __launch_bounds__(BLOCK) void k_compress(const ActT* __restrict__ a, const ActT* __restrict__ a_prev,
                                                     float* __restrict__ ahat, float* __restrict__ err,
                                                     uint8_t* __restrict__ codes, float* __restrict__ scales,
                                                     int64_t ngroups) {
    constexpr int kWaves = BLOCK / 64;
    const int lane = threadIdx.x & 63;
    const int hl = lane & 31;  // lane within the half wave that owns a group
    const int64_t tile = static_cast<int64_t>(run_order_block<kRunWaves / kWaves>()) * kWaves + (threadIdx.x >> 6);
    const int64_t g0 = tile * (2 * IPS) + (lane >> 5);
    if (tile * (2 * IPS) >= ngroups) return;  // uniform per wave

    vf4 x[IPS], h[IPS];
    int64_t gi[IPS];
    bool ok[IPS];
#pragma unroll
    for (int k = 0; k < IPS; ++k) {
        const int64_t g = g0 + 2 * k;
        ok[k] = g < ngroups;
        gi[k] = ok[k] ? g : ngroups - 1;  // ragged tail: reload the last group, skip the stores
        const int64_t off = gi[k] * kGroup + hl * 4;
        x[k] = load_act4(a, off);
        if constexpr (MODE == kNoEF) h[k] = load_act4(a_prev, off);  // reference: previous activation
        else if constexpr (MODE == kEF) h[k] = ld_nt(ahat + off);
        else h[k] = vf4{0.f, 0.f, 0.f, 0.f};
    }
    vf4 hprev[IPS];
    if constexpr (MODE == kNoEF) {
#pragma unroll
        for (int k = 0; k < IPS; ++k) hprev[k] = ld_nt(ahat + gi[k] * kGroup + hl * 4);
    }

#pragma unroll
    for (int k = 0; k < IPS; ++k) {
        const vf4 r = x[k] - h[k];
        float s;
        uint32_t code;
        if constexpr (BITS == 1) {
            float L = fabsf(r.x);
            L = L + fabsf(r.y);
            L = L + fabsf(r.z);
            L = L + fabsf(r.w);
            L = L + xor_lane(L, 16);
            L = L + xor_lane(L, 8);
            L = L + xor_lane(L, 4);
            L = L + xor_lane(L, 2);
            L = L + xor_lane(L, 1);
            s = L / 128.0f;
            code = (r.x < 0.0f ? 1u : 0u) | (r.y < 0.0f ? 2u : 0u) | (r.z < 0.0f ? 4u : 0u) |
                   (r.w < 0.0f ? 8u : 0u);
        } else {
            float M = fmaxf(fmaxf(fabsf(r.x), fabsf(r.y)), fmaxf(fabsf(r.z), fabsf(r.w)));
            M = fmaxf(M, xor_lane(M, 16));
            M = fmaxf(M, xor_lane(M, 8));
            M = fmaxf(M, xor_lane(M, 4));
            M = fmaxf(M, xor_lane(M, 2));
            M = fmaxf(M, xor_lane(M, 1));
            s = M / 1.5f;
            code = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t sign = r[i] < 0.0f ? 1u : 0u;
                const uint32_t mag = fabsf(r[i]) > s ? 1u : 0u;
                code |= (sign | (mag << 1)) << (2 * i);
            }
        }
        const vf4 d = dequant4<BITS>(code, s);
        vf4 hn, e;
        if constexpr (MODE == kEF) {
            hn = h[k] + d;
            e = x[k] - hn;
        } else if constexpr (MODE == kNoEF) {
            hn = hprev[k] + d;
        } else {
            hn = d;
        }

        // Gather the group's codes into dwords: 1-bit lanes hold a nibble (8 lanes
        // per dword), 2-bit lanes a byte (4 lanes per dword).
        uint32_t w;
        if constexpr (BITS == 1) {
            w = code | (down_lane(code, 1) << 4);
            w = w | (down_lane(w, 2) << 8);
            w = w | (down_lane(w, 4) << 16);
        } else {
            w = code | (down_lane(code, 1) << 8);
            w = w | (down_lane(w, 2) << 16);
        }

        if (ok[k]) {
            const int64_t off = gi[k] * kGroup + hl * 4;
            st_nt(ahat + off, hn);
            if constexpr (MODE == kEF) {
                if (err) st_nt(err + off, e);  // the error buffer is optional (wave-uniform test)
            }
            if constexpr (BITS == 1) {
                if ((hl & 7) == 0) *reinterpret_cast<uint32_t*>(codes + gi[k] * 16 + (hl >> 1)) = w;
            } else {
                if ((hl & 3) == 0) *reinterpret_cast<uint32_t*>(codes + gi[k] * 32 + hl) = w;
            }
            if (hl == 0) scales[gi[k]] = s;
        }
    }
}

// RUNS: blocks in runs per XCD (run_order_block), else in plain order.
template <int BITS, int IPS, int BLOCK, bool OUT16, bool RUNS>
__global__ __launch_bounds__(BLOCK) void k_decompress(const uint8_t* __restrict__ codes,
                                                       const float* __restrict__ scales,
                                                       float* __restrict__ ahat, uint16_t* __restrict__ out,
                                                       int64_t ngroups) {
    constexpr int kWaves = BLOCK / 64;
    const int lane = threadIdx.x & 63;
    const int hl = lane & 31;
    const uint32_t block = run_order_block<RUNS ? kRunWaves / kWaves : 0>();
    const int64_t tile = static_cast<int64_t>(block) * kWaves + (threadIdx.x >> 6);
    const int64_t g0 = tile * (2 * IPS) + (lane >> 5);
    if (tile * (2 * IPS) >= ngroups) return;

    vf4 h[IPS];
    float s[IPS];
    uint32_t code[IPS];
    int64_t gi[IPS];
    bool ok[IPS];
#pragma unroll
    for (int k = 0; k < IPS; ++k) {
        const int64_t g = g0 + 2 * k;
        ok[k] = g < ngroups;
        gi[k] = ok[k] ? g : ngroups - 1;
        if constexpr (BITS == 1) {
            code[k] = (static_cast<uint32_t>(codes[gi[k] * 16 + (hl >> 1)]) >> ((hl & 1) * 4)) & 0xFu;
        } else {
            code[k] = codes[gi[k] * 32 + hl];
        }
        s[k] = scales[gi[k]];
        h[k] = ld_nt(ahat + gi[k] * kGroup + hl * 4);
    }
#pragma unroll
    for (int k = 0; k < IPS; ++k) {
        const vf4 hn = h[k] + dequant4<BITS>(code[k], s[k]);
        if (ok[k]) {
            const int64_t off = gi[k] * kGroup + hl * 4;
            st_nt(ahat + off, hn);
            if constexpr (OUT16) __builtin_nontemporal_store(to_bf16x4(hn), reinterpret_cast<vu2*>(out + off));
        }
    }
}

// Warmup: ahat = a (widened), err = 0 when err is given.  4 elements per thread.
template <typename ActT, int BLOCK = 256>
__global__ __launch_bounds__(BLOCK) void k_init(const ActT* __restrict__ a, float* __restrict__ ahat,
                                                 float* __restrict__ err, int64_t nquads) {
    const int64_t q = static_cast<int64_t>(blockIdx.x) * BLOCK + threadIdx.x;
    if (q >= nquads) return;
    st_nt(ahat + q * 4, load_act4(a, q * 4));
    if (err) st_nt(err + q * 4, vf4{0.f, 0.f, 0.f, 0.f});
}

// Decode calls of at least this many groups (about 8 FLUX-shard tensors) take the large
// shape.
constexpr int64_t kLargeCall = int64_t(1) << 17;

template <typename K>
hipError_t launch(K kernel, int64_t ngroups, int ips, int block, void** args, hipStream_t stream) {
    const int64_t tiles = (ngroups + 2 * ips - 1) / (2 * ips);
    const int64_t waves_per_block = block / 64;
    const int64_t blocks = (tiles + waves_per_block - 1) / waves_per_block;
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(static_cast<unsigned>(blocks)),
                           dim3(block), args, 0, stream);
}

template <int BITS, typename ActT, int MODE>
hipError_t run_compress(const ActT* a, const ActT* a_prev, float* ahat, float* err, uint8_t* codes,
                        float* scales, int64_t ngroups, hipStream_t stream) {
    void* args[] = {&a, &a_prev, &ahat, &err, &codes, &scales, &ngroups};
    return launch(&k_compress<BITS, ActT, 1, 64, MODE>, ngroups, 1, 64, args, stream);
}

template <typename ActT, int MODE>
hipError_t compress_bits(int bits, const void* a, const void* a_prev, float* ahat, float* err, uint8_t* codes,
                         float* scales, int64_t ng, hipStream_t stream) {
    const auto* x = static_cast<const ActT*>(a);
    const auto* xp = static_cast<const ActT*>(a_prev);
    return bits == 1 ? run_compress<1, ActT, MODE>(x, xp, ahat, err, codes, scales, ng, stream)
                     : run_compress<2, ActT, MODE>(x, xp, ahat, err, codes, scales, ng, stream);
}

template <int BITS, bool OUT16>
hipError_t run_decompress(const uint8_t* codes, const float* scales, float* ahat, uint16_t* out, int64_t ngroups,
                          hipStream_t stream) {
    void* args[] = {&codes, &scales, &ahat, &out, &ngroups};
    if (ngroups >= kLargeCall) {
        // the decode alone streams fastest in 256-thread blocks, with its bf16 copy in
        // one-wave blocks (FLUX step: 0.44 ms vs 0.45 ms, and 0.56 ms vs 0.57 ms)
        if constexpr (OUT16) return launch(&k_decompress<BITS, 1, 64, OUT16, true>, ngroups, 1, 64, args, stream);
        return launch(&k_decompress<BITS, 1, 256, OUT16, true>, ngroups, 1, 256, args, stream);
    }
    return launch(&k_decompress<BITS, 2, 128, OUT16, false>, ngroups, 2, 128, args, stream);
}

template <typename ActT>
hipError_t run_init(const ActT* a, float* ahat, float* err, int64_t numel, hipStream_t stream) {
    int64_t nquads = numel / 4;
    const int64_t blocks = (nquads + 255) / 256;
    void* args[] = {&a, &ahat, &err, &nquads};
    return hipLaunchKernel(reinterpret_cast<const void*>(&k_init<ActT>), dim3(static_cast<unsigned>(blocks)),
                           dim3(256), args, 0, stream);
}

}  // namespace

hipError_t launch_init(int a_dtype, const void* a, float* ahat, float* err, int64_t numel,
                       hipStream_t stream) {
    if (a_dtype == 0) return run_init(static_cast<const uint16_t*>(a), ahat, err, numel, stream);
    return run_init(static_cast<const float*>(a), ahat, err, numel, stream);
}

hipError_t launch_compress(int bits, int a_dtype, const void* a, float* ahat, float* err,
                           uint8_t* codes, float* scales, int64_t numel, hipStream_t stream) {
    const int64_t ng = numel / kGroup;
    return a_dtype == 0 ? compress_bits<uint16_t, kEF>(bits, a, nullptr, ahat, err, codes, scales, ng, stream)
                        : compress_bits<float, kEF>(bits, a, nullptr, ahat, err, codes, scales, ng, stream);
}

hipError_t launch_compress_ablation(int mode, int bits, int a_dtype, const void* a, const void* a_prev,
                                    float* ahat, uint8_t* codes, float* scales, int64_t numel,
                                    hipStream_t stream) {
    const int64_t ng = numel / kGroup;
    if (mode == kNoEF)
        return a_dtype == 0 ? compress_bits<uint16_t, kNoEF>(bits, a, a_prev, ahat, nullptr, codes, scales, ng, stream)
                            : compress_bits<float, kNoEF>(bits, a, a_prev, ahat, nullptr, codes, scales, ng, stream);
    return a_dtype == 0 ? compress_bits<uint16_t, kNaive>(bits, a, nullptr, ahat, nullptr, codes, scales, ng, stream)
                        : compress_bits<float, kNaive>(bits, a, nullptr, ahat, nullptr, codes, scales, ng, stream);
}

hipError_t launch_decompress(int bits, const uint8_t* codes, const float* scales, float* ahat, uint16_t* out,
                             int64_t numel, hipStream_t stream) {
    const int64_t ng = numel / kGroup;
    if (out)
        return bits == 1 ? run_decompress<1, true>(codes, scales, ahat, out, ng, stream)
                         : run_decompress<2, true>(codes, scales, ahat, out, ng, stream);
    return bits == 1 ? run_decompress<1, false>(codes, scales, ahat, nullptr, ng, stream)
                     : run_decompress<2, false>(codes, scales, ahat, nullptr, ng, stream);
}

}  // namespace cf
