// cf_quant.hip - fused 1/2-bit residual compression with error feedback, its
// receiver-side decode, and the warmup initialisation, for gfx950.
//
// Method: "Accelerating Parallel Diffusion Model Serving with Residual
// Compression" (CompactFusion summary), section Approach (residual against the
// previous reconstruction, sender-side error feedback) and the measured-effects
// table (Compact-1bit, Compact-2bit, warmup steps).
//
// Work mapping (wave64): a group of 128 contiguous elements is owned by one
// 16-lane row of a wavefront, each lane holding 8 consecutive elements, so one
// wave instruction moves 4 whole groups (1 KiB of bf16, 2 KiB of fp32 state) with
// 16-byte per-lane accesses.  The group reduction (sum or max of |r|) runs over
// the 16 lanes of the row with an xor butterfly (8, 4, 2, 1); every lane ends with
// the same value.  The whole step - residual, scale, codes, packing,
// reconstruction update and error - is one pass: each element's activation and
// reconstruction are read once and the reconstruction and error written once.
// Every block covers 16 * TILES groups with TILES independent wave-tiles in
// flight per wave; there are no atomics and no inter-block communication.
//
// Numerics: fp32 throughout, built with -ffp-contract=off so that every add and
// multiply rounds once, in the order written; the 2-bit scale uses IEEE
// division.

#include "cf_internal.h"

namespace cf {
namespace {

constexpr int kBlock = 256;  // 4 waves

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 8 consecutive activations at element offset `off`, widened to fp32 (exact).
__device__ __forceinline__ void load_act8(const uint16_t* __restrict__ a, int64_t off, float (&x)[8]) {
    const uint4 v = *reinterpret_cast<const uint4*>(a + off);
    x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x);
    x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
    x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z);
    x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
}

__device__ __forceinline__ void load_act8(const float* __restrict__ a, int64_t off, float (&x)[8]) {
    const float4 v0 = *reinterpret_cast<const float4*>(a + off);
    const float4 v1 = *reinterpret_cast<const float4*>(a + off + 4);
    x[0] = v0.x; x[1] = v0.y; x[2] = v0.z; x[3] = v0.w;
    x[4] = v1.x; x[5] = v1.y; x[6] = v1.z; x[7] = v1.w;
}

__device__ __forceinline__ void load_f8(const float* __restrict__ p, int64_t off, float (&x)[8]) {
    const float4 v0 = *reinterpret_cast<const float4*>(p + off);
    const float4 v1 = *reinterpret_cast<const float4*>(p + off + 4);
    x[0] = v0.x; x[1] = v0.y; x[2] = v0.z; x[3] = v0.w;
    x[4] = v1.x; x[5] = v1.y; x[6] = v1.z; x[7] = v1.w;
}

__device__ __forceinline__ void store_f8(float* __restrict__ p, int64_t off, const float (&x)[8]) {
    *reinterpret_cast<float4*>(p + off) = make_float4(x[0], x[1], x[2], x[3]);
    *reinterpret_cast<float4*>(p + off + 4) = make_float4(x[4], x[5], x[6], x[7]);
}

// Value held by lane (this lane ^ mask); masks < 16 stay inside the 16-lane row.
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

template <int BITS, typename ActT, int TILES>
__global__ __launch_bounds__(kBlock) void k_compress(const ActT* __restrict__ a, float* __restrict__ ahat,
                                                      float* __restrict__ err, uint8_t* __restrict__ codes,
                                                      float* __restrict__ scales, int64_t ngroups) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int sub = lane & 15;  // lane within the group's 16-lane row
    const int64_t gbase = static_cast<int64_t>(blockIdx.x) * (16 * TILES) + wave * 4 + (lane >> 4);

    float x[TILES][8], h[TILES][8];
    int64_t gi[TILES];
    bool ok[TILES];
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
        const int64_t g = gbase + 16 * t;
        ok[t] = g < ngroups;
        gi[t] = ok[t] ? g : ngroups - 1;  // out-of-range rows reload the last group; stores skipped
        const int64_t off = gi[t] * kGroup + sub * 8;
        load_act8(a, off, x[t]);
        load_f8(ahat, off, h[t]);
    }

#pragma unroll
    for (int t = 0; t < TILES; ++t) {
        float r[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) r[i] = x[t][i] - h[t][i];

        float s;
        uint32_t code = 0;
        if constexpr (BITS == 1) {
            float L = fabsf(r[0]);
#pragma unroll
            for (int i = 1; i < 8; ++i) L = L + fabsf(r[i]);
            L = L + xor_lane(L, 8);
            L = L + xor_lane(L, 4);
            L = L + xor_lane(L, 2);
            L = L + xor_lane(L, 1);
            s = L / 128.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) code |= (r[i] < 0.0f ? 1u : 0u) << i;
        } else {
            float M = fabsf(r[0]);
#pragma unroll
            for (int i = 1; i < 8; ++i) M = fmaxf(M, fabsf(r[i]));
            M = fmaxf(M, xor_lane(M, 8));
            M = fmaxf(M, xor_lane(M, 4));
            M = fmaxf(M, xor_lane(M, 2));
            M = fmaxf(M, xor_lane(M, 1));
            s = M / 1.5f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t sign = r[i] < 0.0f ? 1u : 0u;
                const uint32_t mag = fabsf(r[i]) > s ? 1u : 0u;
                code |= (sign | (mag << 1)) << (2 * i);
            }
        }

        float e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            h[t][i] = h[t][i] + dequant<BITS>(code >> (BITS * i), s);
            e[i] = x[t][i] - h[t][i];
        }

        // Pack: 1-bit -> 4 lanes' bytes per dword, 2-bit -> 2 lanes' halfwords per dword.
        uint32_t packed;
        if constexpr (BITS == 1) {
            packed = code | (down_lane(code, 1) << 8) | (down_lane(code, 2) << 16) | (down_lane(code, 3) << 24);
        } else {
            packed = code | (down_lane(code, 1) << 16);
        }

        if (ok[t]) {
            const int64_t off = gi[t] * kGroup + sub * 8;
            store_f8(ahat, off, h[t]);
            store_f8(err, off, e);
            if constexpr (BITS == 1) {
                if ((sub & 3) == 0) *reinterpret_cast<uint32_t*>(codes + gi[t] * 16 + sub) = packed;
            } else {
                if ((sub & 1) == 0) *reinterpret_cast<uint32_t*>(codes + gi[t] * 32 + sub * 2) = packed;
            }
            if (sub == 0) scales[gi[t]] = s;
        }
    }
}

template <int BITS, int TILES>
__global__ __launch_bounds__(kBlock) void k_decompress(const uint8_t* __restrict__ codes,
                                                        const float* __restrict__ scales,
                                                        float* __restrict__ ahat, int64_t ngroups) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int sub = lane & 15;
    const int64_t gbase = static_cast<int64_t>(blockIdx.x) * (16 * TILES) + wave * 4 + (lane >> 4);

    float h[TILES][8], s[TILES];
    uint32_t code[TILES];
    int64_t gi[TILES];
    bool ok[TILES];
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
        const int64_t g = gbase + 16 * t;
        ok[t] = g < ngroups;
        gi[t] = ok[t] ? g : ngroups - 1;
        if constexpr (BITS == 1) {
            code[t] = codes[gi[t] * 16 + sub];
        } else {
            code[t] = *reinterpret_cast<const uint16_t*>(codes + gi[t] * 32 + sub * 2);
        }
        s[t] = scales[gi[t]];
        load_f8(ahat, gi[t] * kGroup + sub * 8, h[t]);
    }
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
#pragma unroll
        for (int i = 0; i < 8; ++i) h[t][i] = h[t][i] + dequant<BITS>(code[t] >> (BITS * i), s[t]);
        if (ok[t]) store_f8(ahat, gi[t] * kGroup + sub * 8, h[t]);
    }
}

// Warmup: ahat = a (widened), err = 0 when err is given.  8 elements per thread.
template <typename ActT>
__global__ __launch_bounds__(kBlock) void k_init(const ActT* __restrict__ a, float* __restrict__ ahat,
                                                  float* __restrict__ err, int64_t nvec) {
    const int64_t v = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
    if (v >= nvec) return;
    float x[8];
    load_act8(a, v * 8, x);
    store_f8(ahat, v * 8, x);
    if (err) {
        const float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        store_f8(err, v * 8, z);
    }
}

constexpr int kTiles = 2;

template <int BITS, typename ActT>
hipError_t run_compress(const ActT* a, float* ahat, float* err, uint8_t* codes, float* scales,
                        int64_t ngroups, hipStream_t stream) {
    const int64_t blocks = (ngroups + 16 * kTiles - 1) / (16 * kTiles);
    void* args[] = {&a, &ahat, &err, &codes, &scales, &ngroups};
    return hipLaunchKernel(reinterpret_cast<const void*>(&k_compress<BITS, ActT, kTiles>),
                           dim3(static_cast<unsigned>(blocks)), dim3(kBlock), args, 0, stream);
}

template <int BITS>
hipError_t run_decompress(const uint8_t* codes, const float* scales, float* ahat, int64_t ngroups,
                          hipStream_t stream) {
    const int64_t blocks = (ngroups + 16 * kTiles - 1) / (16 * kTiles);
    void* args[] = {&codes, &scales, &ahat, &ngroups};
    return hipLaunchKernel(reinterpret_cast<const void*>(&k_decompress<BITS, kTiles>),
                           dim3(static_cast<unsigned>(blocks)), dim3(kBlock), args, 0, stream);
}

template <typename ActT>
hipError_t run_init(const ActT* a, float* ahat, float* err, int64_t numel, hipStream_t stream) {
    int64_t nvec = numel / 8;
    const int64_t blocks = (nvec + kBlock - 1) / kBlock;
    void* args[] = {&a, &ahat, &err, &nvec};
    return hipLaunchKernel(reinterpret_cast<const void*>(&k_init<ActT>), dim3(static_cast<unsigned>(blocks)),
                           dim3(kBlock), args, 0, stream);
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
    if (a_dtype == 0) {
        const auto* ab = static_cast<const uint16_t*>(a);
        return bits == 1 ? run_compress<1>(ab, ahat, err, codes, scales, ng, stream)
                         : run_compress<2>(ab, ahat, err, codes, scales, ng, stream);
    }
    const auto* af = static_cast<const float*>(a);
    return bits == 1 ? run_compress<1>(af, ahat, err, codes, scales, ng, stream)
                     : run_compress<2>(af, ahat, err, codes, scales, ng, stream);
}

hipError_t launch_decompress(int bits, const uint8_t* codes, const float* scales, float* ahat,
                             int64_t numel, hipStream_t stream) {
    const int64_t ng = numel / kGroup;
    return bits == 1 ? run_decompress<1>(codes, scales, ahat, ng, stream)
                     : run_decompress<2>(codes, scales, ahat, ng, stream);
}

}  // namespace cf
