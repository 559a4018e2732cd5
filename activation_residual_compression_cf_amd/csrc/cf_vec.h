// Device helpers shared by the element-wise kernels: 4-wide fp32 vectors,
// non-temporal loads and stores, bf16 widening and rounding, and the block order of
// the streaming kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace cf {

typedef float vf4 __attribute__((ext_vector_type(4)));
typedef unsigned vu2 __attribute__((ext_vector_type(2)));
typedef int vi4 __attribute__((ext_vector_type(4)));
typedef int vi2 __attribute__((ext_vector_type(2)));

// Non-temporal accesses: every byte of the streamed state is touched once per
// step, so nothing is worth keeping in L2.
__device__ __forceinline__ vf4 ld_nt(const float* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const vf4*>(p));
}
__device__ __forceinline__ void st_nt(float* p, vf4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<vf4*>(p));
}

// Streaming stores through a buffer resource, at device scope and non-temporal (cache
// policy sc1 nt).  A wave builds the resource from a base address it holds in scalar
// registers (one that is the same in every lane: a kernel argument plus a block or
// wave index) and a byte length; each lane passes its byte offset from that base.
// Stores at or past the length are dropped by the hardware.  Measured on a FLUX step of
// 114 tensors of 1024 x 3072, against plain non-temporal stores: the 1-bit sender 1%
// faster, the decode 5%, the low-rank sender 1-1.5%.
constexpr int kStorePolicy = 1 << 1 /* nt */ | 1 << 4 /* sc1 */;
// A value that is the same in every lane, moved to scalar registers.
__device__ __forceinline__ int64_t wave_uniform(int64_t v) {
    const uint64_t u = static_cast<uint64_t>(v);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32));
    return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t stream_rsrc(void* base, uint32_t bytes) {
    // dword 3 of a gfx9 buffer resource: 32-bit data format, the one raw accesses need
    return __builtin_amdgcn_make_buffer_rsrc(base, 0, static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ void st_stream(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, vf4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(vi4, v), r, byte_off, 0, kStorePolicy);
}

// One wave instruction's streaming store of a 1 KiB run: lane l writes bytes
// 16 l .. 16 l + 15 of the run that starts at `run`, an address that must be the same
// in every lane.
__device__ __forceinline__ void st_stream_run(float* run, vf4 v) {
    st_stream(stream_rsrc(run, 1024), (threadIdx.x & 63u) * 16u, v);
}

// The same for 8 bytes per lane: a 512-byte run.
template <typename V8>
__device__ __forceinline__ void st_stream_run8(void* run, V8 v) {
    static_assert(sizeof(V8) == 8, "8 bytes per lane");
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(vi2, v), stream_rsrc(run, 512),
                                          (threadIdx.x & 63u) * 8u, 0, kStorePolicy);
}

// 4 consecutive activations at element offset `off`, widened to fp32 (exact).
__device__ __forceinline__ vf4 load_act4(const uint16_t* __restrict__ a, int64_t off) {
    const vu2 w = __builtin_nontemporal_load(reinterpret_cast<const vu2*>(a + off));
    return vf4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
               __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u)};
}
__device__ __forceinline__ vf4 load_act4(const float* __restrict__ a, int64_t off) { return ld_nt(a + off); }

// Round-to-nearest-even bf16 bits of a finite float, and the exact widening back.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float bf16_widen(uint32_t h) { return __uint_as_float(h << 16); }

// Round-to-nearest-even bf16 of 4 finite floats, packed as 2 words.
__device__ __forceinline__ vu2 to_bf16x4(vf4 v) {
    return vu2{bf16_rne(v.x) | (bf16_rne(v.y) << 16), bf16_rne(v.z) | (bf16_rne(v.w) << 16)};
}

// Block order of the streaming kernels.  The hardware deals consecutive workgroups to
// the eight XCDs in turn, so in plain order the code words and scales of one 128-byte
// line are written (or read) by several L2s, each moving its own partial line (1.15%
// more write traffic for the sender on a FLUX step).  Renumbered, block b, the j-th
// (j = b / 8) dealt to XCD b % 8, takes block ((j / RUN) * 8 + b % 8) * RUN + j % RUN:
// each XCD walks runs of RUN consecutive blocks, and the eight runs of one round lie
// side by side, so lines stay whole while the chip's access front stays compact.
// Blocks past the last whole round keep their own index; the map is a permutation of
// [0, gridDim.x).  RUN = 0 keeps the plain order.  Measured on a FLUX step: runs of
// 128 or 256 waves make the 1-bit sender (one-wave blocks) 1.5% faster than plain
// order, with exactly the algorithmic writes, and the decode about 1.5% faster; runs
// of 512 to 8192 waves are up to 2% slower, and one contiguous range per XCD 3% slower.
// The top-k kernels gain 5% from runs of 64 waves (their own constant); the warmup copy
// and the low-rank reconstruction, whose blocks write whole lines anyway, measured no
// faster in runs and keep the plain order.
constexpr uint32_t kRunWaves = 256;

template <uint32_t RUN>
__device__ __forceinline__ uint32_t run_order_block() {
    const uint32_t b = blockIdx.x;
    if constexpr (RUN == 0) {
        return b;
    } else {
        constexpr uint32_t kRound = 8u * RUN;
        if (b >= gridDim.x / kRound * kRound) return b;
        const uint32_t j = b >> 3;
        return ((j / RUN) * 8u + (b & 7u)) * RUN + j % RUN;
    }
}

}  // namespace cf
