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
// Work mapping.  One wave owns one group: lane l holds elements 2l and 2l+1, so the
// threshold search is wave-uniform and every count is a 64-bit ballot popcount on the
// scalar unit.  Selection needs no sort.  The keys are the bit patterns of |r|, whose
// integer order is the magnitude order, and the k-th largest key T is found bit by bit
// from the top: a candidate T | 2^b is kept while at least k keys reach it.  The
// candidate and the select run on the vector unit (T sits in a VGPR) and the counts on
// the scalar unit, so the two halves of a step issue side by side.  The 31 steps are
// unrolled and stop as soon as exactly k keys reach the candidate.  Keys above T are
// kept, and so are the first k - #(key > T) keys equal to T in index order (a ballot
// prefix count); the same prefix count over the kept flags gives each kept element its
// output slot.
//
// A wave takes kPerWave consecutive groups in straight-line code, with each group's loads
// issued two groups ahead.  Blocks of 8 waves take their groups in per-XCD runs
// (kTopkRunWaves below).  No memory operation sits under a data-dependent branch, so
// the compiler can wait for exactly the loads a group needs.  The payload of the wave's
// groups is one contiguous span of the output (kPerWave*k index bytes, as many bf16
// values).  It is staged in LDS and written as whole dwords once the wave is done; the
// per-element byte stores it replaces cost about a tenth of the kernel's time.  When the
// payload pointers are not 4-byte aligned, and for the last wave's ragged tail, kept
// elements store directly through buffer stores whose unselected lanes get an
// out-of-range offset, which the hardware drops.

#include "cf_internal.h"
#include "cf_vec.h"

namespace cf {
namespace {

typedef float vf2 __attribute__((ext_vector_type(2)));

// Groups per wave and how far ahead their loads are issued.
constexpr int kPerWave = 4;
constexpr int kLead = 2;
constexpr int kBlock = 512;
constexpr uint32_t kDrop = 0x80000000u;  // buffer offset past any range: the store is dropped

// Two consecutive activations of a lane, as loaded, and widened to fp32.
__device__ __forceinline__ uint32_t load_pair(const uint16_t* a, int64_t off) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(a + off));
}
__device__ __forceinline__ vf2 load_pair(const float* a, int64_t off) {
    return __builtin_nontemporal_load(reinterpret_cast<const vf2*>(a + off));
}
__device__ __forceinline__ vf2 widen_pair(uint32_t w) {
    return vf2{__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u)};
}
__device__ __forceinline__ vf2 widen_pair(vf2 w) { return w; }

// acc + the number of set bits of `mask` at lanes below this one (two mbcnt steps).
__device__ __forceinline__ int count_below(uint64_t mask, int acc) {
    return static_cast<int>(__builtin_amdgcn_mbcnt_hi(
        static_cast<uint32_t>(mask >> 32), __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), acc)));
}

// Where a group's payload goes: LDS staging slots, or the output through buffer stores.
struct StagedPayload {
    uint8_t* idx;  // LDS, this group's k slots
    uint16_t* val;
    __device__ void put(int slot, bool keep, uint32_t i, uint32_t v) const {
        if (keep) {
            idx[slot] = static_cast<uint8_t>(i);
            val[slot] = static_cast<uint16_t>(v);
        }
    }
};
struct DirectPayload {
    __amdgpu_buffer_rsrc_t idx, val;  // this group's k bytes / k values
    __device__ void put(int slot, bool keep, uint32_t i, uint32_t v) const {
        const uint32_t o = keep ? static_cast<uint32_t>(slot) : kDrop;
        __builtin_amdgcn_raw_buffer_store_b8(static_cast<uint8_t>(i), idx, o, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(v), val, keep ? o * 2 : kDrop, 0, 0);
    }
};

__device__ __forceinline__ DirectPayload direct_payload(uint8_t* idx, uint16_t* vals, int64_t g, int k) {
    return {__builtin_amdgcn_make_buffer_rsrc(idx + g * k, static_cast<short>(0), k, 0x00020000),
            __builtin_amdgcn_make_buffer_rsrc(vals + g * k, static_cast<short>(0), 2 * k, 0x00020000)};
}

// One group on one wave: selection, state update, payload.
template <bool HAS_E, typename RawT, typename Payload>
__device__ __forceinline__ void topk_group(RawT raw, vf2 h, int64_t g, int lane, int k, float* __restrict__ ahat,
                                           float* __restrict__ err, const Payload& pay) {
    const vf2 x = widen_pair(raw);
    const float r0 = x.x - h.x, r1 = x.y - h.y;
    const uint32_t key0 = __float_as_uint(r0) & 0x7fffffffu, key1 = __float_as_uint(r1) & 0x7fffffffu;
    // T and a copy of k are wave-uniform but kept in VGPRs (plain register moves the
    // compiler cannot fold), so candidate, the "at least k" test and the select run on
    // the vector unit and the scalar unit has only the two counts, their sum and the
    // exact-count exit.  The scalar unit serves each SIMD every fourth cycle, so this
    // split is what bounds a step.
    uint32_t T, kv;
    asm volatile("v_mov_b32 %0, 0" : "=v"(T));
    asm volatile("v_mov_b32 %0, %1" : "=v"(kv) : "s"(k));
    // Lowest set bit of the lane's two keys (31 for two zero keys; keys are below 2^31).
    const uint32_t lsb = __builtin_ctz(key0 | key1 | 0x80000000u);
    if (k < kGroup) {
#pragma unroll
        for (int b = 30; b >= 0; --b) {
            // Once no key has a set bit at or below b, every key is a multiple of
            // 2^(b+1) and T, decided down to bit b+1, is the k-th largest key itself:
            // no later candidate can gain a bit.  Groups that tie at the k-th magnitude
            // (residuals on a coarse grid) end here instead of running every bit.
            if (b <= 19 && (b & 3) == 3 && __ballot(lsb <= static_cast<uint32_t>(b)) == 0) break;
            const uint32_t cand = T | (1u << b);
            const int cnt = __popcll(__ballot(key0 >= cand)) + __popcll(__ballot(key1 >= cand));
            if (cnt >= static_cast<int>(kv)) T = cand;
            if (cnt == k) break;  // exactly the keys >= T are kept
        }
    }
    bool sel0 = key0 >= T, sel1 = key1 >= T;
    const uint64_t ge0 = __ballot(sel0), ge1 = __ballot(sel1);
    int slot0;
    if (__popcll(ge0) + __popcll(ge1) == k) {
        // Exactly the keys >= T are kept (most groups end the search this way).
        slot0 = count_below(ge0, count_below(ge1, 0));
    } else {
        // Ties at T: the keys above T, then the lowest-indexed keys equal to T.
        const int above = __popcll(__ballot(key0 > T)) + __popcll(__ballot(key1 > T));
        const int need = k - above;
        const bool eq0 = key0 == T, eq1 = key1 == T;
        const int eq_before = count_below(__ballot(eq0), count_below(__ballot(eq1), 0));
        sel0 = key0 > T || (eq0 && eq_before < need);
        sel1 = key1 > T || (eq1 && eq_before + (eq0 ? 1 : 0) < need);
        slot0 = count_below(__ballot(sel0), count_below(__ballot(sel1), 0));
    }
    const int slot1 = slot0 + (sel0 ? 1 : 0);
    const uint32_t v0 = bf16_rne(r0), v1 = bf16_rne(r1);
    const float hn0 = sel0 ? h.x + bf16_widen(v0) : h.x;
    const float hn1 = sel1 ? h.y + bf16_widen(v1) : h.y;
    // the group's 512-byte runs of state (g is the same in every lane)
    st_stream_run8(ahat + g * kGroup, vf2{hn0, hn1});
    if constexpr (HAS_E) st_stream_run8(err + g * kGroup, vf2{x.x - hn0, x.y - hn1});
    pay.put(slot0, sel0, lane * 2, v0);
    pay.put(slot1, sel1, lane * 2 + 1, v1);
}

// Block order: runs of 64 waves (256 groups, 128 KB of fp32 state) per XCD
// (run_order_block, cf_vec.h).  On a FLUX step the sender with e and the receiver ran
// 5% faster than in plain order (0.81 against 0.86 ms, 0.46 against 0.49 ms) and the
// sender without e 1% faster; runs of 16 or 32 waves were slower than plain order, and
// 128 waves in between.
constexpr uint32_t kTopkRunWaves = 64;

template <typename ActT, bool STAGED, bool HAS_E, int BLOCK = kBlock>
__global__ __launch_bounds__(BLOCK) void k_topk_compress(const ActT* __restrict__ a, float* __restrict__ ahat,
                                                          float* __restrict__ err, uint8_t* __restrict__ idx,
                                                          uint16_t* __restrict__ vals, int k, int64_t ngroups) {
    using RawT = decltype(load_pair(a, 0));
    constexpr int kWaves = BLOCK / 64;
    __shared__ uint32_t sidx[STAGED ? kWaves : 1][kPerWave * kGroup / 4];
    __shared__ uint32_t sval[STAGED ? kWaves : 1][kPerWave * kGroup / 2];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int64_t g0 =
        (static_cast<int64_t>(run_order_block<kTopkRunWaves / kWaves>()) * kWaves + wave) * kPerWave;
    if (g0 >= ngroups) return;
    if (g0 + kPerWave > ngroups) {  // ragged tail of the last wave
        for (int64_t g = g0; g < ngroups; ++g) {
            const int64_t off = g * kGroup + lane * 2;
            topk_group<HAS_E>(load_pair(a, off), __builtin_nontemporal_load(reinterpret_cast<const vf2*>(ahat + off)), g,
                       lane, k, ahat, err, direct_payload(idx, vals, g, k));
        }
        return;
    }
    RawT xr[kPerWave];
    vf2 hr[kPerWave];
#pragma unroll
    for (int j = 0; j < kLead; ++j) {
        const int64_t off = (g0 + j) * kGroup + lane * 2;
        xr[j] = load_pair(a, off);
        hr[j] = __builtin_nontemporal_load(reinterpret_cast<const vf2*>(ahat + off));
    }
#pragma unroll
    for (int j = 0; j < kPerWave; ++j) {
        if (j + kLead < kPerWave) {
            const int64_t off = (g0 + j + kLead) * kGroup + lane * 2;
            xr[j + kLead] = load_pair(a, off);
            hr[j + kLead] = __builtin_nontemporal_load(reinterpret_cast<const vf2*>(ahat + off));
        }
        if constexpr (STAGED) {
            const StagedPayload pay{reinterpret_cast<uint8_t*>(sidx[wave]) + j * k,
                                    reinterpret_cast<uint16_t*>(sval[wave]) + j * k};
            topk_group<HAS_E>(xr[j], hr[j], g0 + j, lane, k, ahat, err, pay);
        } else {
            topk_group<HAS_E>(xr[j], hr[j], g0 + j, lane, k, ahat, err, direct_payload(idx, vals, g0 + j, k));
        }
    }
    if constexpr (STAGED) {
        // LDS traffic of one wave is processed in order; the fences keep the compiler from
        // moving the reads of other lanes' slots above the writes.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // kPerWave*k index bytes at idx + g0*k and as many values at vals + g0*k, both
        // dword aligned (g0 is a multiple of 4 and the launcher checked the pointers)
        uint32_t* gi = reinterpret_cast<uint32_t*>(idx + g0 * k);
        uint32_t* gv = reinterpret_cast<uint32_t*>(vals + g0 * k);
        const int nwi = kPerWave * k / 4, nwv = kPerWave * k / 2;
        for (int i = lane; i < nwi; i += 64) gi[i] = sidx[wave][i];
        for (int i = lane; i < nwv; i += 64) gv[i] = sval[wave][i];
    }
}

// Receiver: ahat[g*128 + (idx & 127)] += widened value, as one dense pass.  A wave
// owns a group (lane l: elements 2l, 2l+1) and takes kPerWave of them; it reads the
// reconstruction once and writes it once, with non-temporal accesses.  The payload
// of a group (at most 128 slots) is read by lanes slot and slot + 64 through buffer
// loads (slots >= k are out of range and read as 0 without touching memory) and
// scattered into a per-wave LDS table of 128 words, tagged with the group's position
// in the wave so that the table never needs clearing; each lane then reads its two
// elements' words and adds the value where the tag matches.  Scattered 4-byte updates
// would touch most 64-byte sectors of a group anyway and leave them partly written.
template <int BLOCK = kBlock>
__global__ __launch_bounds__(BLOCK) void k_topk_decompress(const uint8_t* __restrict__ idx,
                                                            const uint16_t* __restrict__ vals,
                                                            float* __restrict__ ahat, int k, int64_t ngroups) {
    constexpr int kWaves = BLOCK / 64;
    __shared__ uint32_t table[kWaves][kGroup];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int64_t g0 =
        (static_cast<int64_t>(run_order_block<kTopkRunWaves / kWaves>()) * kWaves + wave) * kPerWave;
    if (g0 >= ngroups) return;
    table[wave][lane] = 0;
    table[wave][lane + 64] = 0;
    vf2 h[kPerWave];
    uint32_t slot_idx[kPerWave][2], slot_val[kPerWave][2];
#pragma unroll
    for (int j = 0; j < kPerWave; ++j) {
        const int64_t g = g0 + j < ngroups ? g0 + j : ngroups - 1;  // the tail re-reads the last group
        h[j] = __builtin_nontemporal_load(reinterpret_cast<const vf2*>(ahat + g * kGroup + lane * 2));
        const auto ri = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(idx + g * k), static_cast<short>(0),
                                                          k, 0x00020000);
        const auto rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vals + g * k),
                                                          static_cast<short>(0), 2 * k, 0x00020000);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            slot_idx[j][s] = __builtin_amdgcn_raw_buffer_load_b8(ri, lane + 64 * s, 0, 0);
            slot_val[j][s] = __builtin_amdgcn_raw_buffer_load_b16(rv, (lane + 64 * s) * 2, 0, 0);
        }
    }
#pragma unroll
    for (int j = 0; j < kPerWave; ++j) {
        const uint32_t tag = static_cast<uint32_t>(j + 1) << 16;
#pragma unroll
        for (int s = 0; s < 2; ++s)
            if (lane + 64 * s < k) table[wave][slot_idx[j][s] & 127] = tag | slot_val[j][s];
        // one wave's LDS traffic is processed in order; the fences only keep the compiler
        // from moving these reads above the other lanes' writes
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const uint32_t w0 = table[wave][lane * 2], w1 = table[wave][lane * 2 + 1];
        const float hn0 = (w0 & 0xffff0000u) == tag ? h[j].x + bf16_widen(w0 & 0xffffu) : h[j].x;
        const float hn1 = (w1 & 0xffff0000u) == tag ? h[j].y + bf16_widen(w1 & 0xffffu) : h[j].y;
        if (g0 + j < ngroups) st_stream_run8(ahat + (g0 + j) * kGroup, vf2{hn0, hn1});
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

template <typename ActT>
hipError_t run_topk(const ActT* a, float* ahat, float* err, uint8_t* idx, uint16_t* vals, int k, int64_t ngroups,
                    hipStream_t stream) {
    void* args[] = {&a, &ahat, &err, &idx, &vals, &k, &ngroups};
    const int64_t waves = (ngroups + kPerWave - 1) / kPerWave;
    const int64_t blocks = (waves + kBlock / 64 - 1) / (kBlock / 64);
    const bool staged = ((reinterpret_cast<uintptr_t>(idx) | reinterpret_cast<uintptr_t>(vals)) & 3u) == 0;
    const void* fn;
    if (err)
        fn = staged ? reinterpret_cast<const void*>(&k_topk_compress<ActT, true, true>)
                    : reinterpret_cast<const void*>(&k_topk_compress<ActT, false, true>);
    else
        fn = staged ? reinterpret_cast<const void*>(&k_topk_compress<ActT, true, false>)
                    : reinterpret_cast<const void*>(&k_topk_compress<ActT, false, false>);
    return hipLaunchKernel(fn, dim3(static_cast<unsigned>(blocks)), dim3(kBlock), args, 0, stream);
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
    const int64_t waves = (ng + kPerWave - 1) / kPerWave;
    const int64_t blocks = (waves + kBlock / 64 - 1) / (kBlock / 64);
    return hipLaunchKernel(reinterpret_cast<const void*>(&k_topk_decompress<kBlock>), dim3(static_cast<unsigned>(blocks)),
                           dim3(kBlock), args, 0, stream);
}

}  // namespace cf
