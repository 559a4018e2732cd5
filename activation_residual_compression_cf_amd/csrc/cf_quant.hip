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
// wave (32 lanes) owns one whole group of 128 elements.  The group reductions (max
// of |r|; for 1-bit also the exact sum that gives the mean) run inside the half wave,
// four steps by DPP within rows of 16 lanes and one lane exchange between the two
// rows; every lane ends with the same value.  Activations and state are read, and
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

// Value held by lane (this lane ^ mask), through the LDS crossbar.
__device__ __forceinline__ float xor_lane(float v, int mask) { return __shfl_xor(v, mask, 64); }

// Lane moves inside a row of 16 lanes by DPP, an operand modifier of the VALU: no LDS
// traffic and a few cycles of latency, against a ds_bpermute round trip.  Reduction
// partners: quad_perm [1,0,3,2] (lane ^ 1), quad_perm [2,3,0,1] (lane ^ 2),
// row_half_mirror (lane i of 8 with lane 7 - i, in the other quad) and row_mirror
// (lane i of 16 with lane 15 - i, in the other half row); after those four steps every
// lane of a row has combined all 16.  row_shl:d gives lane i the value of lane i + d of
// its row; a lane whose source lies past the row's end keeps its own value.
enum : int {
    kDppXor1 = 0xB1,
    kDppXor2 = 0x4E,
    kDppHalfMirror = 0x141,
    kDppMirror = 0x140,
    kDppShl1 = 0x101,
    kDppShl2 = 0x102,
    kDppShl4 = 0x104,
};

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
    return static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __uint_as_float(dpp<CTRL>(__float_as_uint(v)));
}
template <int CTRL>
__device__ __forceinline__ double dpp(double v) {
    const uint64_t u = static_cast<uint64_t>(__double_as_longlong(v));
    const uint64_t lo = dpp<CTRL>(static_cast<uint32_t>(u)), hi = dpp<CTRL>(static_cast<uint32_t>(u >> 32));
    return __longlong_as_double(static_cast<long long>((hi << 32) | lo));
}

// max over the 32 lanes of a half wave, the same value in each of them (max is exact,
// so the order of the steps does not matter)
__device__ __forceinline__ float half_wave_max(float M) {
    M = fmaxf(M, dpp<kDppXor1>(M));
    M = fmaxf(M, dpp<kDppXor2>(M));
    M = fmaxf(M, dpp<kDppHalfMirror>(M));
    M = fmaxf(M, dpp<kDppMirror>(M));
    return fmaxf(M, xor_lane(M, 16));
}

// ---------------------------------------------------------------------------------
// 1-bit group scale: the mean of |r| over the half wave's group of 128, taken exactly
// and rounded once to fp32 (to nearest, ties to even).  That value is unique, so no
// summation order is involved.
//
// Fast path.  With M = max|r| in [2^p, 2^(p+1)), every |r_i| is cut down to a whole
// multiple of u = 2^(p-43) (y_i = |r_i| / u < 2^44, f_i = floor(y_i)).  The f_i are
// integers and their sum stays below 2^51, so it is exact in fp64 in any order, and
// V = u * sum(f_i) / 128 is exact as well.  The exact mean lies in [V, V + u/128).
// When no |r_i| lost bits to the cut, the mean is V and its fp32 rounding is final.
// Otherwise fp32(V) is final when fp32(V + u/128) equals it: rounding is monotone.
// Only when the cut bits could move the rounding across a boundary (never seen on
// activation residuals; it takes terms below 2^-43 of the group's largest and a sum
// within 2^-50 of it from a rounding boundary) does the exact slow path run.

// Adds |x| (any fp32 bit pattern, taken as a whole number of units of 2^-149) to
// the 288-bit integer held in w[0..8], least significant word first.
__device__ __forceinline__ void add_units(uint32_t (&w)[9], float x) {
    const uint32_t u = __float_as_uint(x) & 0x7FFFFFFFu;
    const uint32_t e = u >> 23;
    const uint64_t m = e ? ((u & 0x7FFFFFu) | 0x800000u) : (u & 0x7FFFFFu);
    const uint32_t sh = e ? e - 1 : 0;  // |x| = m * 2^(sh - 149), sh <= 254
    const uint64_t v = m << (sh & 31);  // below 2^55: words sh/32 and sh/32 + 1
    const uint32_t at = sh >> 5, lo = static_cast<uint32_t>(v), hi = static_cast<uint32_t>(v >> 32);
    uint64_t c = 0;
#pragma unroll
    for (uint32_t k = 0; k < 9; ++k) {
        const uint32_t add = k == at ? lo : (k == at + 1 ? hi : 0u);
        c += static_cast<uint64_t>(w[k]) + add;
        w[k] = static_cast<uint32_t>(c);
        c >>= 32;
    }
}

__device__ __forceinline__ uint32_t word_at(const uint32_t (&w)[9], int k) {
    uint32_t out = 0;
#pragma unroll
    for (int j = 0; j < 9; ++j) out = j == k ? w[j] : out;
    return out;
}

// Slow path: the exact sum of the group's |r| as a 288-bit integer in units of
// 2^-149 (each lane adds its four, then an xor butterfly adds the half wave's
// lanes with carries), then N * 2^-156 rounded to fp32 by hand.  Every lane of the
// half wave must take part; all of them return the same value.
__device__ __noinline__ float group_mean_abs_exact(float x0, float x1, float x2, float x3) {
    uint32_t w[9] = {0, 0, 0, 0, 0, 0, 0, 0, 0};
    add_units(w, x0);
    add_units(w, x1);
    add_units(w, x2);
    add_units(w, x3);
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) {
        uint32_t other[9];
#pragma unroll
        for (int k = 0; k < 9; ++k) other[k] = static_cast<uint32_t>(__shfl_xor(static_cast<int>(w[k]), o, 64));
        uint64_t c = 0;
#pragma unroll
        for (int k = 0; k < 9; ++k) {
            c += static_cast<uint64_t>(w[k]) + other[k];
            w[k] = static_cast<uint32_t>(c);
            c >>= 32;
        }
    }
    int top = -1;  // highest set bit
#pragma unroll
    for (int k = 8; k >= 0; --k)
        if (top < 0 && w[k] != 0) top = 32 * k + 31 - __clz(static_cast<int>(w[k]));
    if (top < 0) return 0.0f;
    // keep 24 significant bits, or fewer when the mean is subnormal (its last bit,
    // 2^-149, is bit 7 of N)
    const int low = top - 23 > 7 ? top - 23 : 7;
    const uint64_t win = static_cast<uint64_t>(word_at(w, low >> 5)) |
                         (static_cast<uint64_t>(word_at(w, (low >> 5) + 1)) << 32);
    uint32_t q = static_cast<uint32_t>(win >> (low & 31));  // bits low..top; higher bits are 0
    const int hb = low - 1;                                  // the half-unit bit, >= 6
    const uint32_t half = (word_at(w, hb >> 5) >> (hb & 31)) & 1u;
    uint32_t rest = word_at(w, hb >> 5) & ((1u << (hb & 31)) - 1u);
#pragma unroll
    for (int k = 0; k < 9; ++k) rest |= k < (hb >> 5) ? w[k] : 0u;
    if (half && (rest || (q & 1u))) q += 1u;  // to nearest, ties to even
    return ldexpf(static_cast<float>(q), low - 156);
}

// The half wave's group of 128 |r| (four per lane): its exact mean rounded once to
// fp32, the same value in every lane of the half wave.
__device__ __forceinline__ float group_mean_abs(const vf4 r, int lane) {
    const float x0 = fabsf(r.x), x1 = fabsf(r.y), x2 = fabsf(r.z), x3 = fabsf(r.w);
    const float M = half_wave_max(fmaxf(fmaxf(x0, x1), fmaxf(x2, x3)));
    const int p = __builtin_amdgcn_frexp_expf(M) - 1;  // M in [2^p, 2^(p+1)); M = 0 gives p = -1
    const double y0 = ldexp(static_cast<double>(x0), 43 - p), y1 = ldexp(static_cast<double>(x1), 43 - p);
    const double y2 = ldexp(static_cast<double>(x2), 43 - p), y3 = ldexp(static_cast<double>(x3), 43 - p);
    const double f0 = floor(y0), f1 = floor(y1), f2 = floor(y2), f3 = floor(y3);
    const bool cut = (f0 != y0) | (f1 != y1) | (f2 != y2) | (f3 != y3);
    // whole numbers below 2^53: every sum is exact, in any order
    double L = (f0 + f1) + (f2 + f3);
    L = L + dpp<kDppXor1>(L);
    L = L + dpp<kDppXor2>(L);
    L = L + dpp<kDppHalfMirror>(L);
    L = L + dpp<kDppMirror>(L);
    L = L + __shfl_xor(L, 16, 64);
    const double V = ldexp(L, p - 50);
    float s = static_cast<float>(V);
    const uint64_t cuts = __ballot(cut);
    const uint32_t mine = (lane & 32) ? static_cast<uint32_t>(cuts >> 32) : static_cast<uint32_t>(cuts);
    if (mine != 0u) {  // the same branch in every lane of the half wave
        if (static_cast<float>(V + ldexp(1.0, p - 50)) != s) s = group_mean_abs_exact(x0, x1, x2, x3);
    }
    return s;
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

    // the tile's first element, and stream resources over its 256*IPS elements of state
    const int64_t t0 = wave_uniform(tile) * (2 * IPS) * kGroup;
    const __amdgpu_buffer_rsrc_t rs_h = stream_rsrc(ahat + t0, 2 * IPS * kGroup * 4);
    const __amdgpu_buffer_rsrc_t rs_e = stream_rsrc(err ? err + t0 : nullptr, 2 * IPS * kGroup * 4);
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
            s = group_mean_abs(r, lane);
            code = (r.x < 0.0f ? 1u : 0u) | (r.y < 0.0f ? 2u : 0u) | (r.z < 0.0f ? 4u : 0u) |
                   (r.w < 0.0f ? 8u : 0u);
        } else {
            const float M = half_wave_max(fmaxf(fmaxf(fabsf(r.x), fabsf(r.y)), fmaxf(fabsf(r.z), fabsf(r.w))));
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
        // per dword), 2-bit lanes a byte (4 lanes per dword).  The lanes that store a
        // dword (every 8th or 4th) read only lanes of their own row of 16.
        uint32_t w;
        if constexpr (BITS == 1) {
            w = code | (dpp<kDppShl1>(code) << 4);
            w = w | (dpp<kDppShl2>(w) << 8);
            w = w | (dpp<kDppShl4>(w) << 16);
        } else {
            w = code | (dpp<kDppShl1>(code) << 8);
            w = w | (dpp<kDppShl2>(w) << 16);
        }

        if (ok[k]) {
            const uint32_t boff = static_cast<uint32_t>(gi[k] * kGroup + hl * 4 - t0) * 4u;  // within the tile
            st_stream(rs_h, boff, hn);
            if constexpr (MODE == kEF) {
                if (err) st_stream(rs_e, boff, e);  // the error buffer is optional (wave-uniform test)
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
            const int64_t run = wave_uniform((g0 - (lane >> 5) + 2 * k) * kGroup);  // the two groups' first element
            st_stream_run(ahat + run, hn);
            if constexpr (OUT16) st_stream_run8(out + run, to_bf16x4(hn));
        }
    }
}

// Warmup: ahat = a (widened), err = 0 when err is given.  4 elements per thread.
template <typename ActT, int BLOCK = 256>
__global__ __launch_bounds__(BLOCK) void k_init(const ActT* __restrict__ a, float* __restrict__ ahat,
                                                 float* __restrict__ err, int64_t nquads) {
    const int64_t q = static_cast<int64_t>(blockIdx.x) * BLOCK + threadIdx.x;
    if (q >= nquads) return;
    // the wave's first element (its quads are consecutive), in scalar registers
    const int64_t w0 = wave_uniform((q - (threadIdx.x & 63)) * 4);
    const vf4 x = load_act4(a, q * 4);
    if ((static_cast<int64_t>(blockIdx.x) * BLOCK + (threadIdx.x & ~63u) + 64) <= nquads) {
        st_stream_run(ahat + w0, x);
        if (err) st_stream_run(err + w0, vf4{0.f, 0.f, 0.f, 0.f});
    } else {  // the wave at the end of a ragged tail
        st_nt(ahat + q * 4, x);
        if (err) st_nt(err + q * 4, vf4{0.f, 0.f, 0.f, 0.f});
    }
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
