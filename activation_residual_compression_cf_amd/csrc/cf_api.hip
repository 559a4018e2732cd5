// cf_api.hip - the C ABI of libcf: argument validation and kernel launch.
//
// Every entry point validates all arguments before it enqueues anything, so a
// call that fails leaves every buffer untouched.  Validation order: unsupported
// mode (CF_E_ARG), NULL pointers, sizes, alignment, overlapping ranges, device.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <mutex>

#include "cf.h"
#include "cf_internal.h"

namespace {

// Largest numel of one call.  The element-wise kernels launch up to one work-item per
// 4 elements (rounded up to whole workgroups), and a dispatch counts at most
// 2^32 - 1 work-items, so 2^33 keeps every grid well inside a dispatch (and every
// byte size far from overflow).
constexpr int64_t kMaxNumel = int64_t(1) << 33;

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void* p, int64_t bytes) {
    const auto lo = reinterpret_cast<uintptr_t>(p);
    return {lo, lo + static_cast<uintptr_t>(bytes)};
}

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
// Scales are read and written one float per group: 4-byte alignment suffices, and a
// tensor inside a slab starts its scales at a multiple of 4 bytes only.
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Output range `out` must not overlap any other range in `all` (by index).
template <int N>
bool any_alias(const Range (&all)[N], const bool (&is_out)[N]) {
    for (int i = 0; i < N; ++i) {
        if (!is_out[i]) continue;
        for (int j = 0; j < N; ++j)
            if (j != i && all[j].hi > all[j].lo && overlap(all[i], all[j])) return true;
    }
    return false;
}

// Device check: the current device must be gfx950.  Cached per device id.
constexpr int kMaxDevices = 64;
std::once_flag g_dev_once[kMaxDevices];
bool g_dev_ok[kMaxDevices];

int check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CF_E_DEVICE;
    std::call_once(g_dev_once[dev], [dev] {
        hipDeviceProp_t prop;
        g_dev_ok[dev] = hipGetDeviceProperties(&prop, dev) == hipSuccess &&
                        std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    });
    return g_dev_ok[dev] ? CF_OK : CF_E_DEVICE;
}

// Fixed scratch of cf_lowrank_compress_noalloc: one copy in every device's memory that
// the library's code object is loaded on, for the life of the process.  Host code must
// not use the array's name as an address (it names a host-side stand-in); it takes the
// device address from hipGetSymbolAddress, once per device, with that device current.
static __device__ __align__(256) unsigned char scratch[CF_NOALLOC_SCRATCH_BYTES];

std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch, or nullptr when HIP refuses it.
void* scratch_for_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::call_once(g_scratch_once[dev], [dev] {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) == hipSuccess) g_scratch_ptr[dev] = ptr;
    });
    return g_scratch_ptr[dev];
}

int valid_numel(int64_t numel) {
    return (numel > 0 && numel % CF_GROUP == 0 && numel <= kMaxNumel) ? CF_OK : CF_E_SHAPE;
}

int64_t act_bytes(int a_dtype, int64_t numel) { return numel * (a_dtype == CF_BF16 ? 2 : 4); }

// Checks of cf_lowrank_compress, in the order of the file header: a workspace of
// `ws_bytes` at `workspace` (null for a buffer of the library's own, which then needs no
// NULL or overlap check), `too_small` the status when the call needs more than ws_bytes.
int check_lowrank_compress(int a_dtype, const void* a, float* ahat, float* err, int64_t m, int64_t n, int rank,
                           int iters, int factor_bits, int batch, float* q_state, void* u, float* u_scales,
                           void* v, float* v_scales, const void* workspace, size_t ws_bytes, int too_small) {
    if (a_dtype != CF_BF16 && a_dtype != CF_F32) return CF_E_ARG;
    if (factor_bits != 4 && factor_bits != 16 && factor_bits != 32) return CF_E_ARG;
    if (iters < 1 || iters > 64) return CF_E_ARG;
    if (!a || !ahat || !q_state || !u || !v || (!workspace && too_small == CF_E_WORKSPACE)) return CF_E_NULL;
    if (factor_bits == 4 && (!u_scales || !v_scales)) return CF_E_NULL;
    const size_t need = cf_lowrank_workspace_bytes(m, n, rank, batch);
    if (need == 0 || (factor_bits == 4 && (rank & 1))) return CF_E_SHAPE;
    if (!aligned16(a) || !aligned16(ahat) || (err && !aligned16(err)) || !aligned4(q_state) ||
        !aligned4(u) || !aligned4(v) || (u_scales && !aligned4(u_scales)) ||
        (v_scales && !aligned4(v_scales)) || (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return CF_E_ALIGN;
    if (ws_bytes < need) return too_small;
    const int64_t numel = m * n * batch;
    const int64_t fsz = factor_bits / 4;  // factor bytes per (row, rank) pair, times 2
    const Range r[8] = {range_of(a, act_bytes(a_dtype, numel)),
                        range_of(ahat, numel * 4),
                        range_of(err, err ? numel * 4 : 0),
                        range_of(q_state, int64_t(batch) * n * rank * 4),
                        range_of(u, int64_t(batch) * m * rank * fsz / 2),
                        range_of(v, int64_t(batch) * n * rank * fsz / 2),
                        range_of(u_scales, factor_bits == 4 ? int64_t(batch) * rank * 4 : 0),
                        range_of(v_scales, factor_bits == 4 ? int64_t(batch) * rank * 4 : 0)};
    const bool out[8] = {false, true, err != nullptr, true, true, true, factor_bits == 4, factor_bits == 4};
    if (any_alias(r, out)) return CF_E_ALIAS;
    if (workspace) {
        const Range wsr = range_of(workspace, static_cast<int64_t>(need));
        for (const Range& x : r)
            if (x.hi > x.lo && overlap(x, wsr)) return CF_E_ALIAS;
    }
    return CF_OK;
}

}  // namespace

extern "C" {

int cf_abi_version(void) { return 1; }

const char* cf_strerror(int status) {
    switch (status) {
        case CF_OK: return "ok";
        case CF_E_NULL: return "required pointer is NULL";
        case CF_E_SHAPE: return "size out of range (numel must be a positive multiple of 128, at most 2^33)";
        case CF_E_ALIGN: return "pointer misaligned (16 bytes; scales 4 bytes)";
        case CF_E_ARG: return "unsupported bits, k, dtype or mode";
        case CF_E_ALIAS: return "output range overlaps another operand";
        case CF_E_WORKSPACE: return "workspace missing or too small";
        case CF_E_DEVICE: return "current device is not gfx950";
        case CF_E_HIP: return "HIP runtime refused the launch";
        case CF_E_SCRATCH:
            return "call needs more scratch than cf_lowrank_compress_noalloc's fixed buffer "
                   "(CF_NOALLOC_SCRATCH_BYTES) holds; pass fewer tensors per call";
        default: return "unknown status";
    }
}

int64_t cf_codes_bytes(int64_t numel, int bits) {
    if (bits != 1 && bits != 2) return CF_E_ARG;
    if (valid_numel(numel) != CF_OK) return CF_E_SHAPE;
    return numel * bits / 8;
}

int cf_init_state(int a_dtype, const void* a, float* ahat, float* err, int64_t numel, void* stream) {
    if (a_dtype != CF_BF16 && a_dtype != CF_F32) return CF_E_ARG;
    if (!a || !ahat) return CF_E_NULL;
    if (int rc = valid_numel(numel)) return rc;
    if (!aligned16(a) || !aligned16(ahat) || (err && !aligned16(err))) return CF_E_ALIGN;
    const Range r[3] = {range_of(a, act_bytes(a_dtype, numel)), range_of(ahat, numel * 4),
                        range_of(err, err ? numel * 4 : 0)};
    const bool out[3] = {false, true, err != nullptr};
    if (any_alias(r, out)) return CF_E_ALIAS;
    if (int rc = check_device()) return rc;
    return cf::launch_init(a_dtype, a, ahat, err, numel, static_cast<hipStream_t>(stream)) == hipSuccess
               ? CF_OK
               : CF_E_HIP;
}

int cf_compress(int bits, int a_dtype, const void* a, float* ahat, float* err, uint8_t* codes,
                float* scales, int64_t numel, void* stream) {
    if ((bits != 1 && bits != 2) || (a_dtype != CF_BF16 && a_dtype != CF_F32)) return CF_E_ARG;
    if (!a || !ahat || !codes || !scales) return CF_E_NULL;
    if (int rc = valid_numel(numel)) return rc;
    if (!aligned16(a) || !aligned16(ahat) || (err && !aligned16(err)) || !aligned16(codes) ||
        !aligned4(scales))
        return CF_E_ALIGN;
    const Range r[5] = {range_of(a, act_bytes(a_dtype, numel)), range_of(ahat, numel * 4),
                        range_of(err, err ? numel * 4 : 0), range_of(codes, numel * bits / 8),
                        range_of(scales, numel / CF_GROUP * 4)};
    const bool out[5] = {false, true, err != nullptr, true, true};
    if (any_alias(r, out)) return CF_E_ALIAS;
    if (int rc = check_device()) return rc;
    return cf::launch_compress(bits, a_dtype, a, ahat, err, codes, scales, numel,
                               static_cast<hipStream_t>(stream)) == hipSuccess
               ? CF_OK
               : CF_E_HIP;
}

int cf_decompress(int bits, const uint8_t* codes, const float* scales, float* ahat, int64_t numel,
                  void* stream) {
    if (bits != 1 && bits != 2) return CF_E_ARG;
    if (!codes || !scales || !ahat) return CF_E_NULL;
    if (int rc = valid_numel(numel)) return rc;
    if (!aligned16(codes) || !aligned4(scales) || !aligned16(ahat)) return CF_E_ALIGN;
    const Range r[3] = {range_of(codes, numel * bits / 8), range_of(scales, numel / CF_GROUP * 4),
                        range_of(ahat, numel * 4)};
    const bool out[3] = {false, false, true};
    if (any_alias(r, out)) return CF_E_ALIAS;
    if (int rc = check_device()) return rc;
    return cf::launch_decompress(bits, codes, scales, ahat, nullptr, numel, static_cast<hipStream_t>(stream)) ==
                   hipSuccess
               ? CF_OK
               : CF_E_HIP;
}

int cf_decompress_bf16(int bits, const uint8_t* codes, const float* scales, float* ahat, uint16_t* out,
                       int64_t numel, void* stream) {
    if (bits != 1 && bits != 2) return CF_E_ARG;
    if (!codes || !scales || !ahat || !out) return CF_E_NULL;
    if (int rc = valid_numel(numel)) return rc;
    if (!aligned16(codes) || !aligned4(scales) || !aligned16(ahat) || !aligned16(out)) return CF_E_ALIGN;
    const Range r[4] = {range_of(codes, numel * bits / 8), range_of(scales, numel / CF_GROUP * 4),
                        range_of(ahat, numel * 4), range_of(out, numel * 2)};
    const bool is_out[4] = {false, false, true, true};
    if (any_alias(r, is_out)) return CF_E_ALIAS;
    if (int rc = check_device()) return rc;
    return cf::launch_decompress(bits, codes, scales, ahat, out, numel, static_cast<hipStream_t>(stream)) ==
                   hipSuccess
               ? CF_OK
               : CF_E_HIP;
}

int cf_compress_ablation(int mode, int bits, int a_dtype, const void* a, const void* a_prev, float* ahat,
                         uint8_t* codes, float* scales, int64_t numel, void* stream) {
    if ((mode != CF_MODE_NOEF && mode != CF_MODE_NAIVE) || (bits != 1 && bits != 2) ||
        (a_dtype != CF_BF16 && a_dtype != CF_F32))
        return CF_E_ARG;
    if (!a || !ahat || !codes || !scales || (mode == CF_MODE_NOEF && !a_prev)) return CF_E_NULL;
    if (int rc = valid_numel(numel)) return rc;
    if (!aligned16(a) || (a_prev && !aligned16(a_prev)) || !aligned16(ahat) || !aligned16(codes) ||
        !aligned4(scales))
        return CF_E_ALIGN;
    const Range r[5] = {range_of(a, act_bytes(a_dtype, numel)),
                        range_of(a_prev, mode == CF_MODE_NOEF ? act_bytes(a_dtype, numel) : 0),
                        range_of(ahat, numel * 4), range_of(codes, numel * bits / 8),
                        range_of(scales, numel / CF_GROUP * 4)};
    const bool is_out[5] = {false, false, true, true, true};
    if (any_alias(r, is_out)) return CF_E_ALIAS;
    if (int rc = check_device()) return rc;
    return cf::launch_compress_ablation(mode, bits, a_dtype, a, a_prev, ahat, codes, scales, numel,
                                        static_cast<hipStream_t>(stream)) == hipSuccess
               ? CF_OK
               : CF_E_HIP;
}

int cf_topk_compress(int k, int a_dtype, const void* a, float* ahat, float* err, uint8_t* idx, uint16_t* vals,
                     int64_t numel, void* stream) {
    if (k < 1 || k > CF_GROUP || (a_dtype != CF_BF16 && a_dtype != CF_F32)) return CF_E_ARG;
    if (!a || !ahat || !idx || !vals) return CF_E_NULL;
    if (int rc = valid_numel(numel)) return rc;
    if (!aligned16(a) || !aligned16(ahat) || (err && !aligned16(err)) ||
        (reinterpret_cast<uintptr_t>(vals) & 1u))
        return CF_E_ALIGN;
    const int64_t slots = numel / CF_GROUP * k;
    const Range r[5] = {range_of(a, act_bytes(a_dtype, numel)), range_of(ahat, numel * 4),
                        range_of(err, err ? numel * 4 : 0), range_of(idx, slots), range_of(vals, slots * 2)};
    const bool out[5] = {false, true, err != nullptr, true, true};
    if (any_alias(r, out)) return CF_E_ALIAS;
    if (int rc = check_device()) return rc;
    return cf::launch_topk_compress(k, a_dtype, a, ahat, err, idx, vals, numel,
                                    static_cast<hipStream_t>(stream)) == hipSuccess
               ? CF_OK
               : CF_E_HIP;
}

int cf_topk_decompress(int k, const uint8_t* idx, const uint16_t* vals, float* ahat, int64_t numel,
                       void* stream) {
    if (k < 1 || k > CF_GROUP) return CF_E_ARG;
    if (!idx || !vals || !ahat) return CF_E_NULL;
    if (int rc = valid_numel(numel)) return rc;
    if (!aligned16(ahat) || (reinterpret_cast<uintptr_t>(vals) & 1u)) return CF_E_ALIGN;
    const int64_t slots = numel / CF_GROUP * k;
    const Range r[3] = {range_of(idx, slots), range_of(vals, slots * 2), range_of(ahat, numel * 4)};
    const bool out[3] = {false, false, true};
    if (any_alias(r, out)) return CF_E_ALIAS;
    if (int rc = check_device()) return rc;
    return cf::launch_topk_decompress(k, idx, vals, ahat, numel, static_cast<hipStream_t>(stream)) == hipSuccess
               ? CF_OK
               : CF_E_HIP;
}

size_t cf_lowrank_workspace_bytes(int64_t m, int64_t n, int rank, int batch) {
    if (m <= 0 || n <= 0 || m % 16 || n % 16 || batch < 1 || rank < 1 || rank > cf::kMaxRank ||
        rank > m || rank > n || m > kMaxNumel / n || m * n > kMaxNumel / batch ||
        !cf::lowrank_launches_fit(m, n, rank, batch))
        return 0;
    return cf::lowrank_workspace_total(m, n, rank, batch);
}

int cf_lowrank_compress(int a_dtype, const void* a, float* ahat, float* err, int64_t m, int64_t n,
                        int rank, int iters, int factor_bits, int batch, float* q_state, void* u,
                        float* u_scales, void* v, float* v_scales, void* workspace, size_t ws_bytes,
                        void* stream) {
    if (int rc = check_lowrank_compress(a_dtype, a, ahat, err, m, n, rank, iters, factor_bits, batch, q_state, u,
                                        u_scales, v, v_scales, workspace, ws_bytes, CF_E_WORKSPACE))
        return rc;
    if (int rc = check_device()) return rc;
    return cf::launch_lowrank_compress(a_dtype, a, ahat, err, m, n, rank, iters, factor_bits, batch,
                                       q_state, u, u_scales, v, v_scales, workspace,
                                       static_cast<hipStream_t>(stream)) == hipSuccess
               ? CF_OK
               : CF_E_HIP;
}

int cf_lowrank_compress_noalloc(int a_dtype, const void* a, float* ahat, float* err, int64_t m, int64_t n,
                                int rank, int iters, int factor_bits, int batch, float* q_state, void* u,
                                float* u_scales, void* v, float* v_scales, void* stream) {
    if (int rc = check_lowrank_compress(a_dtype, a, ahat, err, m, n, rank, iters, factor_bits, batch, q_state, u,
                                        u_scales, v, v_scales, nullptr, CF_NOALLOC_SCRATCH_BYTES, CF_E_SCRATCH))
        return rc;
    if (int rc = check_device()) return rc;
    void* ws = scratch_for_current_device();
    if (!ws) return CF_E_HIP;
    return cf::launch_lowrank_compress(a_dtype, a, ahat, err, m, n, rank, iters, factor_bits, batch, q_state,
                                       u, u_scales, v, v_scales, ws, static_cast<hipStream_t>(stream)) ==
                   hipSuccess
               ? CF_OK
               : CF_E_HIP;
}

int cf_lowrank_decompress(int factor_bits, const void* u, const float* u_scales, const void* v,
                          const float* v_scales, float* ahat, int64_t m, int64_t n, int rank,
                          int batch, void* stream) {
    if (factor_bits != 4 && factor_bits != 16 && factor_bits != 32) return CF_E_ARG;
    if (!u || !v || !ahat) return CF_E_NULL;
    if (factor_bits == 4 && (!u_scales || !v_scales)) return CF_E_NULL;
    if (cf_lowrank_workspace_bytes(m, n, rank, batch) == 0 || (factor_bits == 4 && (rank & 1)))
        return CF_E_SHAPE;
    if (!aligned16(ahat) || !aligned4(u) || !aligned4(v) || (u_scales && !aligned4(u_scales)) ||
        (v_scales && !aligned4(v_scales)))
        return CF_E_ALIGN;
    const int64_t numel = m * n * batch;
    const int64_t fsz = factor_bits / 4;
    const Range r[5] = {range_of(ahat, numel * 4),
                        range_of(u, int64_t(batch) * m * rank * fsz / 2),
                        range_of(v, int64_t(batch) * n * rank * fsz / 2),
                        range_of(u_scales, factor_bits == 4 ? int64_t(batch) * rank * 4 : 0),
                        range_of(v_scales, factor_bits == 4 ? int64_t(batch) * rank * 4 : 0)};
    const bool out[5] = {true, false, false, false, false};
    if (any_alias(r, out)) return CF_E_ALIAS;
    if (int rc = check_device()) return rc;
    return cf::launch_lowrank_decompress(factor_bits, u, u_scales, v, v_scales, ahat, m, n, rank, batch,
                                         static_cast<hipStream_t>(stream)) == hipSuccess
               ? CF_OK
               : CF_E_HIP;
}

}  // extern "C"
