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

constexpr int64_t kMaxNumel = int64_t(1) << 40;  // keeps every byte size far from overflow

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

int valid_numel(int64_t numel) {
    return (numel > 0 && numel % CF_GROUP == 0 && numel <= kMaxNumel) ? CF_OK : CF_E_SHAPE;
}

int64_t act_bytes(int a_dtype, int64_t numel) { return numel * (a_dtype == CF_BF16 ? 2 : 4); }

}  // namespace

extern "C" {

int cf_abi_version(void) { return 1; }

const char* cf_strerror(int status) {
    switch (status) {
        case CF_OK: return "ok";
        case CF_E_NULL: return "required pointer is NULL";
        case CF_E_SHAPE: return "size out of range (numel must be a positive multiple of 128)";
        case CF_E_ALIGN: return "pointer misaligned (16 bytes; scales 4 bytes)";
        case CF_E_ARG: return "unsupported bits, dtype or mode";
        case CF_E_ALIAS: return "output range overlaps another operand";
        case CF_E_WORKSPACE: return "workspace missing or too small";
        case CF_E_DEVICE: return "current device is not gfx950";
        case CF_E_HIP: return "HIP runtime refused the launch";
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
    if (!a || !ahat || !err || !codes || !scales) return CF_E_NULL;
    if (int rc = valid_numel(numel)) return rc;
    if (!aligned16(a) || !aligned16(ahat) || !aligned16(err) || !aligned16(codes) || !aligned4(scales))
        return CF_E_ALIGN;
    const Range r[5] = {range_of(a, act_bytes(a_dtype, numel)), range_of(ahat, numel * 4),
                        range_of(err, numel * 4), range_of(codes, numel * bits / 8),
                        range_of(scales, numel / CF_GROUP * 4)};
    const bool out[5] = {false, true, true, true, true};
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
    return cf::launch_decompress(bits, codes, scales, ahat, numel, static_cast<hipStream_t>(stream)) ==
                   hipSuccess
               ? CF_OK
               : CF_E_HIP;
}

}  // extern "C"
