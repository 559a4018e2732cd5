// Host-side memory and undefined-behaviour check of libcf's C ABI (test
// infrastructure, for a machine without a GPU).
//
// libcf's host code is compiled with AddressSanitizer and UBSan (its kernels are
// built as usual but never launched), and this driver runs every entry point's validation on
// the values where size arithmetic could overflow or pointer ranges wrap: element
// counts near 2^63, low-rank shapes whose products leave int64, ranks and batches
// at INT_MAX, buffers that end at the top of the 47-bit user address space, and
// empty ranges.
// Placeholder pointers are never dereferenced: every call either fails validation
// or stops at the device check, which fails where no gfx950 is present.  Prints
// "ok" and exits 0 when every status is the expected one.
//
// Built and run by tests/test_sanitizers.py.
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "cf.h"

namespace {

int failures = 0;

void expect(long long got, long long want, const char* what, int line) {
    if (got != want) {
        std::fprintf(stderr, "line %d: %s gave %lld, expected %lld\n", line, what, got, want);
        ++failures;
    }
}
#define EXPECT(call, want) expect((long long)(call), (long long)(want), #call, __LINE__)

void* P(uintptr_t x) { return reinterpret_cast<void*>(x); }
float* F(uintptr_t x) { return reinterpret_cast<float*>(x); }
uint8_t* B(uintptr_t x) { return reinterpret_cast<uint8_t*>(x); }
uint16_t* H(uintptr_t x) { return reinterpret_cast<uint16_t*>(x); }

constexpr int64_t kBig = INT64_MAX - 127;  // a multiple of 128 near 2^63
constexpr uintptr_t kT = uintptr_t(1) << 40;   // spacing that keeps 2^33-element buffers apart

// Start of a buffer of `bytes` that ends exactly at 2^47, the top of user space.
uintptr_t top(uint64_t bytes) { return (uintptr_t(1) << 47) - bytes; }

}  // namespace

int main() {
    EXPECT(cf_abi_version(), 1);
    for (int s = 1; s >= -9; --s) EXPECT(cf_strerror(s) != nullptr, 1);

    EXPECT(cf_codes_bytes(kBig, 2), CF_E_SHAPE);
    EXPECT(cf_codes_bytes(INT64_MIN, 1), CF_E_SHAPE);
    EXPECT(cf_codes_bytes(int64_t(1) << 33, 2), int64_t(1) << 31);

    // Quantizers: sizes near 2^63, and buffers that end at the top of user space.
    EXPECT(cf_compress(1, CF_BF16, P(0x100000), F(0x200000), F(0x300000), B(0x400000), F(0x500000),
                       kBig, nullptr),
           CF_E_SHAPE);
    EXPECT(cf_compress(2, CF_F32, P(top(4 << 20)), F(0x200000), nullptr, B(0x800000), F(0x900000),
                       1 << 20, nullptr),
           CF_E_DEVICE);
    EXPECT(cf_compress(1, CF_BF16, P(kT), F(top(uint64_t(4) << 33)), F(3 * kT), B(4 * kT), F(5 * kT),
                       int64_t(1) << 33, nullptr),
           CF_E_DEVICE);
    EXPECT(cf_init_state(CF_F32, P(top(512)), F(0x200000), nullptr, INT64_MIN, nullptr), CF_E_SHAPE);
    EXPECT(cf_init_state(CF_F32, P(top(512)), F(0x200000), F(0x300000), 128, nullptr), CF_E_DEVICE);
    EXPECT(cf_decompress(2, B(top(64)), F(0x200000), F(0x300000), kBig, nullptr), CF_E_SHAPE);
    EXPECT(cf_decompress(2, B(0x100000), F(0x200000), F(top(1 << 18)), 1 << 16, nullptr),
           CF_E_DEVICE);
    EXPECT(cf_decompress_bf16(1, B(0x100000), F(0x200000), F(0x300000), H(top(1 << 17)), 1 << 16,
                              nullptr),
           CF_E_DEVICE);
    EXPECT(cf_compress_ablation(CF_MODE_NOEF, 1, CF_BF16, P(0x100000), P(top(1 << 13)), F(0x300000),
                                B(0x400000), F(0x500000), 1 << 12, nullptr),
           CF_E_DEVICE);
    EXPECT(cf_compress_ablation(CF_MODE_NAIVE, 2, CF_F32, P(0x100000), nullptr, F(0x300000),
                                B(0x400000), F(0x500000), kBig, nullptr),
           CF_E_SHAPE);

    // Top-k: k at both ends, sizes near 2^63.
    EXPECT(cf_topk_compress(INT_MAX, CF_BF16, P(0x100000), F(0x200000), nullptr, B(0x300000),
                            H(0x400000), 128, nullptr),
           CF_E_ARG);
    EXPECT(cf_topk_compress(128, CF_BF16, P(0x100000), F(0x200000), nullptr, B(0x300000),
                            H(0x400000), kBig, nullptr),
           CF_E_SHAPE);
    EXPECT(cf_topk_compress(128, CF_F32, P(0x1000000), F(0x2000000), F(0x3000000), B(top(1 << 12)),
                            H(0x5000000), 1 << 12, nullptr),
           CF_E_DEVICE);
    EXPECT(cf_topk_decompress(INT_MIN, B(0x100000), H(0x200000), F(0x300000), 128, nullptr), CF_E_ARG);
    EXPECT(cf_topk_decompress(1, B(0x100000), H(0x200000), F(top(1 << 14)), 1 << 12, nullptr),
           CF_E_DEVICE);

    // Low-rank workspace: products of the shape that would leave int64.
    EXPECT(cf_lowrank_workspace_bytes(INT64_MAX - 15, 16, 16, 1), 0);
    EXPECT(cf_lowrank_workspace_bytes(16, INT64_MAX - 15, 16, 1), 0);
    EXPECT(cf_lowrank_workspace_bytes(int64_t(1) << 32, int64_t(1) << 32, 16, 1), 0);
    EXPECT(cf_lowrank_workspace_bytes(1024, 3072, 32, INT_MAX), 0);
    EXPECT(cf_lowrank_workspace_bytes(1024, 3072, INT_MAX, 1), 0);
    EXPECT(cf_lowrank_workspace_bytes(1024, 3072, INT_MIN, 1), 0);
    EXPECT(cf_lowrank_workspace_bytes(16, 16, 16, INT_MIN), 0);
    EXPECT(cf_lowrank_workspace_bytes(16, 1 << 28, 16, 1) > 0, 1);
    EXPECT(cf_lowrank_workspace_bytes(1 << 28, 16, 16, 1) > 0, 1);
    EXPECT(cf_lowrank_workspace_bytes(16, 16, 16, 1 << 22) > 0, 1);
    EXPECT(cf_lowrank_workspace_bytes(16, 16, 16, 1 << 23), 0);

    const size_t ws = cf_lowrank_workspace_bytes(64, 128, 8, 1);
    EXPECT(ws > 0, 1);
    EXPECT(cf_lowrank_compress(CF_BF16, P(0x100000), F(0x200000), nullptr, 64, 128, 8, INT_MAX, 4, 1,
                               F(0x400000), P(0x500000), F(0x600000), P(0x700000), F(0x800000),
                               P(0x1000000), ws, nullptr),
           CF_E_ARG);
    EXPECT(cf_lowrank_compress(CF_BF16, P(0x100000), F(0x200000), nullptr, INT64_MAX, INT64_MAX, 8, 2,
                               4, INT_MAX, F(0x400000), P(0x500000), F(0x600000), P(0x700000),
                               F(0x800000), P(0x1000000), ws, nullptr),
           CF_E_SHAPE);
    EXPECT(cf_lowrank_compress(CF_BF16, P(0x100000), F(0x200000), nullptr, 64, 128, 8, 2, 4, 1,
                               F(0x400000), P(0x500000), F(0x600000), P(0x700000), F(0x800000),
                               P(0x1000000), SIZE_MAX, nullptr),
           CF_E_DEVICE);
    EXPECT(cf_lowrank_compress(CF_F32, P(0x100000), F(0x200000), F(0x300000), 64, 128, 8, 2, 32, 1,
                               F(0x400000), P(0x500000), nullptr, P(0x700000), nullptr,
                               P(top(ws) & ~uintptr_t(255)), ws, nullptr),
           CF_E_DEVICE);
    EXPECT(cf_lowrank_decompress(16, P(0x500000), nullptr, P(0x700000), nullptr, F(top(64 * 128 * 4)),
                                 64, 128, 8, 1, nullptr),
           CF_E_DEVICE);
    EXPECT(cf_lowrank_decompress(4, P(0x500000), F(0x600000), P(0x700000), F(0x800000), F(0x200000),
                                 INT64_MIN, 128, 8, 1, nullptr),
           CF_E_SHAPE);

    if (failures) {
        std::fprintf(stderr, "%d unexpected statuses\n", failures);
        return 1;
    }
    std::printf("ok\n");
    return 0;
}
