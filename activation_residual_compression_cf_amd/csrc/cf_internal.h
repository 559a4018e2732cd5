// Internal launchers of libcf (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace cf {

// Groups of 128 contiguous elements are the unit of every 1/2-bit kernel.
constexpr int kGroup = 128;

// A dispatch counts its work-items per grid dimension in 32 bits.
constexpr int64_t kMaxDispatchItems = (int64_t(1) << 32) - 1;

hipError_t launch_init(int a_dtype, const void* a, float* ahat, float* err, int64_t numel,
                       hipStream_t stream);
hipError_t launch_compress(int bits, int a_dtype, const void* a, float* ahat, float* err,
                           uint8_t* codes, float* scales, int64_t numel, hipStream_t stream);
hipError_t launch_compress_ablation(int mode, int bits, int a_dtype, const void* a, const void* a_prev,
                                    float* ahat, uint8_t* codes, float* scales, int64_t numel,
                                    hipStream_t stream);
// out (bf16 bits of the updated reconstruction) may be null.
hipError_t launch_decompress(int bits, const uint8_t* codes, const float* scales, float* ahat, uint16_t* out,
                             int64_t numel, hipStream_t stream);

// Top-k sparsification of the residual: k of every 128 kept as (index byte, bf16 value).
hipError_t launch_topk_compress(int k, int a_dtype, const void* a, float* ahat, float* err, uint8_t* idx,
                                uint16_t* vals, int64_t numel, hipStream_t stream);
hipError_t launch_topk_decompress(int k, const uint8_t* idx, const uint16_t* vals, float* ahat, int64_t numel,
                                  hipStream_t stream);

// Low-rank workspace regions (carved from one caller buffer).
struct LowrankWorkspace {
    float* r;      // batch x m x n residual
    float* qt;     // batch x kp x n, Q transposed (rank padded to a multiple of 16)
    float* ypart;  // Y partials: batch x segments x m x kp of a projection, or two per strip
                   // range of a fused pass
    float* p;      // batch x m x kp orthonormal factor
    int* alive;    // batch x kp rank-guard flags
    double* gpart; // batch x row blocks x kp x kp Gram partials
    float* cmax;   // batch x row blocks x kp column maxima of the factors
    bool shared;   // one of two halves of a call, run on two streams at once
};

// Largest rank the low-rank kernels accept.
constexpr int kMaxRank = 64;

// Fills the region pointers of one launch sequence over `batch` tensors for `base` (may
// be null) and its size in *bytes; `shared`: the sequence is one of a call's two halves.
LowrankWorkspace carve_lowrank_workspace(void* base, int64_t m, int64_t n, int rank, int64_t batch, bool shared,
                                         size_t* bytes);
// Workspace bytes of a whole call (a large call runs two halves, each with its own regions).
size_t lowrank_workspace_total(int64_t m, int64_t n, int rank, int64_t batch);
// Whether every launch of one low-rank call (or of its receiver) fits a dispatch.
bool lowrank_launches_fit(int64_t m, int64_t n, int rank, int64_t batch);
hipError_t launch_lowrank_compress(int a_dtype, const void* a, float* ahat, float* err, int64_t m,
                                   int64_t n, int rank, int iters, int factor_bits, int64_t batch,
                                   float* q_state, void* u, float* u_scales, void* v, float* v_scales,
                                   void* workspace, hipStream_t stream);
hipError_t launch_lowrank_decompress(int factor_bits, const void* u, const float* u_scales,
                                     const void* v, const float* v_scales, float* ahat, int64_t m,
                                     int64_t n, int rank, int64_t batch, hipStream_t stream);

}  // namespace cf
