// Internal launchers of libcf (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace cf {

// Groups of 128 contiguous elements are the unit of every 1/2-bit kernel.
constexpr int kGroup = 128;

hipError_t launch_init(int a_dtype, const void* a, float* ahat, float* err, int64_t numel,
                       hipStream_t stream);
hipError_t launch_compress(int bits, int a_dtype, const void* a, float* ahat, float* err,
                           uint8_t* codes, float* scales, int64_t numel, hipStream_t stream);
hipError_t launch_decompress(int bits, const uint8_t* codes, const float* scales, float* ahat,
                             int64_t numel, hipStream_t stream);

}  // namespace cf
