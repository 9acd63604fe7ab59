// dfp_common.h -- types and small device helpers shared by the HIP kernels
// of libdfp.  Internal to the library (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dfp.h"

namespace dfp {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Status of the most recent launch on this thread, mapped to the ABI code.
inline dfp_status launch_status() {
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? DFP_OK : DFP_ERR_HIP;
}

// Sum across the 64 lanes of a wavefront (fixed butterfly order, so every
// lane ends with the same, reproducible value).
template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v += __shfl_xor(v, off, kWave);
    return v;
}

}  // namespace dfp
