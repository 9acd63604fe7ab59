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

// Cross-workgroup hand-off without cache maintenance.  A workgroup that
// publishes partial results writes them with device-scope relaxed atomic
// stores (coherent writes that go through to the device's coherence point
// rather than staying in one XCD's L2), calls published_wait() so they have
// completed, and only then bumps an arrival counter; the last arrival reads
// the partials with device-scope relaxed atomic loads (coherent reads).
// A release/acquire fence pair at device scope would also be correct, but
// it writes back and invalidates the whole L2 of the XCD each time, which
// every other workgroup on that XCD pays for.
__device__ __forceinline__ void published_wait() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <typename T>
__device__ __forceinline__ void publish(T *p, T v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename T>
__device__ __forceinline__ T fetch_published(const T *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ unsigned arrive(unsigned *counter) {
    return __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace dfp
