// ckda_sync.h -- workgroup synchronisation, register-pressure guards and
// wavefront row scans shared by the chunked kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ckda {

// keep the scheduler from hoisting work across this point
#define CKDA_FENCE() __builtin_amdgcn_sched_barrier(0)

// A zero the compiler cannot see through.  Adding it to a base pointer at
// the start of a phase keeps loop-invariant address arithmetic inside the
// loop instead of hoisting it into long-lived registers.
__device__ __forceinline__ int opaque_zero() {
    int z = 0;
    asm volatile("" : "+s"(z));
    return z;
}
// The thread index through the same kind of barrier: lane-derived offsets
// are recomputed where they are used.
__device__ __forceinline__ int opaque_tid() {
    int t = static_cast<int>(threadIdx.x);
    asm volatile("" : "+v"(t));
    return t;
}

// Workgroup barrier that orders LDS only: waits for this wave's LDS traffic,
// not for global loads still in flight (prefetches) or global stores.
__device__ __forceinline__ void lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Value of lane (n - D) of the same 16-lane DPP row, 0 for n < D.
template <int D>
__device__ __forceinline__ float row_shr(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 | D, 0xF, 0xF, true));
}
template <int D>
__device__ __forceinline__ uint32_t row_shr_u(uint32_t x) {
    return static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x110 | D, 0xF, 0xF, true));
}
// inclusive prefix sum over the 16 lanes of each DPP row (lane n gets the
// sum of lanes 0..n of its row)
__device__ __forceinline__ float row_scan_add(float x) {
    x += row_shr<1>(x);
    x += row_shr<2>(x);
    x += row_shr<4>(x);
    x += row_shr<8>(x);
    return x;
}
// the same with exclusive-or
__device__ __forceinline__ uint32_t row_scan_xor(uint32_t x) {
    x ^= row_shr_u<1>(x);
    x ^= row_shr_u<2>(x);
    x ^= row_shr_u<4>(x);
    x ^= row_shr_u<8>(x);
    return x;
}

}  // namespace ckda
