// Shared device/host helpers of the gfx950 kernels (no method arithmetic).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dflash.h"

namespace dflash {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kTopK = 16;

// bf16 bit pattern -> float (exact).
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// float -> bf16 bit pattern, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// Total order used by every top-k and argmax here: larger value first, then
// lower index.  Returns true when (va, ia) ranks before (vb, ib).
__device__ __forceinline__ bool ranks_before(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

__device__ __forceinline__ bool ranks_before_d(double va, int ia, double vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

// Orders the LDS accesses of one wavefront around this point.
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Kernel launch helpers (host side).
inline int launch_status() {
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? DFLASH_OK : DFLASH_ERR_LAUNCH;
}

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace dflash
