// Device helpers shared by the kernel translation units of the library (gfx950).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace w4a8 {

typedef int v4i __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------------------------
// small device helpers
// ------------------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// binary16 bit pattern -> float32 (exact)
__device__ __forceinline__ float f16_to_f32(uint16_t bits) { return static_cast<float>(__builtin_bit_cast(_Float16, bits)); }

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;   // quiet NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// 16-byte load of weight codes that are read once per launch, marked non-temporal: the
// stream then does not evict the activations and scales that every workgroup re-reads from
// L2.  Measured on the 4096 x 14336 decode GEMM: 8.1 -> 7.5 us at 16-row tiles, 10.1 -> 9.3 us
// at 32-row tiles.
__device__ __forceinline__ uint4 stream_load(const uint8_t* p) {
    const v4i v = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(p));
    return make_uint4(uint32_t(v.x), uint32_t(v.y), uint32_t(v.z), uint32_t(v.w));
}

// Workgroup barrier for LDS hand-offs that leaves global loads in flight: wait for this
// wave's LDS (and scalar) operations only, then s_barrier.  The empty asm statements keep
// the compiler from moving memory accesses across it.  (__syncthreads would also drain
// every outstanding global load of the wave.)
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    // s_waitcnt: vmcnt 63 (no wait), expcnt 7 (no wait), lgkmcnt 0
    __builtin_amdgcn_s_waitcnt(0xF | (7 << 4) | (0 << 8) | (3 << 14));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

}  // namespace w4a8
