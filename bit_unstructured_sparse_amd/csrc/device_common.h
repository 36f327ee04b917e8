// device_common.h -- small device helpers shared by the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define BSP_WAVE 64

// Buffer resource over [base, base + bytes): loads at offsets >= bytes return
// zero in hardware instead of touching memory. Dword 3 is the gfx9-family
// default (untyped raw buffer, 32-bit dword format).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t bsp_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// Sign-extend the low 4 bits of v (int4 two's complement).
__device__ __forceinline__ int bsp_sext4(uint32_t v) {
    return (int)(v << 28) >> 28;
}

__device__ __forceinline__ float bsp_h2f(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

// Round-to-nearest-even fp32 -> fp16 bits.
__device__ __forceinline__ uint16_t bsp_f2h(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// Sum over the 64 lanes of a wavefront; every lane receives the total.
template <class T>
__device__ __forceinline__ T bsp_wave_sum(T v) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, BSP_WAVE);
    return v;
}
