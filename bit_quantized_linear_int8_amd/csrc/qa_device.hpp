// qa_device.hpp -- device helpers shared by the gfx950 kernels of libqa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define QA_WAVE 64

namespace qa {

// fp16 bit pattern -> fp32 (exact widening).
__device__ __forceinline__ float h2f(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

// fp32 -> fp16 bits, round to nearest even (v_cvt_f16_f32).
__device__ __forceinline__ uint16_t f2h(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint16_t f2bf(float f) {
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Maximum over the 64 lanes of a wave (every lane receives it).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        v = fmaxf(v, __shfl_xor(v, o, QA_WAVE));
    return v;
}

// Maximum over aligned groups of `width` lanes (width a power of two <= 64).
__device__ __forceinline__ float group_max(float v, int width) {
    for (int o = width >> 1; o >= 1; o >>= 1)
        v = fmaxf(v, __shfl_xor(v, o, QA_WAVE));
    return v;
}

// Quantize one value whose quotient by the scale is bounded by q_max(1+2^-23)
// (dynamic absmax scales): the quotient is formed with the reciprocal r and
// the exact IEEE division is used only when that product lies within 2^-14
// of a rounding boundary (n + 1/2).  Away from a boundary both roundings agree:
// |x*r - x/s| <= |x/s| * 2^-23 (1 + 2^-25) < 1.6e-5 for |x/s| < 128 and
// fl(x/s) is within 2^-18 of x/s, so no half-integer separates them.
__device__ __forceinline__ float quot_rne(float x, float s, float r) {
    float t = x * r;
    float n = __builtin_rintf(t);
    float d = 0.5f - __builtin_fabsf(t - n);
    if (d < 0x1p-14f)
        n = __builtin_rintf(x / s);
    return n;
}

__device__ __forceinline__ int clampi(int v, int lo, int hi) {
    return v < lo ? lo : (v > hi ? hi : v);
}

}  // namespace qa
