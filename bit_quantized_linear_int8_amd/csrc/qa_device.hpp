// qa_device.hpp -- device helpers shared by the gfx950 kernels of libqa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef __bf16 v4bf __attribute__((ext_vector_type(4)));

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

// fp32 -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32; NaN stays NaN).
__device__ __forceinline__ uint16_t f2bf(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
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

// ---------------------------------------------------------------------------
// Buffer loads.  A buffer resource descriptor carries a base address and a
// byte range; raw buffer loads outside the range return zeros, so bounds are
// checked by the hardware and loads never need a branch (a branch around a
// load makes the compiler wait for it inside the branch).
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr uint32_t kOOB = 0x80000000u;        // an offset past every range used here

// Descriptor for [base, base + bytes), bytes clamped to 2^31 - 1.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
    const int n = bytes <= 0 ? 0 : (bytes >= 0x7fffffffLL ? 0x7fffffff : (int)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

// Store of 8 code bytes per lane where a wave instruction covers whole
// 128-byte lines (consecutive lanes, consecutive 8-byte pieces): the
// non-temporal hint streams them to memory during the kernel instead of
// leaving them dirty in L2 for the write-back at its end.
__device__ __forceinline__ void st_codes8(int8_t* p, u32x2 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(p));
}

__device__ __forceinline__ u32x4 bload16(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ u32x2 bload8(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t bload4(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ uint16_t bload2(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
__device__ __forceinline__ uint8_t bload1(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}

// The 8 fp16 values of a 16-byte chunk, widened to fp32.
__device__ __forceinline__ void unpack8(const u32x4& v, float* x) {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = h2f((uint16_t)(v[j >> 1] >> (16 * (j & 1))));
}

// Wave index within the block as a wave-uniform (scalar) value, so values
// derived from it (row pointers, buffer descriptors) stay in SGPRs.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Dynamic-scale codes of 8 values with |x / s| <= q_max (1 + 2^-23), q_max <= 127.
// Fast path: t = fl(x * r + 128) with r = fl32(1/s) (one fused multiply-add).
// |x*r - x/s| <= 128 * 2^-24 and the rounding of t adds at most 2^-17, so
// |t - (x/s + 128)| <= 2^-16, and fl(x/s) lies within 2^-18 of x/s: unless t
// is within 2^-14 of a rounding boundary (n + 1/2), rint(t) - 128 equals
// rint(fl(x/s)).  A chunk with any element that close takes the correctly
// rounded division instead.  Codes are within [-q_max, q_max] by the bound,
// so rint(t) is in [1, 255] and v_cvt_pk_u8_f32 packs it exactly; XOR 0x80
// turns each byte into the two's-complement code.
__device__ __forceinline__ u32x2 codes8_dyn(const float* x, float s, float r) {
    float n[8];
    float dmax = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float t = __builtin_fmaf(x[j], r, 128.0f);
        n[j] = __builtin_rintf(t);
        dmax = fmaxf(dmax, __builtin_fabsf(t - n[j]));
    }
    if (dmax > 0.5f - 0x1p-14f) {
#pragma unroll
        for (int j = 0; j < 8; ++j) n[j] = __builtin_rintf(x[j] / s) + 128.0f;
    }
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) lo = __builtin_amdgcn_cvt_pk_u8_f32(n[j], j, lo);
#pragma unroll
    for (int j = 0; j < 4; ++j) hi = __builtin_amdgcn_cvt_pk_u8_f32(n[j + 4], j, hi);
    return u32x2{lo ^ 0x80808080u, hi ^ 0x80808080u};
}

// codes8_dyn on the eight fp16 values of a 16-byte chunk (widened inside the
// fused multiply-adds, so no separate conversions on the fast path).
__device__ __forceinline__ u32x2 codes8_dyn_h(const u32x4& v, float s, float r) {
    float x[8], n[8];
    float dmax = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        x[j] = h2f((uint16_t)(v[j >> 1] >> (16 * (j & 1))));
        const float t = __builtin_fmaf(x[j], r, 128.0f);
        n[j] = __builtin_rintf(t);
        dmax = fmaxf(dmax, __builtin_fabsf(t - n[j]));
    }
    if (dmax > 0.5f - 0x1p-14f) {
#pragma unroll
        for (int j = 0; j < 8; ++j) n[j] = __builtin_rintf(x[j] / s) + 128.0f;
    }
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) lo = __builtin_amdgcn_cvt_pk_u8_f32(n[j], j, lo);
#pragma unroll
    for (int j = 0; j < 4; ++j) hi = __builtin_amdgcn_cvt_pk_u8_f32(n[j + 4], j, hi);
    return u32x2{lo ^ 0x80808080u, hi ^ 0x80808080u};
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

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Two 16-bit unsigned maxima in one instruction (v_pk_max_u16).
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t,
                              __builtin_elementwise_max(__builtin_bit_cast(u16x2, a), __builtin_bit_cast(u16x2, b)));
}

// Maximum of an unsigned value over the 64 lanes, returned wave-uniform.
// DPP moves (quad_perm [1,0,3,2], [2,3,0,1], row_half_mirror, row_mirror)
// reduce each row of 16 lanes without LDS traffic; the four row maxima are
// combined on the scalar unit.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));
    const uint32_t a = max((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16));
    const uint32_t b = max((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48));
    return max(a, b);
}

// Workgroup barrier that waits for this wave's LDS accesses only (gfx9
// s_waitcnt encoding lgkmcnt(0)); its global loads and stores stay in flight.
// The memory clobbers keep the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_only_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Number of set bits of a 64-bit lane mask held by lanes below this one.
__device__ __forceinline__ int bits_below(uint64_t m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Exchange of a double with the lane whose index differs in bit d (d = 1 or
// 2) by DPP quad permutations of its two 32-bit halves (no LDS traffic).
template <int D>
__device__ __forceinline__ double dpp_xor_f64(double v) {
    static_assert(D == 1 || D == 2, "quad permutations only");
    constexpr int ctrl = D == 1 ? 0xB1 : 0x4E;     // quad_perm [1,0,3,2] / [2,3,0,1]
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, ctrl, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), ctrl, 0xF, 0xF, false);
    return __builtin_bit_cast(double, (uint64_t)lo | ((uint64_t)hi << 32));
}

__device__ __forceinline__ int clampi(int v, int lo, int hi) {
    return v < lo ? lo : (v > hi ? hi : v);
}

// dynamic codes with the clip of a narrower [qmin, qmax] than [-qmax, qmax]
__device__ __forceinline__ u32x2 clip_codes(u32x2 c, int qmin) {
    if (qmin <= -127) return c;
    uint32_t w[2] = {c[0], c[1]};
#pragma unroll
    for (int d = 0; d < 2; ++d) {
        uint32_t o = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int q = (int8_t)(w[d] >> (8 * j));
            q = q < qmin ? qmin : q;
            o |= ((uint32_t)q & 0xffu) << (8 * j);
        }
        w[d] = o;
    }
    return u32x2{w[0], w[1]};
}

// The low nibbles of eight bytes as one 32-bit word: byte i's nibble in
// bits [4i+3 : 4i].
__device__ __forceinline__ uint32_t pack_nibbles(u32x2 c) {
    uint32_t w[2];
#pragma unroll
    for (int d = 0; d < 2; ++d) {
        uint32_t a = c[d] & 0x0f0f0f0fu;          // nibbles of 4 codes in bytes
        a = (a | (a >> 4)) & 0x00ff00ffu;        // codes 0,1 in byte 0; 2,3 in byte 2
        w[d] = (a | (a >> 8)) & 0xffffu;
    }
    return w[0] | (w[1] << 16);
}

// Eight int4 codes of one chunk as one 32-bit word: element i in bits
// [4i+3 : 4i], two's complement.
__device__ __forceinline__ uint32_t pack_codes(const float* x, float s, float r, int qmin) {
    return pack_nibbles(clip_codes(codes8_dyn(x, s, r), qmin));
}

// Largest magnitude of eight values.
__device__ __forceinline__ float absmax8f(const float* x) {
    float a = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) a = fmaxf(a, __builtin_fabsf(x[j]));
    return a;
}

}  // namespace qa
