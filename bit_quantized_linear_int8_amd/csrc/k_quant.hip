// k_quant.hip -- HBM-bound kernels of the quantized linear layer on gfx950:
// outlier-column detection, row-wise int8 quantization and the block
// Hadamard rotation fused with int4 quantization and packing.
//
// Sources (by page title and section):
//   AIInfra 05Quantization01 (模型量化), LLM.int8(): outlier detection by a
//     magnitude threshold; "a. 向量级量化" (per-row scales).
//   模型推理量化 (Inference Quantization notes): §4 scale s = absmax/qmax and
//     q = round(x/s), safe scale for an all-zero group; §6.2 affine clip.
//   低比特量化加速：分组旋转方法从W8A8到W4A4: §二 normalized Hadamard on
//     G-wide blocks, §5.2 rotation fused with dynamic quantization, §5.4
//     eight int4 per 32-bit word.
#include "qa_device.hpp"
#include "qa_launch.hpp"

namespace qa {

// ---------------------------------------------------------------------------
// Zero fill (used instead of hipMemsetAsync so the sequence can be captured).
// ---------------------------------------------------------------------------
__global__ void k_zero_u32(uint32_t* __restrict__ p, int64_t n) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

// ---------------------------------------------------------------------------
// Outlier columns.  Each block reduces a tile of OC_ROWS rows x OC_COLS
// columns (every lane owns 8 adjacent columns, one 16-byte load per row),
// folds the four waves in LDS and merges into the running column max with a
// device-scope atomic max on the fp32 bits (non-negative floats order like
// their bit patterns).  The last block to finish (ticket) turns the column
// max into the mask and the ascending outlier list with a ballot scan.
// ---------------------------------------------------------------------------
constexpr int OC_COLS = 512;
constexpr int OC_ROWS = 64;

__global__ __launch_bounds__(256) void k_outlier_cols(
    const uint16_t* __restrict__ X, int64_t M, int64_t K, float tau, uint32_t* __restrict__ cmax,
    uint32_t* __restrict__ ticket, uint8_t* __restrict__ mask, int32_t* __restrict__ idx,
    int32_t* __restrict__ count, float* __restrict__ colmax_out) {
    __shared__ float red[4][OC_COLS];
    __shared__ int is_last;
    __shared__ int wave_tot[4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t c0 = (int64_t)blockIdx.x * OC_COLS + lane * 8;
    const int64_t r0 = (int64_t)blockIdx.y * OC_ROWS;
    float m[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) m[j] = 0.0f;
    if (c0 < K) {
        const int64_t rend = r0 + OC_ROWS < M ? r0 + OC_ROWS : M;
#pragma unroll 4
        for (int64_t r = r0 + wave; r < rend; r += 4) {
            u32x4 v = *reinterpret_cast<const u32x4*>(X + r * K + c0);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                uint16_t h = (uint16_t)(v[j >> 1] >> (16 * (j & 1)));
                m[j] = fmaxf(m[j], __builtin_fabsf(h2f(h)));
            }
        }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) red[wave][lane * 8 + j] = m[j];
    __syncthreads();
    for (int cc = threadIdx.x; cc < OC_COLS; cc += 256) {
        float v = fmaxf(fmaxf(red[0][cc], red[1][cc]), fmaxf(red[2][cc], red[3][cc]));
        int64_t col = (int64_t)blockIdx.x * OC_COLS + cc;
        if (col < K) atomicMax(&cmax[col], __builtin_bit_cast(uint32_t, v));
    }
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned total = gridDim.x * gridDim.y;
        is_last = (atomicAdd(ticket, 1u) == total - 1u);
    }
    __syncthreads();
    if (!is_last) return;
    __threadfence();
    int running = 0;
    for (int64_t base = 0; base < K; base += 256) {
        const int64_t col = base + threadIdx.x;
        bool o = false;
        if (col < K) {
            uint32_t b = __hip_atomic_load(&cmax[col], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            float cm = __builtin_bit_cast(float, b);
            o = cm > tau;
            mask[col] = o ? 1 : 0;
            if (colmax_out) colmax_out[col] = cm;
        }
        const uint64_t bal = __ballot(o);
        const int pre = __popcll(bal & ((1ull << lane) - 1ull));
        if (lane == 0) wave_tot[wave] = __popcll(bal);
        __syncthreads();
        int off = running;
        for (int w = 0; w < wave; ++w) off += wave_tot[w];
        if (o) idx[off + pre] = (int32_t)col;
        running += wave_tot[0] + wave_tot[1] + wave_tot[2] + wave_tot[3];
        __syncthreads();
    }
    if (threadIdx.x == 0) *count = running;
}

size_t outlier_scratch_bytes(int64_t K) { return (size_t)(K + 64) * 4; }

hipError_t launch_outlier_cols(const uint16_t* X, int64_t M, int64_t K, float tau, uint8_t* mask,
                               int32_t* idx, int32_t* count, float* colmax, void* scratch,
                               hipStream_t st) {
    uint32_t* cmax = static_cast<uint32_t*>(scratch);
    uint32_t* ticket = cmax + K;
    const int64_t nz = K + 1;
    hipLaunchKernelGGL(k_zero_u32, dim3((unsigned)((nz + 255) / 256 < 1024 ? (nz + 255) / 256 : 1024)),
                       dim3(256), 0, st, cmax, nz);
    dim3 grid((unsigned)((K + OC_COLS - 1) / OC_COLS), (unsigned)(M > 0 ? (M + OC_ROWS - 1) / OC_ROWS : 1));
    hipLaunchKernelGGL(k_outlier_cols, grid, dim3(256), 0, st, X, M, K, tau, cmax, ticket, mask, idx,
                       count, colmax);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Row-wise int8 quantization: one wave per row, 8 elements (16 bytes) per
// lane and chunk.  NC > 0 keeps the row in registers (K <= 512 * NC); NC == 0
// reads the row twice (absmax pass, then quantize pass).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void unpack8(const u32x4& v, float* x) {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = h2f((uint16_t)(v[j >> 1] >> (16 * (j & 1))));
}

template <bool STATIC>
__device__ __forceinline__ uint64_t quant8(const float* x, uint64_t mk, float s, float r, int z, int qmin,
                                           int qmax) {
    uint64_t out = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        int code;
        if ((mk >> (8 * j)) & 0xffu) {
            code = clampi(z, qmin, qmax);
        } else if (STATIC) {
            double t = (double)__builtin_rintf(x[j] / s) + (double)z;
            t = t < (double)qmin ? (double)qmin : (t > (double)qmax ? (double)qmax : t);
            code = (int)t;
        } else {
            code = clampi((int)quot_rne(x[j], s, r), qmin, qmax);
        }
        out |= (uint64_t)(uint8_t)(int8_t)code << (8 * j);
    }
    return out;
}

__device__ __forceinline__ float absmax8(const float* x, uint64_t mk) {
    float a = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
        if (!((mk >> (8 * j)) & 0xffu)) a = fmaxf(a, __builtin_fabsf(x[j]));
    return a;
}

template <int NC, bool STATIC>
__global__ __launch_bounds__(256) void k_rowquant_i8(const uint16_t* __restrict__ X, int64_t rows,
                                                     int64_t K, const uint8_t* __restrict__ mask,
                                                     int qmin, int qmax, const float* __restrict__ s_in,
                                                     const int32_t* __restrict__ z_in,
                                                     int8_t* __restrict__ q, float* __restrict__ s_out) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int64_t nch = K >> 3;
    const uint16_t* xr = X + row * K;
    int8_t* qr = q + row * K;
    float s, r = 1.0f;
    int z = 0;
    if constexpr (NC > 0) {
        u32x4 v[NC];
        uint64_t mk[NC];
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const int64_t ch = lane + 64 * i;
            if (ch < nch) {
                v[i] = *reinterpret_cast<const u32x4*>(xr + ch * 8);
                mk[i] = mask ? *reinterpret_cast<const uint64_t*>(mask + ch * 8) : 0ull;
            } else {
                v[i] = u32x4{0u, 0u, 0u, 0u};
                mk[i] = 0ull;
            }
        }
        if constexpr (STATIC) {
            s = s_in[row];
            z = z_in ? z_in[row] : 0;
        } else {
#pragma unroll
            for (int i = 0; i < NC; ++i) {
                float x[8];
                unpack8(v[i], x);
                amax = fmaxf(amax, absmax8(x, mk[i]));
            }
            amax = wave_max(amax);
            s = amax == 0.0f ? 1.0f : amax / (float)qmax;
            r = 1.0f / s;
            if (lane == 0) s_out[row] = s;
        }
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const int64_t ch = lane + 64 * i;
            if (ch < nch) {
                float x[8];
                unpack8(v[i], x);
                *reinterpret_cast<uint64_t*>(qr + ch * 8) = quant8<STATIC>(x, mk[i], s, r, z, qmin, qmax);
            }
        }
    } else {
        if constexpr (STATIC) {
            s = s_in[row];
            z = z_in ? z_in[row] : 0;
        } else {
            float amax = 0.0f;
            for (int64_t ch = lane; ch < nch; ch += 64) {
                float x[8];
                unpack8(*reinterpret_cast<const u32x4*>(xr + ch * 8), x);
                uint64_t mk = mask ? *reinterpret_cast<const uint64_t*>(mask + ch * 8) : 0ull;
                amax = fmaxf(amax, absmax8(x, mk));
            }
            amax = wave_max(amax);
            s = amax == 0.0f ? 1.0f : amax / (float)qmax;
            r = 1.0f / s;
            if (lane == 0) s_out[row] = s;
        }
        for (int64_t ch = lane; ch < nch; ch += 64) {
            float x[8];
            unpack8(*reinterpret_cast<const u32x4*>(xr + ch * 8), x);
            uint64_t mk = mask ? *reinterpret_cast<const uint64_t*>(mask + ch * 8) : 0ull;
            *reinterpret_cast<uint64_t*>(qr + ch * 8) = quant8<STATIC>(x, mk, s, r, z, qmin, qmax);
        }
    }
}

template <bool STATIC>
static void rowquant_dispatch(const uint16_t* X, int64_t rows, int64_t K, const uint8_t* mask, int qmin,
                              int qmax, const float* s_in, const int32_t* z_in, int8_t* q, float* s_out,
                              hipStream_t st) {
    const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
    const int64_t nch = K / 8;
#define QA_RQ(NC) hipLaunchKernelGGL((k_rowquant_i8<NC, STATIC>), grid, block, 0, st, X, rows, K, mask, qmin, \
                                     qmax, s_in, z_in, q, s_out)
    if (nch <= 64) QA_RQ(1);
    else if (nch <= 128) QA_RQ(2);
    else if (nch <= 256) QA_RQ(4);
    else if (nch <= 512) QA_RQ(8);
    else if (nch <= 1024) QA_RQ(16);
    else QA_RQ(0);
#undef QA_RQ
}

hipError_t launch_rowquant_i8(const uint16_t* X, int64_t rows, int64_t K, const uint8_t* mask, int qmin,
                              int qmax, const float* s_in, const int32_t* z_in, int8_t* q, float* s_out,
                              hipStream_t st) {
    if (s_in)
        rowquant_dispatch<true>(X, rows, K, mask, qmin, qmax, s_in, z_in, q, s_out, st);
    else
        rowquant_dispatch<false>(X, rows, K, mask, qmin, qmax, s_in, z_in, q, s_out, st);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Block Hadamard rotation + int4 quantization + packing.  One wave per row;
// lane l owns the 8 adjacent elements of chunk ch = l + 64 i.  A G-block spans
// G/8 lanes (G >= 8) or part of one lane (G < 8).  The butterfly runs in fp64:
// every partial sum of fp16 inputs is exact (multiples of 2^-24 below 2^16,
// at most 256 of them), then y * fl64(1/sqrt(G)) is rounded once to fp32.
// ---------------------------------------------------------------------------
template <int G>
__device__ __forceinline__ void fwht_chunk(const u32x4& v, double c, int lane, float* xo) {
    double y[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] = (double)h2f((uint16_t)(v[j >> 1] >> (16 * (j & 1))));
    // in-lane stages: element strides 1, 2, 4 (those below G)
#pragma unroll
    for (int h = 1; h < 8 && h < G; h <<= 1) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if ((j & h) == 0) {
                double a = y[j], b = y[j + h];
                y[j] = a + b;
                y[j + h] = a - b;
            }
        }
    }
    // cross-lane stages: lane distance d <-> element distance 8d
#pragma unroll
    for (int d = 1; d < G / 8; d <<= 1) {
        const double sg = (lane & d) ? -1.0 : 1.0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            double p = __shfl_xor(y[j], d, QA_WAVE);
            y[j] = __builtin_fma(sg, y[j], p);   // lower: y + p, upper: p - y (exact)
        }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) xo[j] = (float)(y[j] * c);
}

__device__ __forceinline__ uint32_t pack_codes(const float* x, float s, float r, int qmin, int qmax) {
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        int code = clampi((int)quot_rne(x[j], s, r), qmin, qmax);
        w |= ((uint32_t)code & 0xFu) << (4 * j);
    }
    return w;
}

__device__ __forceinline__ float absmax8f(const float* x) {
    float a = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) a = fmaxf(a, __builtin_fabsf(x[j]));
    return a;
}

// Per-row scale, row held in registers (NC > 0) or recomputed (NC == 0).
template <int G, int NC>
__global__ __launch_bounds__(256) void k_hq4_row(const uint16_t* __restrict__ X, int64_t rows, int64_t K,
                                                 int qmin, int qmax, double c, uint32_t* __restrict__ packed,
                                                 float* __restrict__ s_out) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int64_t nch = K >> 3;
    const uint16_t* xr = X + row * K;
    uint32_t* pr = packed + row * nch;
    if constexpr (NC > 0) {
        float xs[NC][8];
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const int64_t ch = lane + 64 * i;
            u32x4 v = ch < nch ? *reinterpret_cast<const u32x4*>(xr + ch * 8) : u32x4{0u, 0u, 0u, 0u};
            fwht_chunk<G>(v, c, lane, xs[i]);
            amax = fmaxf(amax, absmax8f(xs[i]));
        }
        amax = wave_max(amax);
        const float s = amax == 0.0f ? 1.0f : amax / (float)qmax;
        const float r = 1.0f / s;
        if (lane == 0) s_out[row] = s;
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const int64_t ch = lane + 64 * i;
            if (ch < nch) pr[ch] = pack_codes(xs[i], s, r, qmin, qmax);
        }
    } else {
        float amax = 0.0f;
        for (int64_t base = 0; base < nch; base += 64) {
            const int64_t ch = base + lane;
            u32x4 v = ch < nch ? *reinterpret_cast<const u32x4*>(xr + ch * 8) : u32x4{0u, 0u, 0u, 0u};
            float xo[8];
            fwht_chunk<G>(v, c, lane, xo);
            amax = fmaxf(amax, absmax8f(xo));
        }
        amax = wave_max(amax);
        const float s = amax == 0.0f ? 1.0f : amax / (float)qmax;
        const float r = 1.0f / s;
        if (lane == 0) s_out[row] = s;
        for (int64_t base = 0; base < nch; base += 64) {
            const int64_t ch = base + lane;
            u32x4 v = ch < nch ? *reinterpret_cast<const u32x4*>(xr + ch * 8) : u32x4{0u, 0u, 0u, 0u};
            float xo[8];
            fwht_chunk<G>(v, c, lane, xo);
            if (ch < nch) pr[ch] = pack_codes(xo, s, r, qmin, qmax);
        }
    }
}

// Per-group scale (G >= 8): the G/8 lanes of a block reduce their absmax.
template <int G>
__global__ __launch_bounds__(256) void k_hq4_group(const uint16_t* __restrict__ X, int64_t rows, int64_t K,
                                                   int qmin, int qmax, double c, uint32_t* __restrict__ packed,
                                                   float* __restrict__ s_out) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int64_t nch = K >> 3;
    const int64_t ngr = K / G;
    const uint16_t* xr = X + row * K;
    uint32_t* pr = packed + row * nch;
    for (int64_t base = 0; base < nch; base += 64) {
        const int64_t ch = base + lane;
        u32x4 v = ch < nch ? *reinterpret_cast<const u32x4*>(xr + ch * 8) : u32x4{0u, 0u, 0u, 0u};
        float xo[8];
        fwht_chunk<G>(v, c, lane, xo);
        float amax = group_max(absmax8f(xo), G / 8);
        const float s = amax == 0.0f ? 1.0f : amax / (float)qmax;
        const float r = 1.0f / s;
        if (ch < nch) {
            pr[ch] = pack_codes(xo, s, r, qmin, qmax);
            if ((lane & (G / 8 - 1)) == 0) s_out[row * ngr + (ch * 8) / G] = s;
        }
    }
}

template <int G>
static void hq4_dispatch(const uint16_t* X, int64_t rows, int64_t K, bool per_group, int qmin, int qmax,
                         uint32_t* packed, float* s, hipStream_t st) {
    const double c = 1.0 / __builtin_sqrt((double)G);
    const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
    if (per_group) {
        if constexpr (G >= 8)
            hipLaunchKernelGGL((k_hq4_group<G>), grid, block, 0, st, X, rows, K, qmin, qmax, c, packed, s);
        return;
    }
    const int64_t nch = K / 8;
#define QA_HQ(NC) hipLaunchKernelGGL((k_hq4_row<G, NC>), grid, block, 0, st, X, rows, K, qmin, qmax, c, packed, s)
    if (nch <= 64) QA_HQ(1);
    else if (nch <= 128) QA_HQ(2);
    else if (nch <= 256) QA_HQ(4);
    else if (nch <= 512) QA_HQ(8);
    else QA_HQ(0);
#undef QA_HQ
}

hipError_t launch_hadamard_quant_i4(const uint16_t* X, int64_t rows, int64_t K, int G, bool per_group,
                                    int qmin, int qmax, uint32_t* packed, float* s, hipStream_t st) {
    switch (G) {
        case 1: hq4_dispatch<1>(X, rows, K, per_group, qmin, qmax, packed, s, st); break;
        case 2: hq4_dispatch<2>(X, rows, K, per_group, qmin, qmax, packed, s, st); break;
        case 4: hq4_dispatch<4>(X, rows, K, per_group, qmin, qmax, packed, s, st); break;
        case 8: hq4_dispatch<8>(X, rows, K, per_group, qmin, qmax, packed, s, st); break;
        case 16: hq4_dispatch<16>(X, rows, K, per_group, qmin, qmax, packed, s, st); break;
        case 32: hq4_dispatch<32>(X, rows, K, per_group, qmin, qmax, packed, s, st); break;
        case 64: hq4_dispatch<64>(X, rows, K, per_group, qmin, qmax, packed, s, st); break;
        case 128: hq4_dispatch<128>(X, rows, K, per_group, qmin, qmax, packed, s, st); break;
        case 256: hq4_dispatch<256>(X, rows, K, per_group, qmin, qmax, packed, s, st); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace qa
