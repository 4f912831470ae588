// k_smooth.hip -- SmoothQuant on gfx950: the migration factors and the
// per-input-channel smoothing fused with int8 absmax quantization.
//
// Source: "Quantization explained, part 2" (tanjunchen.github.io), §4.2: the
// product X W is unchanged when column j of X is divided by s_j and the
// matching input channel of W is multiplied by it, with
// s_j = max|X_j|^alpha / max|W_j|^(1-alpha); §4.4: the factors are fixed
// offline, so the weight side is smoothed and quantized once.
//
// Rounding (bit-exact with a plain CPU evaluation): the smoothed value is one
// IEEE fp32 division (activations) or multiplication (weights) of the exact
// fp32 widening of the fp16 input; the scale is fl32(absmax / 127) (1.0 for an
// all-zero row or tensor) and the code rint(fl32(x^ / s)), ties to even.
#include "qa_device.hpp"
#include "qa_launch.hpp"

namespace qa {

// s_j = fl32(pow(cx_j, alpha) / pow(cw_j, 1 - alpha)) in fp64; 1 where either
// maximum is 0 (the formula has no value or gives 0 there).
__global__ __launch_bounds__(256) void k_smooth_factors(const float* __restrict__ cx, const float* __restrict__ cw,
                                                        int64_t K, double alpha, float* __restrict__ s) {
    const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (j >= K) return;
    const float a = cx[j], w = cw[j];
    float r = 1.0f;
    if (a != 0.0f && w != 0.0f) r = (float)(pow((double)a, alpha) / pow((double)w, 1.0 - alpha));
    s[j] = r;
}

hipError_t launch_smooth_factors(const float* cx, const float* cw, int64_t K, float alpha, float* s, hipStream_t st) {
    hipLaunchKernelGGL(k_smooth_factors, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, st, cx, cw, K,
                       (double)alpha, s);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Smoothing + int8 quantization.  NC > 0 holds the smoothed row in registers
// (K <= 512 NC) and reads X once, split over WPR waves (part p of the row's
// WPR waves owns chunks p 64 NC / WPR + l + 64 i in lane l), which combine
// their row maxima through LDS; NC == 0 is one wave per row, lane l owning
// the chunks l + 64 i, and reads the row twice (absmax pass, codes pass).
// The factor vector is read with the row (it is shared by every row, so
// after the first rows it comes from the caches).
//
// Phases:
//   SQ_ROW     per-row dynamic scale: s_out[row] = fl32(absmax / 127), codes
//   SQ_ROWMAX  first pass of a per-tensor scale: s_out[row] = smoothed absmax
//   SQ_CODES   codes with the scale s_out[row] left by k_tensor_scale
// SQ_ROW and SQ_CODES set a non-null `count` to 0 (block 0), the empty
// outlier list the int8 GEMM epilogue reads.
// ---------------------------------------------------------------------------
enum { SQ_DIVIDE = 0, SQ_MULTIPLY = 1 };
enum { SQ_ROW = 0, SQ_ROWMAX = 1, SQ_CODES = 2 };

// Smoothed values of one chunk.  Chunks past the row end (loads read zeros)
// are forced to 0 so 0/0 never reaches the absmax.
template <int OP>
__device__ __forceinline__ void smooth8(const u32x4& v, const u32x4& f0, const u32x4& f1, bool valid, float* x) {
    unpack8(v, x);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float f = __builtin_bit_cast(float, j < 4 ? f0[j] : f1[j - 4]);
        float y = OP == SQ_DIVIDE ? x[j] / f : x[j] * f;
        x[j] = valid ? y : 0.0f;
    }
}

template <int NC, int OP, int PHASE, int WPR>
__global__ __launch_bounds__(256) void k_smoothquant_i8(const uint16_t* __restrict__ X, int64_t rows, int64_t K,
                                                        const float* __restrict__ sm, int8_t* __restrict__ q,
                                                        float* __restrict__ s_out, int32_t* __restrict__ count) {
    static_assert(WPR == 1 || ((WPR == 2 || WPR == 4) && NC >= WPR), "waves per row need a row held in registers");
    constexpr int NCW = NC / WPR;
    constexpr bool XCHG = WPR > 1 && PHASE != SQ_CODES;      // row maxima combined over the row's waves
    __shared__ uint32_t pmx[XCHG ? 4 : 1];
    if (PHASE != SQ_ROWMAX && count && blockIdx.x == 0 && threadIdx.x == 0) *count = 0;
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int64_t row = (int64_t)blockIdx.x * (4 / WPR) + wave / WPR;
    const int part = wave % WPR;
    const bool live = row < rows;
    if (!XCHG && !live) return;
    const int64_t nch = K >> 3;
    const rsrc_t rx = make_rsrc(X + (live ? row : 0) * K, live ? K * 2 : 0);
    const rsrc_t rs = make_rsrc(sm, K * 4);
    int8_t* qr = q + row * K;
    float s = 1.0f, r = 1.0f;
    if constexpr (PHASE == SQ_CODES) {
        s = s_out[row];
        r = 1.0f / s;
    }
    auto cho = [&](int i) -> int64_t { return (int64_t)part * 64 * NCW + lane + 64 * i; };
    auto load_smooth = [&](int64_t ch, float* x) {
        const u32x4 v = bload16(rx, (uint32_t)ch * 16);
        const u32x4 f0 = bload16(rs, (uint32_t)ch * 32);
        const u32x4 f1 = bload16(rs, (uint32_t)ch * 32 + 16);
        smooth8<OP>(v, f0, f1, ch < nch, x);
    };
    // returns false in the waves of a row past the end (after the exchange)
    auto finish_scale = [&](float amax) -> bool {
        amax = wave_max(amax);
        if constexpr (XCHG) {
            // amax >= 0: with the sign bit cleared (-0.0 would order last)
            // its bit pattern orders like the value
            if (lane == 0) pmx[wave] = __builtin_bit_cast(uint32_t, amax) & 0x7fffffffu;
            lds_only_barrier();
            uint32_t ab = 0u;
#pragma unroll
            for (int w = 0; w < WPR; ++w) ab = max(ab, pmx[wave - part + w]);
            amax = __builtin_bit_cast(float, ab);
            if (!live) return false;
        }
        if constexpr (PHASE == SQ_ROWMAX) {
            if (lane == 0 && part == 0) s_out[row] = amax;
        } else {
            s = amax == 0.0f ? 1.0f : amax / 127.0f;
            r = 1.0f / s;
            if (lane == 0 && part == 0) s_out[row] = s;
        }
        return true;
    };
    if constexpr (NC > 0) {
        float x[NCW][8];
        u32x4 v[NCW], f0[NCW], f1[NCW];
#pragma unroll
        for (int i = 0; i < NCW; ++i) {                // every load of the wave's part in flight at once
            const uint32_t ch = (uint32_t)cho(i);
            v[i] = bload16(rx, ch * 16);
            f0[i] = bload16(rs, ch * 32);
            f1[i] = bload16(rs, ch * 32 + 16);
        }
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < NCW; ++i) {
            smooth8<OP>(v[i], f0[i], f1[i], live && cho(i) < nch, x[i]);
            if constexpr (PHASE != SQ_CODES) amax = fmaxf(amax, absmax8f(x[i]));
        }
        if constexpr (PHASE != SQ_CODES)
            if (!finish_scale(amax)) return;
        if constexpr (PHASE != SQ_ROWMAX) {
#pragma unroll
            for (int i = 0; i < NCW; ++i) {
                const int64_t ch = cho(i);
                if (ch < nch) st_codes8(qr + ch * 8, codes8_dyn(x[i], s, r));
            }
        }
    } else {
        if constexpr (PHASE != SQ_CODES) {
            float amax = 0.0f;
            for (int64_t ch = lane; ch < nch; ch += 64) {
                float x[8];
                load_smooth(ch, x);
                amax = fmaxf(amax, absmax8f(x));
            }
            finish_scale(amax);
        }
        if constexpr (PHASE != SQ_ROWMAX) {
            for (int64_t ch = lane; ch < nch; ch += 64) {
                float x[8];
                load_smooth(ch, x);
                st_codes8(qr + ch * 8, codes8_dyn(x, s, r));
            }
        }
    }
}

// Per-tensor scale from the per-row maxima in s[0..rows): one block takes the
// maximum, then writes fl32(max / 127) (1.0 if 0) into every s[r].  Each
// thread rewrites only the entries it read, so no entry is overwritten before
// it has been read.
__global__ __launch_bounds__(1024) void k_tensor_scale(float* __restrict__ s, int64_t rows) {
    __shared__ float red[16];
    float a = 0.0f;
    for (int64_t i = threadIdx.x; i < rows; i += 1024) a = fmaxf(a, s[i]);
    a = wave_max(a);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
    __syncthreads();
    a = red[0];
#pragma unroll
    for (int w = 1; w < 16; ++w) a = fmaxf(a, red[w]);
    const float st = a == 0.0f ? 1.0f : a / 127.0f;
    for (int64_t i = threadIdx.x; i < rows; i += 1024) s[i] = st;
}

template <int OP, int PHASE>
static void smoothquant_dispatch(const uint16_t* X, int64_t rows, int64_t K, const float* sm, int8_t* q,
                                 float* s_out, int32_t* count, hipStream_t st) {
    // four waves per row for rows of 16 chunks per lane, else one (two waves
    // per row measured slightly slower on 8 chunks, where the per-value
    // division dominates)
    const int64_t nch = K / 8;
    const int wpr = nch > 512 && nch <= 1024 ? 4 : 1;
    const dim3 grid((unsigned)((rows + 4 / wpr - 1) / (4 / wpr))), block(256);
#define QA_SQ(NC) hipLaunchKernelGGL((k_smoothquant_i8<NC, OP, PHASE, (NC >= 16 ? 4 : 1)>), grid, block, 0, st, X, \
                                     rows, K, sm, q, s_out, count)
    if (nch <= 64) QA_SQ(1);
    else if (nch <= 128) QA_SQ(2);
    else if (nch <= 256) QA_SQ(4);
    else if (nch <= 512) QA_SQ(8);
    else if (nch <= 1024) QA_SQ(16);
    else QA_SQ(0);
#undef QA_SQ
}

template <int OP>
static void smoothquant_launch(const uint16_t* X, int64_t rows, int64_t K, const float* sm, bool per_tensor,
                               int8_t* q, float* s_out, int32_t* count, hipStream_t st) {
    if (!per_tensor) {
        smoothquant_dispatch<OP, SQ_ROW>(X, rows, K, sm, q, s_out, count, st);
        return;
    }
    smoothquant_dispatch<OP, SQ_ROWMAX>(X, rows, K, sm, q, s_out, nullptr, st);
    hipLaunchKernelGGL(k_tensor_scale, dim3(1), dim3(1024), 0, st, s_out, rows);
    smoothquant_dispatch<OP, SQ_CODES>(X, rows, K, sm, q, s_out, count, st);
}

hipError_t launch_smoothquant_i8(const uint16_t* X, int64_t rows, int64_t K, const float* sm, bool multiply,
                                 bool per_tensor, int8_t* q, float* s_out, int32_t* count, hipStream_t st) {
    if (multiply)
        smoothquant_launch<SQ_MULTIPLY>(X, rows, K, sm, per_tensor, q, s_out, count, st);
    else
        smoothquant_launch<SQ_DIVIDE>(X, rows, K, sm, per_tensor, q, s_out, count, st);
    return hipGetLastError();
}

}  // namespace qa
