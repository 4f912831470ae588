// k_decode.hip -- the LLM.int8() mixed linear for decode shapes (M <= 16
// tokens) as one fused kernel on gfx950.
//
// Decode is bound by streaming the int8 weight from HBM; the activation is a
// few KB.  Every workgroup owns 16 output channels; its four waves split K in
// quarters.  A workgroup
//   1. issues its X loads, then ALL of its weight loads (directly in the
//      B-operand layout of v_mfma_i32_16x16x64_i8, 16 x 16 bytes per lane),
//   2. while the weight bytes are in flight, recomputes -- identically in every
//      workgroup -- the outlier columns (column max over the tokens, on the
//      sign-cleared fp16 bit patterns with packed 16-bit max), the per-token
//      scales and the int8 codes of X into LDS (the A operand), the ascending
//      outlier list, the fp16 outlier activations, and starts the gather of
//      the fp16 outlier weights,
//   3. multiplies its K quarter on the MFMA, sums the four int32 partial tiles
//      in LDS, dequantizes by s_x[m] * s_w[n] and adds the outlier product.
// Loads retire in order (vmcnt), so the X loads go first: the prologue only
// waits for X, not for the weight stream behind it.
//
// Method: AIInfra 05Quantization01, LLM.int8(): outlier columns by magnitude
// threshold, "a. 向量级量化" (per-token / per-channel absmax scales),
// "b. INT8 矩阵乘法与反量化" (int32 accumulation, outer-product dequant) and
// the merge with the fp16 outlier product; Quantization explained part 2 §1.2.
#include "qa_device.hpp"
#include "qa_launch.hpp"

namespace qa {

constexpr int DEC_MAXK = 4096;             // K <= 4096, K % 256 == 0
constexpr int DEC_MAXSTEPS = DEC_MAXK / 256;
constexpr int DEC_LDA = DEC_MAXK + 16;     // LDS row stride of the codes (spreads banks)
constexpr int DEC_OCAP = 64;               // outliers whose operands are staged in LDS

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Two 16-bit unsigned maxima in one instruction (v_pk_max_u16).
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t,
                              __builtin_elementwise_max(__builtin_bit_cast(u16x2, a), __builtin_bit_cast(u16x2, b)));
}

__device__ __forceinline__ float half_lo(uint32_t v) { return h2f((uint16_t)(v & 0xffffu)); }
__device__ __forceinline__ float half_hi(uint32_t v) { return h2f((uint16_t)(v >> 16)); }

template <int MB>
__global__ __launch_bounds__(256) void k_decode_mixed(const uint16_t* __restrict__ X, int M, int K,
                                                      const int8_t* __restrict__ Wq, const float* __restrict__ s_w,
                                                      const uint16_t* __restrict__ W16, int64_t N, float tau,
                                                      void* __restrict__ out, int out_dtype) {
    __shared__ __attribute__((aligned(16))) int8_t aq[16 * DEC_LDA];
    __shared__ int32_t oidx[DEC_MAXK];
    __shared__ int32_t red[4][256];
    __shared__ float xo[DEC_OCAP][16];       // outlier activations  [h][m]
    __shared__ float wo[DEC_OCAP][16];       // outlier weights w~   [h][channel]
    __shared__ uint32_t rmax[4][MB];
    __shared__ float sx_s[16];
    __shared__ int wtot[4];

    const int t = threadIdx.x, lane = t & 63, wave = wave_id();
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    const int steps = K >> 8;                         // 64-wide MFMA steps per wave
    const int kw = wave * (K >> 2);                   // this wave's K quarter
    const int nch = K >> 3;                           // 8-column chunks of X

    // 1a. X chunks: thread t owns chunks t and t + 256 (8 columns each).  Up to
    //     8 tokens they stay in registers; beyond that the code pass re-reads.
    constexpr bool KEEPX = MB <= 8;
    const rsrc_t rsx = make_rsrc(X, (int64_t)M * K * 2);           // tokens past M read zeros
    auto xload = [&](int m, int i) -> u32x4 {
        const int c = t + 256 * i;
        return bload16(rsx, c < nch ? (uint32_t)(m * K + 8 * c) * 2 : kOOB);
    };
    u32x4 xv[KEEPX ? MB : 1][2];
    if constexpr (KEEPX) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int m = 0; m < MB; ++m) xv[m][i] = xload(m, i);
    }
    // 1b. the weight slice: row n0 + lane % 16, bytes kw + 64 s + 16 (lane / 16)
    v4i wv[DEC_MAXSTEPS];
    const rsrc_t rsw = make_rsrc(Wq + n0 * K, (N - n0) * K);       // channels past N read zeros
    {
        const uint32_t wo0 = (uint32_t)((lane & 15) * K + kw + 16 * (lane >> 4));
#pragma unroll
        for (int s = 0; s < DEC_MAXSTEPS; ++s)
            wv[s] = __builtin_bit_cast(v4i, bload16(rsw, s < steps ? wo0 + 64 * s : kOOB));
    }

    // 2a. column max over the tokens on |x| bit patterns (fp16 magnitudes order
    //     like their bits), outlier flags per chunk (8 bits), then the per-token
    //     absmax over the non-outlier columns.
    uint32_t flags[2];
    u32x4 keepw[2];                                   // 0xffff per ordinary column, 0 per outlier
    uint32_t ra[MB];
#pragma unroll
    for (int m = 0; m < MB; ++m) ra[m] = 0u;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        u32x4 xt[MB];
#pragma unroll
        for (int m = 0; m < MB; ++m) {
            if constexpr (KEEPX)
                xt[m] = xv[m][i];
            else
                xt[m] = xload(m, i);
        }
        uint32_t cm[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int d = 0; d < 4; ++d) cm[d] = pk_max_u16(cm[d], xt[m][d] & 0x7fff7fffu);
        uint32_t f = 0;
        uint32_t keep[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const bool olo = half_lo(cm[d]) > tau, ohi = half_hi(cm[d]) > tau;
            f |= (olo ? 1u : 0u) << (2 * d);
            f |= (ohi ? 1u : 0u) << (2 * d + 1);
            keep[d] = (olo ? 0u : 0xffffu) | (ohi ? 0u : 0xffff0000u);
        }
        f = (t + 256 * i < nch) ? f : 0u;
        flags[i] = f;
        keepw[i] = u32x4{keep[0], keep[1], keep[2], keep[3]};
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int d = 0; d < 4; ++d) ra[m] = pk_max_u16(ra[m], xt[m][d] & 0x7fff7fffu & keep[d]);
    }
#pragma unroll
    for (int m = 0; m < MB; ++m) {
        uint32_t a = max(ra[m] & 0xffffu, ra[m] >> 16);
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) a = max(a, (uint32_t)__shfl_xor((int)a, o, QA_WAVE));
        if (lane == 0) rmax[wave][m] = a;
    }

    // 2b. ascending outlier list (block-wide exclusive scan per chunk slot);
    //     the owner of an outlier column also stages its activations.
    int base = 0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int cnt = __popc(flags[i]);
        int x = cnt;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            int y = __shfl_up(x, d, QA_WAVE);
            if (lane >= d) x += y;
        }
        if (lane == 63) wtot[wave] = x;
        __syncthreads();
        int off = base + x - cnt;
        for (int w = 0; w < wave; ++w) off += wtot[w];
        const int c = t + 256 * i;
        uint32_t f = flags[i];
        while (f) {
            const int j = __builtin_ctz(f);
            f &= f - 1u;
            oidx[off] = 8 * c + j;
            if (off < DEC_OCAP) {
#pragma unroll
                for (int m = 0; m < MB; ++m) {
                    const uint32_t w32 = KEEPX ? xv[KEEPX ? m : 0][i][j >> 1]
                                               : (uint32_t)bload2(rsx, (uint32_t)(m * K + 8 * c + j) * 2);
                    xo[off][m] = KEEPX ? ((j & 1) ? half_hi(w32) : half_lo(w32)) : half_lo(w32);
                }
            }
            ++off;
        }
        base += wtot[0] + wtot[1] + wtot[2] + wtot[3];
        __syncthreads();
    }
    const int count = base;

    // 2c. start the gather of the fp16 outlier weights w~[n][h] (first 64)
    const int gch = t & 15, gh = t >> 4;              // channel n0 + gch, outlier slots gh + 16 q
    const rsrc_t rsn = make_rsrc(s_w + n0, (N - n0) * 4);
    const rsrc_t rs16 = make_rsrc(W16 ? W16 + n0 * K : nullptr, W16 ? (N - n0) * K * 2 : 0);
    const float swg = __builtin_bit_cast(float, bload4(rsn, (uint32_t)gch * 4));
    float gw[DEC_OCAP / 16];
#pragma unroll
    for (int q = 0; q < DEC_OCAP / 16; ++q) {
        const int h = gh + 16 * q;
        const uint32_t k = (uint32_t)oidx[h < count ? h : 0];
        const uint32_t off = h < count ? (uint32_t)gch * K + k : kOOB;
        if (W16)
            gw[q] = h2f(bload2(rs16, off == kOOB ? kOOB : off * 2));
        else
            gw[q] = h2f(f2h(swg * (float)(int8_t)bload1(rsw, off)));
    }

    // 2d. per-token scales (every thread derives the same values), int8 codes
    float sxm[MB];
#pragma unroll
    for (int m = 0; m < MB; ++m) {
        const uint32_t ab = max(max(rmax[0][m], rmax[1][m]), max(rmax[2][m], rmax[3][m]));
        const float a = h2f((uint16_t)ab);
        sxm[m] = a == 0.0f ? 1.0f : a / 127.0f;
        if (t == m) sx_s[m] = sxm[m];
    }
#pragma unroll
    for (int m = 0; m < MB; ++m) {
        if (m >= M) break;
        const float s = sxm[m], r = 1.0f / s;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int c = t + 256 * i;
            if (c >= nch) continue;
            u32x4 xc;
            if constexpr (KEEPX)
                xc = xv[m][i];
            else
                xc = xload(m, i);
            float xf[8];
            unpack8(xc & keepw[i], xf);                   // outlier columns -> 0 -> code 0
            const u32x2 cw = codes8_dyn(xf, s, r);
            const uint32_t lo = cw[0], hi = cw[1];
            *reinterpret_cast<u32x2*>(aq + m * DEC_LDA + 8 * c) = u32x2{lo, hi};
        }
    }
    __syncthreads();

    // 3a. int32 MFMA over this wave's K quarter
    v4i acc = v4i{0, 0, 0, 0};
    const int arow = lane & 15;
#pragma unroll
    for (int s = 0; s < DEC_MAXSTEPS; ++s) {
        if (s < steps) {
            v4i fa = v4i{0, 0, 0, 0};
            if (arow < M) fa = *reinterpret_cast<const v4i*>(aq + arow * DEC_LDA + kw + 64 * s + 16 * (lane >> 4));
            acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa, wv[s], acc, 0, 0, 0);
        }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) red[wave][(4 * (lane >> 4) + e) * 16 + (lane & 15)] = acc[e];
#pragma unroll
    for (int q = 0; q < DEC_OCAP / 16; ++q)
        if (gh + 16 * q < DEC_OCAP) wo[gh + 16 * q][gch] = gw[q];
    __syncthreads();

    // 3b. epilogue: thread t -> token m = t / 16, channel n0 + t % 16
    const int m = t >> 4, ch = t & 15;
    const int64_t n = n0 + ch;
    if (m < M && n < N) {
        const int32_t c = red[0][t] + red[1][t] + red[2][t] + red[3][t];
        const float sw = s_w[n];
        float v = (float)c * sx_s[m] * sw;
        const int hs = count < DEC_OCAP ? count : DEC_OCAP;
        for (int h = 0; h < hs; ++h) v = v + xo[h][m] * wo[h][ch];
        for (int h = DEC_OCAP; h < count; ++h) {          // beyond the staged outliers
            const int k = oidx[h];
            const float wt = W16 ? h2f(W16[n * K + k]) : h2f(f2h(sw * (float)Wq[n * K + k]));
            v = v + h2f(X[(int64_t)m * K + k]) * wt;
        }
        const int64_t o = (int64_t)m * N + n;
        if (out_dtype == 0)
            static_cast<float*>(out)[o] = v;
        else if (out_dtype == 1)
            static_cast<uint16_t*>(out)[o] = f2h(v);
        else
            static_cast<uint16_t*>(out)[o] = f2bf(v);
    }
}

bool decode_supported(int64_t M, int64_t K) {
    return M >= 1 && M <= 16 && K >= 256 && K <= DEC_MAXK && K % 256 == 0;
}

hipError_t launch_decode_mixed(const uint16_t* X, int64_t M, int64_t K, const int8_t* Wq, const float* s_w,
                               const uint16_t* W16, int64_t N, float tau, void* out, int out_dtype,
                               hipStream_t st) {
    const dim3 grid((unsigned)((N + 15) / 16)), block(256);
    if (M <= 4)
        hipLaunchKernelGGL(k_decode_mixed<4>, grid, block, 0, st, X, (int)M, (int)K, Wq, s_w, W16, N, tau, out,
                           out_dtype);
    else if (M <= 8)
        hipLaunchKernelGGL(k_decode_mixed<8>, grid, block, 0, st, X, (int)M, (int)K, Wq, s_w, W16, N, tau, out,
                           out_dtype);
    else
        hipLaunchKernelGGL(k_decode_mixed<16>, grid, block, 0, st, X, (int)M, (int)K, Wq, s_w, W16, N, tau, out,
                           out_dtype);
    return hipGetLastError();
}

}  // namespace qa
