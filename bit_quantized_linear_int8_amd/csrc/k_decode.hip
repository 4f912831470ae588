// k_decode.hip -- the LLM.int8() mixed linear for decode shapes (M <= 16
// tokens) as one fused kernel on gfx950.
//
// Decode is bound by streaming the int8 weight from HBM; the activation is a
// few KB.  Every workgroup owns 16 output channels and has eight waves; wave w
// multiplies the 64-byte K steps w, w + 8, w + 16, ... so each weight load
// instruction of the block covers 16 rows x 512 contiguous bytes.  A workgroup
//   1. issues its X loads (thread t owns the 8-column chunk t of every token),
//      the scale of the channel it writes in the epilogue, then ALL of its
//      weight loads (directly in the B-operand layout of
//      v_mfma_i32_16x16x64_i8, 16 bytes per lane and step),
//   2. while the weight bytes are in flight, recomputes -- identically in every
//      workgroup -- the outlier columns (column max over the tokens, on the
//      sign-cleared fp16 bit patterns with packed 16-bit max), the per-token
//      scales and the int8 codes of X into LDS (the A operand), the ascending
//      outlier list, the fp16 outlier activations, and starts the gather of
//      the fp16 outlier weights,
//   3. multiplies its K steps on the MFMA, sums the eight int32 partial tiles
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
constexpr int DEC_WAVES = 8, DEC_THREADS = 64 * DEC_WAVES;
constexpr int DEC_MAXSTEPS = DEC_MAXK / 64 / DEC_WAVES;   // MFMA steps per wave
constexpr int DEC_LDA = DEC_MAXK + 16;     // LDS row stride of the codes (spreads banks)
constexpr int DEC_OCAP = 64;               // outliers whose operands are staged in LDS
static_assert(DEC_MAXK / 8 == DEC_THREADS, "one 8-column chunk of X per thread");
static_assert(DEC_WAVES == 8, "the wave totals are read as two 16-byte vectors");

__device__ __forceinline__ float half_lo(uint32_t v) { return h2f((uint16_t)(v & 0xffffu)); }
__device__ __forceinline__ float half_hi(uint32_t v) { return h2f((uint16_t)(v >> 16)); }

// Workgroup barrier for LDS traffic only: waits for this wave's LDS accesses
// (lgkmcnt(0)), not for its global loads, so the weight stream stays in
// flight across it (__syncthreads also waits for every outstanding load).
// The memory clobbers keep the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);      // gfx9 encoding: lgkmcnt(0), vmcnt and expcnt not waited
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Element i of a 4-word vector by selects (no dynamically indexed registers).
__device__ __forceinline__ uint32_t pick4(const u32x4& v, int i) {
    const uint32_t lo = (i & 1) ? v[1] : v[0], hi = (i & 1) ? v[3] : v[2];
    return (i & 2) ? hi : lo;
}

// Maximum of an unsigned value over the 64 lanes, in every lane: DPP within
// rows of 16, then gfx950's row-pair and half-wave swaps (no scalar round trip).
__device__ __forceinline__ uint32_t wave_max_all_u32(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));    // quad_perm [1,0,3,2]
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));    // quad_perm [2,3,0,1]
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));   // row_half_mirror
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));   // row_mirror
    const auto p16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = max(p16[0], p16[1]);
    const auto p32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return max(p32[0], p32[1]);
}

// Eight int8 codes rint(fl32(x / s)) of one chunk without a division, with
// r = fl32(1 / s).  The fast code is rint(fma(x, r, 128)); a chunk holding a
// value with |t - rint(t)| > 0.5 - 2^-16 (near a tie) is redone with
//   q0 = fl32(x r),  e = x - q0 s (exact, one fused multiply-add),
//   q  = fl32(q0 + e r)  (one fused multiply-add),
// Markstein's correction step for division (P. W. Markstein, "Computation of
// elementary functions on the IBM RISC System/6000 processor", 1990), which
// is the correctly rounded fl32(x / s).  Both facts hold for every fp16 x and
// every scale fl32(a / 127) of an fp16 a >= |x| -- the per-token scales here;
// the test suite checks all 1.0e9 such pairs on the CPU.
__device__ __forceinline__ u32x2 codes8_dec(const u32x4& v, float s, float r) {
    float x[8], n[8];
    float dmax = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        x[j] = h2f((uint16_t)(v[j >> 1] >> (16 * (j & 1))));
        const float t = __builtin_fmaf(x[j], r, 128.0f);
        n[j] = __builtin_rintf(t);
        dmax = fmaxf(dmax, __builtin_fabsf(t - n[j]));
    }
    if (dmax > 0.5f - 0x1p-16f) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float q0 = x[j] * r;
            const float e = __builtin_fmaf(-q0, s, x[j]);
            n[j] = __builtin_rintf(__builtin_fmaf(e, r, q0)) + 128.0f;
        }
    }
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) lo = __builtin_amdgcn_cvt_pk_u8_f32(n[j], j, lo);
#pragma unroll
    for (int j = 0; j < 4; ++j) hi = __builtin_amdgcn_cvt_pk_u8_f32(n[j + 4], j, hi);
    return u32x2{lo ^ 0x80808080u, hi ^ 0x80808080u};
}

template <int MB>
__global__ __launch_bounds__(DEC_THREADS) void k_decode_mixed(const uint16_t* __restrict__ X, int M, int K,
                                                              const int8_t* __restrict__ Wq,
                                                              const float* __restrict__ s_w,
                                                              const uint16_t* __restrict__ W16, int64_t N, float tau,
                                                              void* __restrict__ out, int out_dtype,
                                                              DecodeStages st) {
    __shared__ __attribute__((aligned(16))) int8_t aq[MB * DEC_LDA];
    __shared__ int32_t oidx[DEC_MAXK];
    __shared__ int32_t red[DEC_WAVES][256];
    __shared__ float xo[DEC_OCAP][16];       // outlier activations  [h][m]
    __shared__ float wo[DEC_OCAP][16];       // outlier weights w~   [h][channel]
    __shared__ uint32_t rmax[DEC_WAVES][MB];
    __shared__ float sx_s[16];
    __shared__ __attribute__((aligned(16))) int wtot[DEC_WAVES];

    const int t = threadIdx.x, lane = t & 63, wave = wave_id();
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    const int S = K >> 6;                             // 64-byte MFMA steps in K
    const int nch = K >> 3;                           // 8-column chunks of X
    const bool own = t < nch;

    // 1a. X chunk t of every token (tokens past M read zeros)
    const rsrc_t rsx = make_rsrc(X, (int64_t)M * K * 2);
    u32x4 xv[MB];
#pragma unroll
    for (int m = 0; m < MB; ++m) xv[m] = bload16(rsx, own ? (uint32_t)(m * K + 8 * t) * 2 : kOOB);
    // 1b. scale of channel n0 + t % 16 (outlier gather and epilogue), ahead of
    //     the weight stream so that nothing in the prologue waits for the latter
    const rsrc_t rsn = make_rsrc(s_w + n0, (N - n0) * 4);
    const float swg = __builtin_bit_cast(float, bload4(rsn, (uint32_t)(t & 15) * 4));
    // Every wave has issued its X loads before any wave issues weight loads,
    // so the X requests are not queued behind weight traffic (no wait here).
    __builtin_amdgcn_s_barrier();
    // 1c. the weight slice: row n0 + lane % 16, bytes 64 s + 16 (lane / 16) of step s = wave + 8 j
    v4i wv[DEC_MAXSTEPS];
    const rsrc_t rsw = make_rsrc(Wq + n0 * K, (N - n0) * K);       // channels past N read zeros
    {
        const uint32_t wo0 = (uint32_t)((lane & 15) * K + 16 * (lane >> 4));
#pragma unroll
        for (int j = 0; j < DEC_MAXSTEPS; ++j) {
            const int s = wave + DEC_WAVES * j;
            wv[j] = __builtin_bit_cast(v4i, bload16(rsw, s < S ? wo0 + 64 * s : kOOB));
        }
    }

    // 2a. column max over the tokens on |x| bit patterns (fp16 magnitudes order
    //     like their bits), outlier flags of the chunk (8 bits), then the
    //     per-token absmax over the non-outlier columns.
    uint32_t cm[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int d = 0; d < 4; ++d) cm[d] = pk_max_u16(cm[d], xv[m][d] & 0x7fff7fffu);
    uint32_t flags = 0;
    uint32_t keep[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const bool olo = half_lo(cm[d]) > tau, ohi = half_hi(cm[d]) > tau;
        flags |= (olo ? 1u : 0u) << (2 * d);
        flags |= (ohi ? 1u : 0u) << (2 * d + 1);
        keep[d] = (olo ? 0u : 0xffffu) | (ohi ? 0u : 0xffff0000u);
    }
    flags = own ? flags : 0u;
    const u32x4 keepw = u32x4{keep[0], keep[1], keep[2], keep[3]};   // 0xffff per ordinary column
    {
        uint32_t mine = 0u;                           // lane m keeps token m's maximum
#pragma unroll
        for (int m = 0; m < MB; ++m) {
            uint32_t r = 0u;
#pragma unroll
            for (int d = 0; d < 4; ++d) r = pk_max_u16(r, xv[m][d] & 0x7fff7fffu & keep[d]);
            const uint32_t a = wave_max_all_u32(max(r & 0xffffu, r >> 16));
            mine = lane == m ? a : mine;
        }
        if (lane < MB) rmax[wave][lane] = mine;
    }

    float s_l = 1.0f, r_l = 1.0f;                     // lane m < MB: scale of token m, its reciprocal

    // 2b. ascending outlier list (block-wide exclusive scan over the chunks,
    //     the in-wave part from one ballot per flag bit); the owner of an
    //     outlier column also stages its activations.
    {
        int below = 0, wsum = 0;
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const uint64_t mb = __ballot((flags >> b) & 1u);
            below += bits_below(mb);
            wsum += __popcll(mb);
        }
        if (lane == 0) wtot[wave] = wsum;
        lds_barrier();

        // per-token scales: lane m < MB reduces token m over the waves
        // (every wave does, so no further barrier is needed)
        if (lane < MB) {
            uint32_t ab = 0u;
#pragma unroll
            for (int w = 0; w < DEC_WAVES; ++w) ab = max(ab, rmax[w][lane]);
            const float a = h2f((uint16_t)ab);
            s_l = a == 0.0f ? 1.0f : a / 127.0f;
            r_l = 1.0f / s_l;
            if (wave == 0) sx_s[lane] = s_l;
        }

        const int4 wt0 = *reinterpret_cast<const int4*>(wtot), wt1 = *reinterpret_cast<const int4*>(wtot + 4);
        const int wt[8] = {wt0.x, wt0.y, wt0.z, wt0.w, wt1.x, wt1.y, wt1.z, wt1.w};
        int off = below;
#pragma unroll
        for (int w = 0; w < DEC_WAVES; ++w) off += w < wave ? wt[w] : 0;
        uint32_t f = flags;
        while (f) {
            const int j = __builtin_ctz(f);
            f &= f - 1u;
            oidx[off] = 8 * t + j;
            if (off < DEC_OCAP) {
#pragma unroll
                for (int m = 0; m < MB; ++m) {
                    const uint32_t w32 = pick4(xv[m], j >> 1);
                    xo[off][m] = (j & 1) ? half_hi(w32) : half_lo(w32);
                }
            }
            ++off;
        }
    }
    int count = 0;
#pragma unroll
    for (int w = 0; w < DEC_WAVES; ++w) count += wtot[w];

    // 2c. int8 codes of X into LDS (outlier columns -> 0 -> code 0; tokens
    //     past M read zeros, have scale 1 and get codes 0, which no MFMA reads)
    if (own) {
#pragma unroll
        for (int m = 0; m < MB; ++m) {
            const float s = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s_l), m));
            const float r = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, r_l), m));
            *reinterpret_cast<u32x2*>(aq + m * DEC_LDA + 8 * t) = codes8_dec(xv[m] & keepw, s, r);
        }
    }
    lds_barrier();


    // 2d. start the gather of the outlier weights (first 64): the fp16 W[n][h]
    //     or the int8 code Wq[n][h], as the aligned 32-bit word holding it.
    //     The loads are unconditional (the descriptor is selected) and their
    //     values are used only after the MFMA, so no wait lands here.
    const int gch = t & 15, gh = t >> 4;              // channel n0 + gch, outlier slots gh + 32 q
    const rsrc_t rs16 = make_rsrc(W16 ? W16 + n0 * K : nullptr, W16 ? (N - n0) * K * 2 : 0);
    const rsrc_t rsg = W16 ? rs16 : rsw;
    constexpr int GQ = DEC_OCAP / (DEC_THREADS / 16);
    uint32_t graw[GQ], gsh[GQ];
#pragma unroll
    for (int q = 0; q < GQ; ++q) {
        const int h = gh + (DEC_THREADS / 16) * q;
        const uint32_t k = (uint32_t)oidx[h < count ? h : 0];
        const uint32_t e = (uint32_t)gch * K + k;     // element offset in the channel block
        const uint32_t b = W16 ? 2 * e : e;           // byte offset
        graw[q] = bload4(rsg, h < count ? (b & ~3u) : kOOB);
        gsh[q] = (b & 3u) * 8;
    }

    // 3a. int32 MFMA over this wave's K steps
    v4i acc = v4i{0, 0, 0, 0};
    const int arow = lane & 15;
#pragma unroll
    for (int j = 0; j < DEC_MAXSTEPS; ++j) {
        const int s = wave + DEC_WAVES * j;
        if (s < S) {
            v4i fa = v4i{0, 0, 0, 0};
            if (arow < M) fa = *reinterpret_cast<const v4i*>(aq + arow * DEC_LDA + 64 * s + 16 * (lane >> 4));
            acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa, wv[j], acc, 0, 0, 0);
        }
    }
    // acc: lane l, element e = token 4 (l / 16) + e, channel l % 16
#pragma unroll
    for (int e = 0; e < 4; ++e) red[wave][(4 * (lane >> 4) + e) * 16 + (lane & 15)] = acc[e];
#pragma unroll
    for (int q = 0; q < GQ; ++q) {
        const uint32_t v = graw[q] >> gsh[q];         // zero for an empty slot
        wo[gh + (DEC_THREADS / 16) * q][gch] = W16 ? h2f((uint16_t)v) : h2f(f2h(swg * (float)(int8_t)(uint8_t)v));
    }
    lds_barrier();

    // 3b. epilogue: thread t < 256 -> token m = t / 16, channel n0 + t % 16
    const int m = t >> 4, ch = t & 15;
    const int64_t n = n0 + ch;
    if (t < 256 && m < M && n < N) {
        int32_t c = 0;
#pragma unroll
        for (int w = 0; w < DEC_WAVES; ++w) c += red[w][t];
        float v = (float)c * sx_s[m] * swg;
        const int hs = count < DEC_OCAP ? count : DEC_OCAP;
        for (int h = 0; h < hs; ++h) v = v + xo[h][m] * wo[h][ch];
        for (int h = DEC_OCAP; h < count; ++h) {          // beyond the staged outliers
            const int k = oidx[h];
            const float wt = W16 ? h2f(W16[n * K + k]) : h2f(f2h(swg * (float)Wq[n * K + k]));
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

    // 4. workgroup 0 leaves the integer stages (outlier list, count, per-token
    //    scales, codes) where the general path keeps them
    if (blockIdx.x == 0) {
        for (int h = t; h < count; h += DEC_THREADS) st.idx[h] = oidx[h];
        if (t == 0) *st.count = count;
        if (t < M) st.s_x[t] = sx_s[t];
        const int cpr = K >> 4;                       // 16-byte chunks per row
        for (int c = t; c < M * cpr; c += DEC_THREADS) {
            const int r = c / cpr, j = c - r * cpr;
            *reinterpret_cast<v4i*>(st.xq + (int64_t)r * K + 16 * j) =
                *reinterpret_cast<const v4i*>(aq + r * DEC_LDA + 16 * j);
        }
    }
}

bool decode_supported(int64_t M, int64_t K) {
    return M >= 1 && M <= 16 && K >= 256 && K <= DEC_MAXK && K % 256 == 0;
}

hipError_t launch_decode_mixed(const uint16_t* X, int64_t M, int64_t K, const int8_t* Wq, const float* s_w,
                               const uint16_t* W16, int64_t N, float tau, void* out, int out_dtype,
                               const DecodeStages& stages, hipStream_t st) {
    const dim3 grid((unsigned)((N + 15) / 16)), block(DEC_THREADS);
    if (M <= 4)
        hipLaunchKernelGGL(k_decode_mixed<4>, grid, block, 0, st, X, (int)M, (int)K, Wq, s_w, W16, N, tau, out,
                           out_dtype, stages);
    else if (M <= 8)
        hipLaunchKernelGGL(k_decode_mixed<8>, grid, block, 0, st, X, (int)M, (int)K, Wq, s_w, W16, N, tau, out,
                           out_dtype, stages);
    else
        hipLaunchKernelGGL(k_decode_mixed<16>, grid, block, 0, st, X, (int)M, (int)K, Wq, s_w, W16, N, tau, out,
                           out_dtype, stages);
    return hipGetLastError();
}

}  // namespace qa
