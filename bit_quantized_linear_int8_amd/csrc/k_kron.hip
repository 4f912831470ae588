// k_kron.hip -- FlatQuant's Kronecker affine transform fused with int4
// quantization and packing, on gfx950.
//
// Source: AIInfra 05Quantization01 (模型量化), FlatQuant section: each token x
// (n = n1 n2 features) is reshaped to X~ [n1 x n2] and transformed as
// X~ x1 P1^T x2 P2 with P = P1 (x) P2, i.e. X' = P1^T X~ P2 = x (P1 (x) P2);
// the transformed activation is quantized to int4 per token in the same
// kernel, and the offline weight goes through the same transform (with
// P1^-T, P2^-T) and per-group int4 quantization.
//
// Arithmetic (bit-exact with a plain CPU evaluation): mode 1 first,
//   Y[a][j]  = fma-chain over i = 0 .. n1-1 of P1[i][a] * X~[i][j]   (from 0)
//   X'[a][b] = fma-chain over j = 0 .. n2-1 of Y[a][j] * P2[j][b]
// in fp32, each output one sequential chain of fused multiply-adds; then
// s = fl32(absmax / q_max) (per token or per G-wide group of the row, 1.0 if
// 0) and code = clip(rint(fl32(x' / s)), q_min, q_max), packed eight per word.
// The chains stay sequential (no split of the contraction), so the work is
// VALU fp32: 2 n1 n2 (n1 + n2) flops per token.
//
// Layout: a workgroup owns TB tokens; P1, P2 (fp32), each token's X~ (fp16)
// and an fp32 buffer per token (Y transposed, then X') live in LDS.  Thread
// lt of a token computes an R x R output block in each stage (R x R
// independent chains, 2R LDS reads per R^2 fused multiply-adds).
#include "qa_device.hpp"
#include "qa_launch.hpp"

namespace qa {

template <int N1, int N2, int R, int TB>
struct KronCfg {
    static constexpr int N = N1 * N2;
    static constexpr int TT = N / (R * R);          // threads per token
    static constexpr int THREADS = TB * TT;
    static constexpr int NCH = N / 8;                // 8-element chunks per token
    static_assert(N1 % R == 0 && N2 % R == 0 && R % 2 == 0, "block shape");
    static_assert(THREADS % 64 == 0 && THREADS <= 1024, "whole waves");
    static_assert(NCH % TT == 0, "chunks per thread");
    static constexpr size_t LDS = 4 * (N1 * N1 + N2 * N2) + (size_t)TB * N * 6;
    static_assert(LDS <= 160 * 1024, "LDS");
};

// Maximum over the TT threads of one token (TT lanes aligned in a wave when
// TT <= 64, else TT / 64 whole waves combined through LDS).
template <int TT>
__device__ __forceinline__ float token_max(float v, float* red) {
    if constexpr (TT <= 64) {
        return group_max(v, TT);
    } else {
        v = wave_max(v);
        const int w = threadIdx.x >> 6;
        if ((threadIdx.x & 63) == 0) red[w] = v;
        __syncthreads();
        const int w0 = w / (TT / 64) * (TT / 64);
        float m = red[w0];
#pragma unroll
        for (int i = 1; i < TT / 64; ++i) m = fmaxf(m, red[w0 + i]);
        return m;
    }
}

template <int N1, int N2, int R, int TB>
__global__ __launch_bounds__((KronCfg<N1, N2, R, TB>::THREADS)) void k_kron_quant4(
    const uint16_t* __restrict__ X, int64_t rows, const float* __restrict__ P1, const float* __restrict__ P2, int G,
    int qmin, int qmax, uint32_t* __restrict__ packed, float* __restrict__ s_out) {
    using C = KronCfg<N1, N2, R, TB>;
    constexpr int N = C::N, TT = C::TT;
    __shared__ __attribute__((aligned(16))) float p1[N1 * N1];
    __shared__ __attribute__((aligned(16))) float p2[N2 * N2];
    __shared__ __attribute__((aligned(16))) uint16_t xs[TB][N];
    __shared__ __attribute__((aligned(16))) float ys[TB][N];
    __shared__ float red[C::THREADS / 64];
    const int t = threadIdx.x, tok = t / TT, lt = t % TT;
    const int64_t row = (int64_t)blockIdx.x * TB + tok;
    {
        const rsrc_t r1 = make_rsrc(P1, N1 * N1 * 4), r2 = make_rsrc(P2, N2 * N2 * 4);
        for (int i = t; i < N1 * N1 / 4; i += C::THREADS)
            reinterpret_cast<u32x4*>(p1)[i] = bload16(r1, (uint32_t)i * 16);
        for (int i = t; i < N2 * N2 / 4; i += C::THREADS)
            reinterpret_cast<u32x4*>(p2)[i] = bload16(r2, (uint32_t)i * 16);
        const rsrc_t rx = make_rsrc(X + (row < rows ? row : 0) * N, row < rows ? N * 2 : 0);
#pragma unroll
        for (int c = lt; c < C::NCH; c += TT)
            reinterpret_cast<u32x4*>(xs[tok])[c] = bload16(rx, (uint32_t)c * 16);
    }
    __syncthreads();
    // stage 1: Y = P1^T X~, block (a0.., j0..); stored transposed: ys[j][a]
    const int a0 = (lt / (N2 / R)) * R, c0 = (lt % (N2 / R)) * R;
    {
        float acc[R][R];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int c = 0; c < R; ++c) acc[r][c] = 0.0f;
        for (int i = 0; i < N1; ++i) {
            float pa[R], xj[R];
#pragma unroll
            for (int r = 0; r < R; ++r) pa[r] = p1[i * N1 + a0 + r];
#pragma unroll
            for (int c = 0; c < R; ++c) xj[c] = h2f(xs[tok][i * N2 + c0 + c]);
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int c = 0; c < R; ++c) acc[r][c] = __builtin_fmaf(pa[r], xj[c], acc[r][c]);
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int c = 0; c < R; ++c) ys[tok][(c0 + c) * N1 + a0 + r] = acc[r][c];
    }
    __syncthreads();
    // stage 2: X' = Y P2, block (a0.., b0 = c0..)
    float o[R][R];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < R; ++c) o[r][c] = 0.0f;
    for (int j = 0; j < N2; ++j) {
        float ya[R], pb[R];
#pragma unroll
        for (int r = 0; r < R; ++r) ya[r] = ys[tok][j * N1 + a0 + r];
#pragma unroll
        for (int c = 0; c < R; ++c) pb[c] = p2[j * N2 + c0 + c];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int c = 0; c < R; ++c) o[r][c] = __builtin_fmaf(ya[r], pb[c], o[r][c]);
    }
    __syncthreads();                                     // every read of Y is done
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < R; ++c) ys[tok][(a0 + r) * N2 + c0 + c] = o[r][c];
    __syncthreads();
    // int4 codes: thread lt owns chunks lt + TT u (8 consecutive elements each)
    constexpr int U = C::NCH / TT;
    float xv[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) xv[u][e] = ys[tok][(lt + TT * u) * 8 + e];
    uint32_t* pr = packed + row * (N / 8);
    if (G == 0) {
        float amax = 0.0f;
#pragma unroll
        for (int u = 0; u < U; ++u) amax = fmaxf(amax, absmax8f(xv[u]));
        amax = token_max<TT>(amax, red);
        const float s = amax == 0.0f ? 1.0f : amax / (float)qmax;
        const float rs = 1.0f / s;
        if (row < rows) {
            if (lt == 0) s_out[row] = s;
#pragma unroll
            for (int u = 0; u < U; ++u) pr[lt + TT * u] = pack_codes(xv[u], s, rs, qmin);
        }
    } else {
        // a G-wide group is G / 8 consecutive chunks: aligned lanes of one u
        const int ng = N / G;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float amax = group_max(absmax8f(xv[u]), G / 8);
            const float s = amax == 0.0f ? 1.0f : amax / (float)qmax;
            const float rs = 1.0f / s;
            const int ch = lt + TT * u;
            if (row < rows) {
                if (ch % (G / 8) == 0) s_out[row * ng + ch / (G / 8)] = s;
                pr[ch] = pack_codes(xv[u], s, rs, qmin);
            }
        }
    }
}

// (n1, n2) pairs with a kernel, and the G values each supports per group.
template <int N1, int N2, int R, int TB>
static bool kron_try(int n1, int n2, const uint16_t* X, int64_t rows, const float* P1, const float* P2, int G,
                     int qmin, int qmax, uint32_t* packed, float* s, hipStream_t st, bool* ok) {
    if (n1 != N1 || n2 != N2) return false;
    using C = KronCfg<N1, N2, R, TB>;
    if (G != 0 && (G % 8 != 0 || G / 8 > C::TT || G / 8 > 64 || (N1 * N2) % G != 0)) {
        *ok = false;
        return true;
    }
    hipLaunchKernelGGL((k_kron_quant4<N1, N2, R, TB>), dim3((unsigned)((rows + TB - 1) / TB)), dim3(C::THREADS), 0,
                       st, X, rows, P1, P2, G, qmin, qmax, packed, s);
    *ok = true;
    return true;
}

bool kron_supported(int64_t n1, int64_t n2, int G) {
    auto gok = [&](int tt) { return G == 0 || (G % 8 == 0 && G / 8 <= tt && G / 8 <= 64 && (n1 * n2) % G == 0); };
    if (n1 == 8 && n2 == 8) return gok(KronCfg<8, 8, 4, 16>::TT);
    if (n1 == 8 && n2 == 16) return gok(KronCfg<8, 16, 4, 8>::TT);
    if (n1 == 16 && n2 == 16) return gok(KronCfg<16, 16, 4, 16>::TT);
    if (n1 == 16 && n2 == 32) return gok(KronCfg<16, 32, 4, 8>::TT);
    if (n1 == 32 && n2 == 32) return gok(KronCfg<32, 32, 4, 4>::TT);
    if (n1 == 32 && n2 == 64) return gok(KronCfg<32, 64, 4, 2>::TT);
    if (n1 == 64 && n2 == 64) return gok(KronCfg<64, 64, 8, 4>::TT);
    if (n1 == 64 && n2 == 128) return gok(KronCfg<64, 128, 8, 1>::TT);
    return false;
}

hipError_t launch_kron_quant_i4(const uint16_t* X, int64_t rows, int64_t n1, int64_t n2, const float* P1,
                                const float* P2, int G, int qmin, int qmax, uint32_t* packed, float* s,
                                hipStream_t st) {
    bool ok = false;
    const int a = (int)n1, b = (int)n2;
    kron_try<8, 8, 4, 16>(a, b, X, rows, P1, P2, G, qmin, qmax, packed, s, st, &ok) ||
        kron_try<8, 16, 4, 8>(a, b, X, rows, P1, P2, G, qmin, qmax, packed, s, st, &ok) ||
        kron_try<16, 16, 4, 16>(a, b, X, rows, P1, P2, G, qmin, qmax, packed, s, st, &ok) ||
        kron_try<16, 32, 4, 8>(a, b, X, rows, P1, P2, G, qmin, qmax, packed, s, st, &ok) ||
        kron_try<32, 32, 4, 4>(a, b, X, rows, P1, P2, G, qmin, qmax, packed, s, st, &ok) ||
        kron_try<32, 64, 4, 2>(a, b, X, rows, P1, P2, G, qmin, qmax, packed, s, st, &ok) ||
        kron_try<64, 64, 8, 4>(a, b, X, rows, P1, P2, G, qmin, qmax, packed, s, st, &ok) ||
        kron_try<64, 128, 8, 1>(a, b, X, rows, P1, P2, G, qmin, qmax, packed, s, st, &ok);
    return ok ? hipGetLastError() : hipErrorInvalidValue;
}

}  // namespace qa
