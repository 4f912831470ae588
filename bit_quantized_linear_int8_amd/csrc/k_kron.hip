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
// Layout: a workgroup owns TB tokens; P1, P2 (fp32) and one fp32 buffer per
// token live in LDS.  The buffer holds X~ (widened once), then Y (stored
// transposed), then X'; each stage's results wait in registers across the
// barrier before they overwrite it.  Thread lt of a token computes an R x R
// output block in each stage (R x R independent chains, 2R LDS reads per R^2
// fused multiply-adds), with the contraction loop unrolled so the next steps'
// reads are in flight during the current step's arithmetic.
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
    static constexpr size_t LDS = 4 * (N1 * N1 + N2 * N2) + (size_t)TB * N * 4;
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
        constexpr int U0 = C::NCH / TT;
        u32x4 v[U0];
#pragma unroll
        for (int u = 0; u < U0; ++u) v[u] = bload16(rx, (uint32_t)(lt + TT * u) * 16);
#pragma unroll
        for (int u = 0; u < U0; ++u) {
            float x[8];
            unpack8(v[u], x);
            float* d = &ys[tok][(lt + TT * u) * 8];
            *reinterpret_cast<v4f*>(d) = v4f{x[0], x[1], x[2], x[3]};
            *reinterpret_cast<v4f*>(d + 4) = v4f{x[4], x[5], x[6], x[7]};
        }
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
#pragma unroll 4
        for (int i = 0; i < N1; ++i) {
            float pa[R], xj[R];
#pragma unroll
            for (int r = 0; r < R; ++r) pa[r] = p1[i * N1 + a0 + r];
#pragma unroll
            for (int c = 0; c < R; ++c) xj[c] = ys[tok][i * N2 + c0 + c];
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int c = 0; c < R; ++c) acc[r][c] = __builtin_fmaf(pa[r], xj[c], acc[r][c]);
        }
        __syncthreads();                                 // every read of X~ is done
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
#pragma unroll 4
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

// ---------------------------------------------------------------------------
// n1 = 64 (n2 = 64 or 128): register-blocked outer products with the shared
// factor on the scalar path.  A 512-thread block owns TB = 512 / n2 tokens in
// one fp32 LDS buffer each (X~, then Y stored j-major, then X').
//   Stage 1: wave w owns rows a0 = 8w of Y for every token; lane l owns token
//     l / (n2/8) and the columns 4q .. 4q+3 and n2/2 + 4q .. +3, q = l % (n2/8)
//     (eight lanes then read 128 contiguous bytes: no LDS bank conflict); per
//     step i the eight
//     P1[i][a0..a0+7] are wave-uniform (scalar loads, 32 bytes) and the eight
//     X~[i][j0..j0+7] come from LDS: 64 fused multiply-adds per 8 LDS floats.
//   Stage 2: wave w owns columns b0 = RB w of X' (RB = n2 / 8); lane l owns
//     token l / (64/RA) and RA = 64 / RB rows (RA = 8: rows 4q .. 4q+3 and
//     32 + 4q .. +3; RA = 4: rows 4q .. 4q+3, q = l % (64/RA)), so the 64
//     lanes cover TB tokens x 64 rows; per step j, RB wave-uniform P2[j][b0..]
//     and RA values Y[a..][j] from LDS.
// With n2 = 64 the factor rows come from a 16 KB LDS copy (P1, then P2 in the
// same place) as broadcast reads instead: scalar loads may return out of
// order, so every wait for one drains all of them and nothing can be fetched
// ahead, while LDS reads complete in order.  (n2 = 128 keeps the scalar path:
// its P2 does not fit beside the token buffers.)  The 64-wide transposes
// through LDS (Y j-major, X' row-major) XOR each row's 16-byte units with
// (row / 4) mod 8, so the eight lanes that write rows four apart, and the
// lanes that read them back, hit distinct banks.
// Every output is still one chain over the contraction index in ascending
// order, the same arithmetic as k_kron_quant4.
// ---------------------------------------------------------------------------
template <int N2>
struct Kron64 {
    static constexpr int N1 = 64, N = N1 * N2, TB = 512 / N2, TS = N + 4;   // token stride (bank shift)
    static constexpr int JB = N2 / 8;                                        // stage-1 column blocks
    static constexpr int RB = N2 / 8;                                        // stage-2 columns per wave
    static constexpr int RA = 8 * 8 / RB;                                    // stage-2 rows per lane
    static constexpr int TT = 512 / TB;                                      // quantizer threads per token
    static constexpr int U = N / 8 / TT;                                     // chunks per quantizer thread
    static constexpr bool PLDS = N2 == 64;                                   // factors from LDS
    static_assert(TB * JB == 64 && TB * (64 / RA) == 64, "lane maps");
};

template <int N2>
__global__ __launch_bounds__(512) void k_kron64_quant4(const uint16_t* __restrict__ X, int64_t rows,
                                                       const float* __restrict__ P1, const float* __restrict__ P2,
                                                       int G, int qmin, int qmax, uint32_t* __restrict__ packed,
                                                       float* __restrict__ s_out) {
    using C = Kron64<N2>;
    constexpr int N = C::N, TS = C::TS, TB = C::TB, RA = C::RA, RB = C::RB, TT = C::TT, U = C::U;
    __shared__ __attribute__((aligned(16))) float buf[TB * TS];
    __shared__ float red[8];
    const int t = threadIdx.x, lane = t & 63, wave = wave_id();
    __shared__ __attribute__((aligned(16))) float pl[C::PLDS ? 64 * 64 : 4];
    auto load_factor = [&](const float* P) {
        const rsrc_t rp = make_rsrc(P, 64 * 64 * 4);
#pragma unroll
        for (int u = 0; u < 2; ++u)
            reinterpret_cast<u32x4*>(pl)[t + 512 * u] = bload16(rp, (uint32_t)(t + 512 * u) * 16);
    };
    // swizzled position of element (row, col) of a 64-wide row-major array
    auto sw = [](int rw, int col) { return rw * 64 + (col ^ (4 * ((rw >> 2) & 7))); };
    const int64_t row0 = (int64_t)blockIdx.x * TB;
    {
        // X~ of the block's tokens, widened: thread t loads chunks t + 512 u
        const int64_t nrow = rows - row0 < TB ? rows - row0 : TB;
        const rsrc_t rx = make_rsrc(X + row0 * N, nrow * N * 2);
        constexpr int UL = TB * N / 8 / 512;
        u32x4 v[UL];
#pragma unroll
        for (int u = 0; u < UL; ++u) v[u] = bload16(rx, (uint32_t)(t + 512 * u) * 16);
#pragma unroll
        for (int u = 0; u < UL; ++u) {
            const int e0 = (t + 512 * u) * 8, tok = e0 / N, e = e0 % N;
            float x[8];
            unpack8(v[u], x);
            float* d = buf + tok * TS + e;
            *reinterpret_cast<v4f*>(d) = v4f{x[0], x[1], x[2], x[3]};
            *reinterpret_cast<v4f*>(d + 4) = v4f{x[4], x[5], x[6], x[7]};
        }
        if constexpr (C::PLDS) load_factor(P1);
    }
    __syncthreads();
    // stage 1
    {
        const int a0 = 8 * wave, tok = lane / C::JB, j0 = 4 * (lane % C::JB), j1 = j0 + N2 / 2;
        const float* xb = buf + tok * TS;
        float acc[8][8];
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[r][c] = 0.0f;
#pragma unroll 4
        for (int i = 0; i < 64; ++i) {
            float p[8], x[8];
            if constexpr (C::PLDS) {
                const v4f q0 = *reinterpret_cast<const v4f*>(pl + i * 64 + a0);
                const v4f q1 = *reinterpret_cast<const v4f*>(pl + i * 64 + a0 + 4);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    p[r] = q0[r];
                    p[r + 4] = q1[r];
                }
            } else {
                const float* p1r = P1 + i * 64 + a0;         // wave-uniform: scalar loads
#pragma unroll
                for (int r = 0; r < 8; ++r) p[r] = p1r[r];
            }
            const v4f x0 = *reinterpret_cast<const v4f*>(xb + i * N2 + j0);
            const v4f x1 = *reinterpret_cast<const v4f*>(xb + i * N2 + j1);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                x[c] = x0[c];
                x[c + 4] = x1[c];
            }
#pragma unroll
            for (int r = 0; r < 8; ++r)
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[r][c] = __builtin_fmaf(p[r], x[c], acc[r][c]);
        }
        __syncthreads();                                     // every read of X~ (and of P1) is done
        if constexpr (C::PLDS) load_factor(P2);
        // Y j-major, swizzled: Y[a][j] at sw(j, a)
        float* yb = buf + tok * TS;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int jr = c < 4 ? j0 + c : j1 + c - 4;
            *reinterpret_cast<v4f*>(yb + sw(jr, a0)) = v4f{acc[0][c], acc[1][c], acc[2][c], acc[3][c]};
            *reinterpret_cast<v4f*>(yb + sw(jr, a0 + 4)) = v4f{acc[4][c], acc[5][c], acc[6][c], acc[7][c]};
        }
    }
    __syncthreads();
    // stage 2
    {
        const int b0 = RB * wave, tok = lane / (64 / RA), q = lane % (64 / RA);
        // row r of this lane's block: 4q + r (r < 4), 32 + 4q + r - 4 (RA = 8)
        auto arow = [&](int r) { return r < 4 ? 4 * q + r : 32 + 4 * q + r - 4; };
        const float* yb = buf + tok * TS;
        float o[RA][RB];
#pragma unroll
        for (int r = 0; r < RA; ++r)
#pragma unroll
            for (int c = 0; c < RB; ++c) o[r][c] = 0.0f;
#pragma unroll 4
        for (int j = 0; j < N2; ++j) {
            float p[RB], y[RA];
            if constexpr (C::PLDS) {
#pragma unroll
                for (int c = 0; c < RB; c += 4) {
                    const v4f q = *reinterpret_cast<const v4f*>(pl + j * N2 + b0 + c);
#pragma unroll
                    for (int e = 0; e < 4; ++e) p[c + e] = q[e];
                }
            } else {
                const float* p2r = P2 + j * N2 + b0;         // wave-uniform: scalar loads
#pragma unroll
                for (int c = 0; c < RB; ++c) p[c] = p2r[c];
            }
#pragma unroll
            for (int r = 0; r < RA; r += 4) {
                const v4f yv = *reinterpret_cast<const v4f*>(yb + sw(j, arow(r)));
#pragma unroll
                for (int e = 0; e < 4; ++e) y[r + e] = yv[e];
            }
#pragma unroll
            for (int r = 0; r < RA; ++r)
#pragma unroll
                for (int c = 0; c < RB; ++c) o[r][c] = __builtin_fmaf(y[r], p[c], o[r][c]);
        }
        __syncthreads();                                     // every read of Y is done
        float* xb = buf + tok * TS;
#pragma unroll
        for (int r = 0; r < RA; ++r)
#pragma unroll
            for (int c = 0; c < RB; c += 4)
                *reinterpret_cast<v4f*>(xb + (N2 == 64 ? sw(arow(r), b0 + c) : arow(r) * N2 + b0 + c)) =
                    v4f{o[r][c], o[r][c + 1], o[r][c + 2], o[r][c + 3]};
    }
    __syncthreads();
    // int4 codes: TT threads per token, thread lt owns chunks lt + TT u
    const int tok = t / TT, lt = t % TT;
    const int64_t row = row0 + tok;
    float xv[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int e0 = (lt + TT * u) * 8;                    // X' row-major (swizzled when 64 wide)
        const float* tb = buf + tok * TS;
        const v4f v0 = *reinterpret_cast<const v4f*>(tb + (N2 == 64 ? sw(e0 >> 6, e0 & 63) : e0));
        const v4f v1 = *reinterpret_cast<const v4f*>(tb + (N2 == 64 ? sw(e0 >> 6, (e0 & 63) + 4) : e0 + 4));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            xv[u][e] = v0[e];
            xv[u][e + 4] = v1[e];
        }
    }
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
    if (n1 == 64 && (n2 == 64 || n2 == 128)) return gok(n2 == 64 ? Kron64<64>::TT : Kron64<128>::TT);
    return false;
}

hipError_t launch_kron_quant_i4(const uint16_t* X, int64_t rows, int64_t n1, int64_t n2, const float* P1,
                                const float* P2, int G, int qmin, int qmax, uint32_t* packed, float* s,
                                hipStream_t st) {
    if (n1 == 64 && n2 == 64) {
        hipLaunchKernelGGL(k_kron64_quant4<64>, dim3((unsigned)((rows + Kron64<64>::TB - 1) / Kron64<64>::TB)),
                           dim3(512), 0, st, X, rows, P1, P2, G, qmin, qmax, packed, s);
        return hipGetLastError();
    }
    if (n1 == 64 && n2 == 128) {
        hipLaunchKernelGGL(k_kron64_quant4<128>, dim3((unsigned)((rows + Kron64<128>::TB - 1) / Kron64<128>::TB)),
                           dim3(512), 0, st, X, rows, P1, P2, G, qmin, qmax, packed, s);
        return hipGetLastError();
    }
    bool ok = false;
    const int a = (int)n1, b = (int)n2;
    kron_try<8, 8, 4, 16>(a, b, X, rows, P1, P2, G, qmin, qmax, packed, s, st, &ok) ||
        kron_try<8, 16, 4, 8>(a, b, X, rows, P1, P2, G, qmin, qmax, packed, s, st, &ok) ||
        kron_try<16, 16, 4, 16>(a, b, X, rows, P1, P2, G, qmin, qmax, packed, s, st, &ok) ||
        kron_try<16, 32, 4, 8>(a, b, X, rows, P1, P2, G, qmin, qmax, packed, s, st, &ok) ||
        kron_try<32, 32, 4, 4>(a, b, X, rows, P1, P2, G, qmin, qmax, packed, s, st, &ok) ||
        kron_try<32, 64, 4, 2>(a, b, X, rows, P1, P2, G, qmin, qmax, packed, s, st, &ok);
    return ok ? hipGetLastError() : hipErrorInvalidValue;
}

}  // namespace qa
