// k_decode.hip -- the LLM.int8() mixed linear for decode shapes (M <= 16
// tokens) as one fused kernel on gfx950.
//
// Decode is bound by streaming the int8 weight from HBM; the activation is a
// few KB.  Every workgroup owns 16 output channels and has eight waves; wave w
// multiplies the 64-byte K steps w, w + 8, w + 16, ... so each weight load
// instruction of the block covers 16 rows x 512 contiguous bytes.  A workgroup
//   1. loads X (thread t owns the 8-column chunks t and t + 512 of every
//      token) and the scale of the channel it writes in the epilogue; once
//      every X request of the block has been issued, the weight waves issue
//      ALL of their weight loads (directly in the B-operand layout of
//      v_mfma_i32_16x16x64_i8, 16 bytes per lane and step).  Issued behind
//      the weight requests, the X requests (hits on lines every workgroup
//      reads) queue behind weight misses in the caches and arrive about
//      1.5 us later; issued first, they keep their place ahead of the weight
//      stream, and the stream need not wait for them to arrive;
//   2. while the weight bytes are in flight, recomputes -- identically in every
//      workgroup -- the outlier columns (column max over the tokens on the
//      sign-cleared fp16 bit patterns, compared as integers with a threshold
//      pattern), the per-token maxima over the other columns (a reduce-scatter
//      over the lanes), the per-token scales, the ascending outlier list and
//      the fp16 outlier activations, and the int8 codes of X into LDS (the A
//      operand); then starts the gather of the fp16 outlier weights,
//   3. multiplies its K steps on the MFMA, sums the eight int32 partial tiles
//      in LDS, dequantizes by s_x[m] * s_w[n] and adds the outlier product.
// Its barriers wait only for LDS traffic, so the weight stream stays in
// flight across them.
//
// SmoothQuant mode (SM = 1 per-token, 2 per-tensor scales): no outlier
// columns; step 2 instead divides every value by its column's migration
// factor (IEEE fp32 division, as the separate smoothing quantizer does),
// takes the per-token maxima of the smoothed values and codes them; the
// weight is the offline-smoothed int8 weight.
//
// Method: AIInfra 05Quantization01, LLM.int8(): outlier columns by magnitude
// threshold, "a. 向量级量化" (per-token / per-channel absmax scales),
// "b. INT8 矩阵乘法与反量化" (int32 accumulation, outer-product dequant) and
// the merge with the fp16 outlier product; Quantization explained part 2 §1.2;
// SmoothQuant: Quantization explained part 2 §4.2 (X / s by column), §4.4.
#include <cmath>
#include <cstring>

#include "qa_device.hpp"
#include "qa_launch.hpp"

namespace qa {

constexpr int DEC_WAVES = 8, DEC_THREADS = 64 * DEC_WAVES;
constexpr int DEC_CHUNK_K = 8 * DEC_THREADS;    // columns covered by one chunk per thread (4096)
constexpr int DEC_OCAP = 64;                    // outliers whose operands are staged in LDS
constexpr int DEC_OCAP_TOPK = 256;              // the same for the top-k set (k <= 256 takes this kernel)
static_assert(DEC_WAVES == 8, "the wave totals are read as two 16-byte vectors");

typedef unsigned short u16x2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t u32_of(u16x2v v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ u16x2v v_of(uint32_t v) { return __builtin_bit_cast(u16x2v, v); }

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

// Two 16-bit maxima per lane with the value of another lane (DPP move, then
// v_pk_max_u16; the packed max takes no DPP operand on gfx9).
template <int CTRL>
__device__ __forceinline__ uint32_t pkmax_dpp(uint32_t v) {
    return pk_max_u16(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false));
}

// Reduce-scatter of eight per-token values (two 16-bit maxima each) over the
// 64 lanes: on return lane L holds the wave-wide maximum of token L >> 3 (both
// halves, not yet combined).  Three halving steps -- v_permlane32_swap pairs
// tokens (m, m + 4), v_permlane16_swap pairs (0, 2) and (1, 3), a row_ror:8
// move pairs the last two -- then three DPP steps within groups of 8 lanes.
// 18 VALU instructions instead of 8 full wave reductions.
__device__ __forceinline__ uint32_t reduce_scatter8(const uint32_t* v) {
    uint32_t a[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {      // lanes 0-31: token m, lanes 32-63: token m + 4
        const auto p = __builtin_amdgcn_permlane32_swap(v[m], v[m + 4], false, false);
        a[m] = pk_max_u16(p[0], p[1]);
    }
    uint32_t b[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {      // rows 0..3: tokens m, m + 2, m + 4, m + 6
        const auto p = __builtin_amdgcn_permlane16_swap(a[m], a[m + 2], false, false);
        b[m] = pk_max_u16(p[0], p[1]);
    }
    const bool hi8 = (__lane_id() & 8) != 0;   // lanes with bit 3 set keep the odd tokens
    const uint32_t mine = hi8 ? b[1] : b[0], other = hi8 ? b[0] : b[1];
    uint32_t r = pk_max_u16(mine, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)other, 0x128, 0xF, 0xF, false));  // row_ror:8
    r = pkmax_dpp<0xB1>(r);            // quad_perm [1,0,3,2]
    r = pkmax_dpp<0x4E>(r);            // quad_perm [2,3,0,1]
    r = pkmax_dpp<0x141>(r);           // row_half_mirror
    return r;
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
// the test suite checks all 1.0e9 such pairs on the CPU.  The codes are
// returned biased by 128 (bytes rint + 128); the caller un-biases and masks.
__device__ __forceinline__ u32x2 codes8_biased(const u32x4& v, float s, float r) {
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
    return u32x2{lo, hi};
}

// Barrier over the eight activation waves only (the weight waves may be
// stalled issuing their loads): an LDS counter, set to zero before the first
// workgroup barrier, that every activation wave increments once its LDS
// writes are done, then waits for until it reaches `target` (8 times the
// number of such barriers passed so far, this one included).
__device__ __forceinline__ void activation_barrier(int* ctr, int lane, int target) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);      // this wave's LDS writes are done
    if (lane == 0) __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < target)
        __builtin_amdgcn_s_sleep(1);
    asm volatile("" ::: "memory");
}

// Inclusive sum over the 64 lanes: DPP row shifts within rows of 16, then
// the totals of the rows below (lanes 15, 31, 47) added by row.
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t v, int lane) {
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);   // row_shr:1
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);   // row_shr:2
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);   // row_shr:4
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);   // row_shr:8
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 15);
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 31);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 47);
    const int row = lane >> 4;
    return v + (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
}

// One radix digit of the k-th largest key: lane l holds the counts h[0..B-1]
// of digits D - B l, D - B l - 1, ... (descending from the top digit D); the
// digit holding the `rem`-th largest key (1 <= rem <= the total) and the
// number of keys in higher digits, plus that digit's count, the same in
// every lane.
template <int B>
__device__ __forceinline__ void pick_digit(const uint32_t* h, uint32_t rem, int top, int lane, uint32_t& digit,
                                           uint32_t& above_out, uint32_t& count_out) {
    uint32_t cs = 0u;
#pragma unroll
    for (int i = 0; i < B; ++i) cs += h[i];
    const uint32_t incl = wave_incl_sum(cs, lane);
    uint32_t above = incl - cs, dg = 0u, he = 0u;
    bool found = false;
#pragma unroll
    for (int i = 0; i < B; ++i) {
        if (!found && above + h[i] >= rem) {
            dg = (uint32_t)(top - B * lane - i);
            he = h[i];
            found = true;
        } else if (!found) {
            above += h[i];
        }
    }
    const int src = __builtin_ctzll(__ballot(incl - cs < rem && rem <= incl));
    digit = (uint32_t)__builtin_amdgcn_readlane((int)dg, src);
    above_out = (uint32_t)__builtin_amdgcn_readlane((int)above, src);
    count_out = (uint32_t)__builtin_amdgcn_readlane((int)he, src);
}

// The top-k flags of this thread's chunks (bit j of flags[c]: column
// 8 (t + 512 c) + j is taken) from its packed column-max keys cmx (chunks at
// or past nch hold no columns); called by every activation wave with the same
// k.  red and hist2 are [8][256] and cleared; nbar returns the target of the
// next activation barrier.
template <int CH>
__device__ __forceinline__ void topk_flags(const uint32_t (&cmx)[CH][4], uint32_t k, int nch, int t, int lane,
                                           int wave, int32_t* red, uint32_t* hist2, uint32_t* tie_tot, int* abar,
                                           uint32_t* flags, int& nbar) {
#pragma unroll
    for (int c = 0; c < CH; ++c) flags[c] = 0u;
    nbar = DEC_WAVES;
    if (k == 0) return;
    // high digit: bits 14..8 of the key (bit 15, the sign, is clear)
    uint32_t* h1 = reinterpret_cast<uint32_t*>(red) + 256 * wave + 128 * (lane & 1);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        if (t + DEC_THREADS * c < nch) {
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t v = cmx[c][d];
                __hip_atomic_fetch_add(h1 + ((v >> 8) & 0x7fu), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                __hip_atomic_fetch_add(h1 + (v >> 24), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            }
        }
    }
    activation_barrier(abar, lane, DEC_WAVES);
    uint32_t h[4];
    {
        uint32_t hh = 0u, hl = 0u;                    // digits 127 - 2 lane and 126 - 2 lane
#pragma unroll
        for (int w = 0; w < DEC_WAVES; ++w)
#pragma unroll
            for (int cp = 0; cp < 2; ++cp) {
                const uint32_t* q = reinterpret_cast<const uint32_t*>(red) + 256 * w + 128 * cp + 126 - 2 * lane;
                hl += q[0];
                hh += q[1];
            }
        h[0] = hh;
        h[1] = hl;
    }
    uint32_t d1, a1, n1;
    pick_digit<2>(h, k, 127, lane, d1, a1, n1);
    const uint32_t rem = k - a1;                      // keys still to take from digit d1: 1 <= rem <= n1
    // low digit over the keys in high digit d1
    uint32_t* h2 = hist2 + 256 * wave;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        if (t + DEC_THREADS * c < nch) {
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t v = cmx[c][d];
                if (((v >> 8) & 0x7fu) == d1)
                    __hip_atomic_fetch_add(h2 + (v & 0xffu), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                if ((v >> 24) == d1)
                    __hip_atomic_fetch_add(h2 + ((v >> 16) & 0xffu), 1u, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_WORKGROUP);
            }
        }
    }
    activation_barrier(abar, lane, 2 * DEC_WAVES);
    {
        u32x4 a = u32x4{0u, 0u, 0u, 0u};              // digits 252 - 4 lane .. 255 - 4 lane
#pragma unroll
        for (int w = 0; w < DEC_WAVES; ++w) a += *reinterpret_cast<const u32x4*>(hist2 + 256 * w + 252 - 4 * lane);
        h[0] = a[3];
        h[1] = a[2];
        h[2] = a[1];
        h[3] = a[0];
    }
    uint32_t d2, a2, neq;
    pick_digit<4>(h, rem, 255, lane, d2, a2, neq);
    const uint32_t kth = (d1 << 8) | d2, take = rem - a2;   // keys equal to kth: neq, of which take are taken
    uint32_t eq[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        uint32_t gt = 0u, e = 0u;
        if (t + DEC_THREADS * c < nch) {
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t lo = cmx[c][d] & 0xffffu, hi = cmx[c][d] >> 16;
                gt |= ((lo > kth ? 1u : 0u) | (hi > kth ? 2u : 0u)) << (2 * d);
                e |= ((lo == kth ? 1u : 0u) | (hi == kth ? 2u : 0u)) << (2 * d);
            }
        }
        flags[c] = gt;
        eq[c] = e;
    }
    nbar = 3 * DEC_WAVES;
    if (take == neq) {                                // every tie taken (the same branch in every wave)
#pragma unroll
        for (int c = 0; c < CH; ++c) flags[c] |= eq[c];
        return;
    }
    // ties split: rank the equal keys in column order (chunk set 0, then 1)
    uint32_t below[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const uint32_t n = (uint32_t)__builtin_popcount(eq[c]);
        const uint32_t incl = wave_incl_sum(n, lane);
        below[c] = incl - n;
        if (lane == 63) tie_tot[DEC_WAVES * c + wave] = incl;
    }
    activation_barrier(abar, lane, 3 * DEC_WAVES);
    nbar = 4 * DEC_WAVES;
    uint32_t base = 0u;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        uint32_t before = 0u, tot = 0u;
#pragma unroll
        for (int w = 0; w < DEC_WAVES; ++w) {
            const uint32_t x = tie_tot[DEC_WAVES * c + w];
            tot += x;
            before += w < wave ? x : 0u;
        }
        uint32_t r = base + before + below[c], e = eq[c];
        while (e) {
            const int b = __builtin_ctz(e);
            e &= e - 1u;
            if (r < take) flags[c] |= 1u << b;
            ++r;
        }
        base += tot;
    }
}

// MB: tokens per block (4, 8 or 16); CH: 8-column chunks per thread (K <= 4096 CH).
//
// Sixteen waves in two roles, two of each per SIMD.  Activation waves 0-7
// (threads t < 512) load X and compute everything that depends only on it;
// weight waves 8-15 issue the weight stream and run the MFMAs.  A wave that
// issues more loads than its compute unit can keep in flight stalls until
// earlier ones return -- about 2 us for this 64 KB per workgroup -- so the
// weight loads are issued by waves that have nothing else to do meanwhile.
//
// TOPK: the outlier set is the k = thr1 columns of largest column maximum
// (equal maxima: lower column first) instead of those above a threshold.  The
// activation waves find the k-th largest key (the sign-cleared fp16 pattern
// of the column maximum; patterns order like magnitudes) by a two-digit radix
// select -- per-wave histograms of the high byte in LDS (two copies by lane
// parity, fewer same-address atomics), the digit from a lane scan that every
// wave does itself, the same for the low byte over the keys in that high
// digit -- then take the keys above it and, in column order, as many keys
// equal to it as are still missing (a ballot scan over the ties, skipped
// when every tie is taken).
template <int MB, int CH, bool TOPK, int SM>
__global__ __launch_bounds__(2 * DEC_THREADS) void k_decode_mixed(const uint16_t* __restrict__ X, int M, int K,
                                                                  const int8_t* __restrict__ Wq,
                                                                  const float* __restrict__ s_w,
                                                                  const uint16_t* __restrict__ W16, int64_t N,
                                                                  uint32_t thr1, void* __restrict__ out,
                                                                  int out_dtype, DecodeStages st,
                                                                  const float* __restrict__ sm) {
    static_assert(SM == 0 || !TOPK, "SmoothQuant mode has no outlier set");
    // SmoothQuant: the smoothed values are held in registers from the maxima
    // to the codes when they fit (one chunk, at most 8 tokens); otherwise the
    // codes pass divides again (the same IEEE operation, the same values)
    constexpr bool HOLD = SM != 0 && CH == 1 && MB <= 8;
    constexpr int OCAP = TOPK ? DEC_OCAP_TOPK : DEC_OCAP;
    constexpr int MAXK = DEC_CHUNK_K * CH;
    constexpr int LDA = MAXK + 16;                  // LDS row stride of the codes (spreads banks)
    constexpr int STEPS = MAXK / 64 / DEC_WAVES;    // MFMA steps per weight wave
    constexpr int NG = MB > 8 ? 2 : 1;              // groups of eight tokens for the lane reductions
    __shared__ __attribute__((aligned(16))) int8_t aq[MB * LDA];
    __shared__ int16_t oidx[MAXK];
    __shared__ __attribute__((aligned(16))) int32_t red[DEC_WAVES][256];
    __shared__ float xo[OCAP][16];           // outlier activations  [h][m]
    __shared__ float wo[OCAP][16];           // outlier weights w~   [h][channel]
    __shared__ __attribute__((aligned(16))) uint32_t hist2[TOPK ? DEC_WAVES : 1][256];   // low-digit histograms
    __shared__ uint32_t tie_tot[TOPK ? CH : 1][DEC_WAVES];
    __shared__ __attribute__((aligned(16))) uint32_t rmax[16][DEC_WAVES];   // [token][activation wave]
    __shared__ float sx_s[16];
    __shared__ __attribute__((aligned(16))) int wtot[CH][DEC_WAVES];
    __shared__ int abar;
    __shared__ int count_s;

    const int lane = threadIdx.x & 63, wave = wave_id();
    const bool act = wave < DEC_WAVES;
    const int t = threadIdx.x & (DEC_THREADS - 1);    // index within the role
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    const int S = K >> 6;                             // 64-byte MFMA steps in K
    const int nch = K >> 3;                           // 8-column chunks of X
    const rsrc_t rsn = make_rsrc(s_w + n0, (N - n0) * 4);
    const float swg = __builtin_bit_cast(float, bload4(rsn, (uint32_t)(t & 15) * 4));   // scale of channel n0 + t % 16
    const rsrc_t rsw = make_rsrc(Wq + n0 * K, (N - n0) * K);       // channels past N read zeros
    // Read the arguments used only late (the second 64 bytes of the argument
    // block) into registers now: a scalar-cache miss after the weight stream
    // has started waits behind it in the memory queues.
    asm volatile("" ::"s"(out_dtype), "s"(st.idx), "s"(st.count), "s"(st.s_x), "s"(st.xq), "s"(out));
    (void)sm;
    if (threadIdx.x == 0) abar = 0;

    v4i acc = v4i{0, 0, 0, 0};
    int count = 0;
    if (act) {
        // ---------------------------------------------------------------- activation waves
        // 1. X chunks t + 512 c of every token (tokens past M and chunks past K read zeros)
        const rsrc_t rsx = make_rsrc(X, (int64_t)M * K * 2);
        u32x4 xv[CH][MB];
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int ch = t + DEC_THREADS * c;
#pragma unroll
            for (int m = 0; m < MB; ++m) xv[c][m] = bload16(rsx, ch < nch ? (uint32_t)(m * K + 8 * ch) * 2 : kOOB);
        }
        u32x4 fv[SM ? CH : 1][2];                     // SmoothQuant: the factors of each chunk's 8 columns
        if constexpr (SM != 0) {
            const rsrc_t rsf = make_rsrc(sm, (int64_t)K * 4);
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                const int ch = t + DEC_THREADS * c;
                fv[c][0] = bload16(rsf, ch < nch ? (uint32_t)ch * 32 : kOOB);
                fv[c][1] = bload16(rsf, ch < nch ? (uint32_t)ch * 32 + 16 : kOOB);
            }
        }
        if constexpr (TOPK) {   // clear the histograms (the high-digit ones live in red until the epilogue)
            reinterpret_cast<u32x4*>(&red[0][0])[t] = u32x4{0u, 0u, 0u, 0u};
            reinterpret_cast<u32x4*>(&hist2[0][0])[t] = u32x4{0u, 0u, 0u, 0u};
        }
        // the weight waves issue their stream once every X request is issued
        lds_barrier();                                                  // barrier 1
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        if constexpr (SM != 0) {
            // Pin the loaded X and factors here: the smoothing divisions are
            // plain arithmetic that the compiler otherwise hoists above barrier 1
            // (with the waits for X they need), which holds the weight waves
            // at that barrier until X has arrived.
#pragma unroll
            for (int c = 0; c < CH; ++c) {
#pragma unroll
                for (int m = 0; m < MB; ++m) asm volatile("" : "+v"(xv[c][m]));
                asm volatile("" : "+v"(fv[c][0]), "+v"(fv[c][1]));
            }
        }

        // 2a. column max over the tokens on |x| bit patterns (fp16 magnitudes
        //     order like their bits); column j is an outlier when that max is
        //     >= thr1 (the threshold as an fp16 pattern, see launch_decode_mixed).
        //     keep: 0xffff per ordinary column.  Then the per-token maxima over
        //     the ordinary columns, reduce-scattered over the lanes.
        uint32_t keep[CH][4];
        uint32_t flags[CH];
        uint32_t rm[NG * 8];
        int nbar = DEC_WAVES;                         // activation-barrier target of step 2b
#pragma unroll
        for (int m = 0; m < NG * 8; ++m) rm[m] = 0u;
        if constexpr (TOPK) {
            uint32_t cmx[CH][4];
#pragma unroll
            for (int c = 0; c < CH; ++c)
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    uint32_t a = 0u;
#pragma unroll
                    for (int m = 0; m < MB; ++m) a = pk_max_u16(a, xv[c][m][d] & 0x7fff7fffu);
                    cmx[c][d] = a;
                }
            topk_flags<CH>(cmx, thr1, nch, t, lane, wave, &red[0][0], &hist2[0][0], &tie_tot[0][0], &abar, flags,
                           nbar);
#pragma unroll
            for (int c = 0; c < CH; ++c)
#pragma unroll
                for (int d = 0; d < 4; ++d)
                    keep[c][d] = (((flags[c] >> (2 * d)) & 1u) ? 0u : 0xffffu) |
                                 (((flags[c] >> (2 * d + 1)) & 1u) ? 0u : 0xffff0000u);
        }
        const u16x2v T = u16x2v{(unsigned short)thr1, (unsigned short)thr1};
        // SmoothQuant: y = fl32(x / f) for the lane's chunks and every token (0
        // past the row), per-token maxima of |y| as bit patterns (non-negative
        // floats order like their bits), one wave reduction per token
        // (each factor element is copied to a scalar before its bit cast: a
        // bit cast of a vector-element expression read element 0 here)
        // Past the row X reads 0 and the divisor is taken as 1, so y = 0 there
        // with no branch: a division under a condition became a branch whose
        // X load the compiler sank past barrier 1, behind the weight stream.
        auto smooth_chunk = [&](int c, int m, float* y8) __attribute__((always_inline)) {
            const bool valid = t + DEC_THREADS * c < nch;
            float x[8];
            unpack8(xv[c][m], x);
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t f0 = fv[SM ? c : 0][0][d], f1 = fv[SM ? c : 0][1][d];
                y8[d] = x[d] / (valid ? __builtin_bit_cast(float, f0) : 1.0f);
                y8[d + 4] = x[d + 4] / (valid ? __builtin_bit_cast(float, f1) : 1.0f);
            }
        };
        float y[HOLD ? MB : 1][8];
        if constexpr (SM != 0) {
#pragma unroll
            for (int m = 0; m < MB; ++m) {
                uint32_t a = 0u;
#pragma unroll
                for (int c = 0; c < CH; ++c) {
                    float yt[8];
                    float* yc = HOLD ? y[HOLD ? m : 0] : yt;
                    smooth_chunk(c, m, yc);
#pragma unroll
                    for (int j = 0; j < 8; ++j) a = max(a, __builtin_bit_cast(uint32_t, yc[j]) & 0x7fffffffu);
                }
                a = wave_max_u32(a);
                if (lane == 0) rmax[m][wave] = a;
            }
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                flags[c] = 0u;
#pragma unroll
                for (int d = 0; d < 4; ++d) keep[c][d] = 0xffffffffu;
            }
        }
#pragma unroll
        for (int c = 0; c < (SM ? 0 : CH); ++c) {
            if constexpr (!TOPK) {
                uint32_t cm[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int m = 0; m < MB; ++m)
#pragma unroll
                    for (int d = 0; d < 4; ++d) cm[d] = pk_max_u16(cm[d], xv[c][m][d] & 0x7fff7fffu);
                uint32_t f = 0u;
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    // 1 per ordinary half (thr1 - cm > 0), 0 per outlier half
                    const u16x2v k1 = __builtin_elementwise_min(__builtin_elementwise_sub_sat(T, v_of(cm[d])),
                                                                u16x2v{1, 1});
                    keep[c][d] = u32_of(u16x2v{0, 0} - k1);
                    const uint32_t kb = u32_of(k1);
                    f |= ((kb & 1u) | ((kb >> 15) & 2u)) << (2 * d);
                }
                flags[c] = (t + DEC_THREADS * c < nch) ? (~f & 0xffu) : 0u;
            }
#pragma unroll
            for (int m = 0; m < MB; ++m) {
                const uint32_t r01 = pk_max_u16(xv[c][m][0] & 0x7fff7fffu & keep[c][0],
                                                xv[c][m][1] & 0x7fff7fffu & keep[c][1]);
                const uint32_t r23 = pk_max_u16(xv[c][m][2] & 0x7fff7fffu & keep[c][2],
                                                xv[c][m][3] & 0x7fff7fffu & keep[c][3]);
                rm[m] = pk_max_u16(rm[m], pk_max_u16(r01, r23));
            }
        }
#pragma unroll
        for (int g = 0; g < (SM ? 0 : NG); ++g) {
            const uint32_t r = reduce_scatter8(rm + 8 * g);
            const uint32_t a = max(r & 0xffffu, r >> 16);
            if ((lane & 7) == 0) rmax[8 * g + (lane >> 3)][wave] = a;
        }

        // 2b. ascending outlier list: the columns of chunk set 0 (chunks t) come
        //     before those of set 1 (chunks t + 512); within a set, an exclusive
        //     scan over the chunks, the in-wave part from one ballot per flag bit
        //     (skipped by waves without outlier columns).  The owner of an
        //     outlier column also stages its activations.
        uint32_t anyf = 0u;
#pragma unroll
        for (int c = 0; c < CH; ++c) anyf |= flags[c];
        const bool any = __ballot(anyf != 0u) != 0ull;
        int below[CH], wsum[CH];
#pragma unroll
        for (int c = 0; c < CH; ++c) below[c] = wsum[c] = 0;
        if (any) {
#pragma unroll
            for (int c = 0; c < CH; ++c)
#pragma unroll
                for (int b = 0; b < 8; ++b) {
                    const uint64_t mb = __ballot((flags[c] >> b) & 1u);
                    below[c] += bits_below(mb);
                    wsum[c] += __popcll(mb);
                }
        }
        if (lane == 0) {
#pragma unroll
            for (int c = 0; c < CH; ++c) wtot[c][wave] = wsum[c];
        }
        activation_barrier(&abar, lane, nbar);

        // per-token scales: lane m < MB reduces token m over the waves (every
        // activation wave does, so no further barrier is needed)
        float s_l = 1.0f, r_l = 1.0f;
        {
            uint32_t ab = 0u;
            if (lane < MB) {
                const u32x4 r0 = *reinterpret_cast<const u32x4*>(&rmax[lane][0]);
                const u32x4 r1 = *reinterpret_cast<const u32x4*>(&rmax[lane][4]);
                ab = max(max(max(r0[0], r0[1]), max(r0[2], r0[3])), max(max(r1[0], r1[1]), max(r1[2], r1[3])));
            }
            // SmoothQuant per-tensor: the maximum over every token (tokens past M are 0)
            if constexpr (SM == 2) ab = wave_max_u32(ab);
            if (lane < MB) {
                // LLM.int8(): an fp16 magnitude pattern; SmoothQuant: an fp32 one
                const float a = SM ? __builtin_bit_cast(float, ab) : h2f((uint16_t)ab);
                s_l = a == 0.0f ? 1.0f : a / 127.0f;
                r_l = 1.0f / s_l;
                if (wave == 0) sx_s[lane] = s_l;
            }
        }

        int total0 = 0, wbase[CH];
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int4 wt0 = *reinterpret_cast<const int4*>(&wtot[c][0]);
            const int4 wt1 = *reinterpret_cast<const int4*>(&wtot[c][4]);
            const int wt[8] = {wt0.x, wt0.y, wt0.z, wt0.w, wt1.x, wt1.y, wt1.z, wt1.w};
            int tot = 0, bs = 0;
#pragma unroll
            for (int w = 0; w < DEC_WAVES; ++w) {
                tot += wt[w];
                bs += w < wave ? wt[w] : 0;
            }
            wbase[c] = bs + (c == 1 ? total0 : 0);
            if (c == 0) total0 = tot;
            count += tot;
        }
        if (t == 0) count_s = count;
        if (any) {
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                uint32_t f = flags[c];
                int o = wbase[c] + below[c];
                while (f) {
                    const int j = __builtin_ctz(f);
                    f &= f - 1u;
                    oidx[o] = (int16_t)(8 * (t + DEC_THREADS * c) + j);
                    if (o < OCAP) {
#pragma unroll
                        for (int m = 0; m < MB; ++m) {
                            const uint32_t w32 = pick4(xv[c][m], j >> 1);
                            xo[o][m] = h2f((uint16_t)((j & 1) ? (w32 >> 16) : (w32 & 0xffffu)));
                        }
                    }
                    ++o;
                }
            }
        }

        // 2c. int8 codes of X into LDS: biased codes from the division-free
        //     rounding, un-biased (XOR 0x80) and zeroed in the outlier columns
        //     by the byte mask of the keep words; tokens past M read zeros, have
        //     scale 1 and get codes 0, which no MFMA reads
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int ch = t + DEC_THREADS * c;
            if (ch < nch) {
                const uint32_t kb0 = __builtin_amdgcn_perm(keep[c][1], keep[c][0], 0x06040200u);
                const uint32_t kb1 = __builtin_amdgcn_perm(keep[c][3], keep[c][2], 0x06040200u);
#pragma unroll
                for (int m = 0; m < MB; ++m) {
                    const float s = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s_l), m));
                    const float r = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, r_l), m));
                    if constexpr (SM != 0) {
                        // two's-complement codes of the smoothed values (no outlier columns)
                        float yt[8];
                        if constexpr (!HOLD) smooth_chunk(c, m, yt);
                        *reinterpret_cast<u32x2*>(aq + m * LDA + 8 * ch) = codes8_dyn(HOLD ? y[HOLD ? m : 0] : yt, s, r);
                    } else {
                        const u32x2 q = codes8_biased(xv[c][m], s, r);
                        *reinterpret_cast<u32x2*>(aq + m * LDA + 8 * ch) =
                            u32x2{(q[0] ^ 0x80808080u) & kb0, (q[1] ^ 0x80808080u) & kb1};
                    }
                }
            }
        }
        lds_barrier();                                                  // barrier 2: codes, list, scales
        lds_barrier();                                                  // barrier 3: partial tiles
    } else {
        // ---------------------------------------------------------------- weight waves
        const int ww = wave - DEC_WAVES;
        lds_barrier();                                                  // barrier 1: X requests issued
        // the weight slice: row n0 + lane % 16, bytes 64 s + 16 (lane / 16) of step s = ww + 8 j
        v4i wv[STEPS];
        {
            const uint32_t wo0 = (uint32_t)((lane & 15) * K + 16 * (lane >> 4));
#pragma unroll
            for (int j = 0; j < STEPS; ++j) {
                const int s = ww + DEC_WAVES * j;
                wv[j] = __builtin_bit_cast(v4i, bload16(rsw, s < S ? wo0 + 64 * s : kOOB));
            }
        }
        lds_barrier();                                                  // barrier 2
        count = count_s;
        // start the gather of the outlier weights (first 64): the fp16 W[n][h]
        // or the int8 code Wq[n][h], as the aligned 32-bit word holding it; the
        // loads are unconditional (the descriptor is selected) and queue behind
        // the weight stream, whose use waits for them anyway
        const int gch = t & 15, gh = t >> 4;          // channel n0 + gch, outlier slots gh + 32 q
        const rsrc_t rs16 = make_rsrc(W16 ? W16 + n0 * K : nullptr, W16 ? (N - n0) * K * 2 : 0);
        const rsrc_t rsg = W16 ? rs16 : rsw;
        constexpr int GQ = OCAP / (DEC_THREADS / 16);
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
        // 3a. int32 MFMA over this wave's K steps.  The MFMAs are unconditional
        // (a step past the end has an all-zero weight fragment, so it adds
        // nothing): under a branch on s < S the compiler moves the step's
        // weight load into the branch, behind barrier 2, where its whole
        // latency lands after the activation codes.
        const int arow = lane & 15;
#pragma unroll
        for (int j = 0; j < STEPS; ++j) {
            const int s = ww + DEC_WAVES * j;
            v4i fa = v4i{0, 0, 0, 0};
            if (arow < M && s < S) fa = *reinterpret_cast<const v4i*>(aq + arow * LDA + 64 * s + 16 * (lane >> 4));
            acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa, wv[j], acc, 0, 0, 0);
        }
        // acc: lane l, element e = token 4 (l / 16) + e, channel l % 16
#pragma unroll
        for (int e = 0; e < 4; ++e) red[ww][(4 * (lane >> 4) + e) * 16 + (lane & 15)] = acc[e];
#pragma unroll
        for (int q = 0; q < GQ; ++q) {
            const uint32_t v = graw[q] >> gsh[q];         // zero for an empty slot
            wo[gh + (DEC_THREADS / 16) * q][gch] = W16 ? h2f((uint16_t)v) : h2f(f2h(swg * (float)(int8_t)(uint8_t)v));
        }
        lds_barrier();                                                  // barrier 3
        return;
    }

    // 3b. epilogue (activation threads t < 256): token m = t / 16, channel n0 + t % 16
    const int m = t >> 4, ch = t & 15;
    const int64_t n = n0 + ch;
    if (t < 256 && m < M && n < N) {
        int32_t c = 0;
#pragma unroll
        for (int w = 0; w < DEC_WAVES; ++w) c += red[w][t];
        float v = (float)c * sx_s[m] * swg;
        const int hs = count < OCAP ? count : OCAP;
        for (int h = 0; h < hs; ++h) v = v + xo[h][m] * wo[h][ch];
        for (int h = OCAP; h < count; ++h) {              // beyond the staged outliers
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

    // 4. the integer stages (outlier list, count, per-token scales, codes)
    //    go where the general path keeps them: workgroup 0 writes the list,
    //    count and scales, and every workgroup an equal share of the 16-byte
    //    chunks of the codes (all of them hold the same codes), so that no
    //    single workgroup carries the whole 32 KB store at the kernel's end
    if (blockIdx.x == 0) {
        for (int h = t; h < count; h += DEC_THREADS) st.idx[h] = oidx[h];
        if (t == 0) *st.count = count;
        if (t < M) st.s_x[t] = sx_s[t];
    }
    {
        const int cpr = K >> 4;                       // 16-byte chunks per row
        const int total = M * cpr, per = (total + (int)gridDim.x - 1) / (int)gridDim.x;
        const int q0 = (int)blockIdx.x * per, q1 = q0 + per < total ? q0 + per : total;
        for (int q = q0 + t; q < q1; q += DEC_THREADS) {
            const int r = q / cpr, j = q - r * cpr;
            *reinterpret_cast<v4i*>(st.xq + (int64_t)r * K + 16 * j) =
                *reinterpret_cast<const v4i*>(aq + r * LDA + 16 * j);
        }
    }
}

bool decode_supported(int64_t M, int64_t K) {
    if (M < 1 || K < 256 || K % 256 != 0) return false;
    return (M <= 16 && K <= DEC_CHUNK_K) || (M <= 8 && K <= 2 * DEC_CHUNK_K);
}

// The threshold as an fp16 bit pattern: column j is an outlier when
// max_i |X[i][j]| > tau (fp32), i.e. when its largest |x| pattern is >= thr1,
// with thr1 = 1 + the pattern of the largest fp16 <= tau (0 when tau < 0: every
// column; 0x7c00 when tau >= 65504: no finite magnitude exceeds it).
static uint32_t threshold_pattern(float tau) {
    if (!(tau >= 0.0f)) return 0u;
    if (tau >= 65504.0f) return 0x7c00u;
    uint32_t lo = 0, hi = 0x7bff;                     // largest pattern p with value(p) <= tau
    while (lo < hi) {
        const uint32_t mid = (lo + hi + 1) / 2;
        const int e = (int)(mid >> 10), f = (int)(mid & 1023);
        const double v = e == 0 ? std::ldexp((double)f, -24) : std::ldexp((double)(f | 1024), e - 25);
        if (v <= (double)tau)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo + 1;
}

template <int MB, int CH, bool TOPK, int SM = 0>
static void launch_mb(const dim3& grid, hipStream_t st, const uint16_t* X, int64_t M, int64_t K, const int8_t* Wq,
                      const float* s_w, const uint16_t* W16, int64_t N, uint32_t thr1, void* out, int out_dtype,
                      const DecodeStages& stages, const float* sm = nullptr) {
    hipLaunchKernelGGL((k_decode_mixed<MB, CH, TOPK, SM>), grid, dim3(2 * DEC_THREADS), 0, st, X, (int)M, (int)K, Wq,
                       s_w, W16, N, thr1, out, out_dtype, stages, sm);
}

template <bool TOPK>
static void launch_decode(const uint16_t* X, int64_t M, int64_t K, const int8_t* Wq, const float* s_w,
                          const uint16_t* W16, int64_t N, uint32_t thr1, void* out, int out_dtype,
                          const DecodeStages& stages, hipStream_t st) {
    const dim3 grid((unsigned)((N + 15) / 16));
    if (K > DEC_CHUNK_K) {
        if (M <= 4)
            launch_mb<4, 2, TOPK>(grid, st, X, M, K, Wq, s_w, W16, N, thr1, out, out_dtype, stages);
        else
            launch_mb<8, 2, TOPK>(grid, st, X, M, K, Wq, s_w, W16, N, thr1, out, out_dtype, stages);
    } else if (M <= 4) {
        launch_mb<4, 1, TOPK>(grid, st, X, M, K, Wq, s_w, W16, N, thr1, out, out_dtype, stages);
    } else if (M <= 8) {
        launch_mb<8, 1, TOPK>(grid, st, X, M, K, Wq, s_w, W16, N, thr1, out, out_dtype, stages);
    } else {
        launch_mb<16, 1, TOPK>(grid, st, X, M, K, Wq, s_w, W16, N, thr1, out, out_dtype, stages);
    }
}

hipError_t launch_decode_mixed(const uint16_t* X, int64_t M, int64_t K, const int8_t* Wq, const float* s_w,
                               const uint16_t* W16, int64_t N, float tau, void* out, int out_dtype,
                               const DecodeStages& stages, hipStream_t st) {
    launch_decode<false>(X, M, K, Wq, s_w, W16, N, threshold_pattern(tau), out, out_dtype, stages, st);
    return hipGetLastError();
}

int64_t decode_topk_max() { return DEC_OCAP_TOPK; }

// SmoothQuant in the fused kernel: the shapes whose smoothing fits the
// registers of four waves per SIMD without spilling (M <= 8 at K <= 4096,
// M <= 4 at K <= 8192); larger ones keep the smoothing quantizer + GEMV.
bool decode_smooth_supported(int64_t M, int64_t K) {
    if (M < 1 || K < 256 || K % 256 != 0) return false;
    return (M <= 8 && K <= DEC_CHUNK_K) || (M <= 4 && K <= 2 * DEC_CHUNK_K);
}

template <int SM>
static void launch_smooth_sm(const dim3& grid, hipStream_t st, const uint16_t* X, int64_t M, int64_t K,
                             const int8_t* Wq, const float* s_w, int64_t N, void* out, int out_dtype,
                             const DecodeStages& stages, const float* sm) {
    // (no outlier columns: the threshold pattern is above every finite magnitude)
    constexpr uint32_t NOT = 0x7c00u;
    if (K > DEC_CHUNK_K)
        launch_mb<4, 2, false, SM>(grid, st, X, M, K, Wq, s_w, nullptr, N, NOT, out, out_dtype, stages, sm);
    else if (M <= 4)
        launch_mb<4, 1, false, SM>(grid, st, X, M, K, Wq, s_w, nullptr, N, NOT, out, out_dtype, stages, sm);
    else
        launch_mb<8, 1, false, SM>(grid, st, X, M, K, Wq, s_w, nullptr, N, NOT, out, out_dtype, stages, sm);
}

hipError_t launch_decode_smooth(const uint16_t* X, int64_t M, int64_t K, const float* sm, bool per_tensor,
                                const int8_t* Wq, const float* s_w, int64_t N, void* out, int out_dtype,
                                const DecodeStages& stages, hipStream_t st) {
    if (!decode_smooth_supported(M, K)) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((N + 15) / 16));
    if (per_tensor)
        launch_smooth_sm<2>(grid, st, X, M, K, Wq, s_w, N, out, out_dtype, stages, sm);
    else
        launch_smooth_sm<1>(grid, st, X, M, K, Wq, s_w, N, out, out_dtype, stages, sm);
    return hipGetLastError();
}

hipError_t launch_decode_topk(const uint16_t* X, int64_t M, int64_t K, int64_t k, const int8_t* Wq, const float* s_w,
                              const uint16_t* W16, int64_t N, void* out, int out_dtype, const DecodeStages& stages,
                              hipStream_t st) {
    if (k < 0 || k > K || k > DEC_OCAP_TOPK) return hipErrorInvalidValue;
    launch_decode<true>(X, M, K, Wq, s_w, W16, N, (uint32_t)k, out, out_dtype, stages, st);
    return hipGetLastError();
}

}  // namespace qa
