// k_gemm.hip -- integer GEMMs of the quantized linear layer on gfx950 MFMA.
//
//   int8:  C = Xq * Wq^T on v_mfma_i32_16x16x64_i8 with int32 accumulation,
//          then either an int32 store or the LLM.int8() epilogue: dequantize
//          by s_x[m] * s_w[n] (outer product of the vector-wise scales) and
//          add the fp16 product over the outlier columns, gathered from X and
//          W and run on v_mfma_f32_16x16x32_f16 with the dequantized tile as
//          the accumulator input.
//          [AIInfra 05Quantization01, LLM.int8(): "b. INT8 矩阵乘法与反量化"
//           and the merge of the fp16 outlier part]
//   W4A4:  packed int4 operands (eight per 32-bit word) are unpacked into the
//          high nibble of each int8 lane of the same MFMA, so every product is
//          256 x the int4 product; each G-group is accumulated in int32 on its
//          own and dequantized by s_w[n][g] * 2^-8 into an fp32 sum, scaled
//          by s_x[m] at the end.
//          [低比特量化加速：分组旋转方法从W8A8到W4A4, §5.4]
//
// Both operands are K-contiguous ([rows x K]).  A stage of BK bytes of K per
// row is staged in LDS with the 16-byte chunk index XOR-swizzled by the row
// (chunk c of row r lives at chunk c ^ (r & 7)), so the 16-byte fragment
// reads of one MFMA hit distinct banks.  Global loads of stage k+1 are in
// flight while stage k is multiplied (two LDS buffers, one barrier per stage).
// The MFMA k-permutation only has to agree between the two operands, which
// is what lets the int4 unpack skip the nibble interleave.
#include <utility>

#include "qa_device.hpp"
#include "qa_launch.hpp"

namespace qa {

// Compile-time loop: f(std::integral_constant<int, I>) for I in [0, N), so
// register arrays are always indexed by constants.
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

template <int BM_, int BN_, int WM_, int WN_>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
    static constexpr int BK = 128;                        // bytes of K per stage
    static constexpr int THREADS = 64 * WM * WN;
    static constexpr int TM = BM / WM, TN = BN / WN;      // wave tile
    static constexpr int FM = TM / 16, FN = TN / 16;      // 16x16 fragments per wave
    static constexpr int A_CH = BM * (BK / 16) / THREADS; // 16-byte chunks per thread
    static constexpr int B_CH = BN * (BK / 16) / THREADS;
    static constexpr int LDS_A = BM * BK, LDS_B = BN * BK;
    static constexpr int LDS = 2 * (LDS_A + LDS_B);
    static_assert(A_CH * THREADS == BM * (BK / 16) && B_CH * THREADS == BN * (BK / 16), "tile/threads");
};

// Block -> output tile.  Blocks are dispatched round-robin over the 8 XCDs
// (block b runs on XCD b % 8); the remap gives every XCD a contiguous range of
// tiles, walked GROUP tile-rows at a time so neighbouring blocks of one XCD
// share A rows and B columns in its L2.
__device__ __forceinline__ void tile_of_block(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
    const int ntiles = tiles_m * tiles_n;
    const int per = ntiles >> 3, rem = ntiles & 7;
    const int xcd = bid & 7, slot = bid >> 3;
    const int t = xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
    constexpr int GROUP = 8;
    const int gsz = GROUP * tiles_n;
    const int g = t / gsz;
    const int first = g * GROUP;
    const int gm = tiles_m - first < GROUP ? tiles_m - first : GROUP;
    const int r = t - g * gsz;
    tm = first + r % gm;
    tn = r / gm;
}

__device__ __forceinline__ int swz(int r, int c) { return r * 128 + ((c ^ (r & 7)) << 4); }

// Global -> registers for one stage: rows [0, ROWS) of the block's rows of a
// K-contiguous byte matrix (row stride ld bytes; `rs` covers the block's first
// row to the end of the matrix, so rows past the end read zeros), byte columns
// [kb, kb + 128); chunks at or past kbytes read zeros.
template <int NCH, int THREADS>
__device__ __forceinline__ void g2r(rsrc_t rs, uint32_t ld, uint32_t kb, uint32_t kbytes, u32x4* reg) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int q = threadIdx.x + i * THREADS;
        const uint32_t r = q >> 3, gk = kb + (q & 7) * 16;
        reg[i] = bload16(rs, gk < kbytes ? r * ld + gk : kOOB);
    }
}

template <int NCH, int THREADS>
__device__ __forceinline__ void r2s(uint8_t* lds, const u32x4* reg) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int q = threadIdx.x + i * THREADS;
        *reinterpret_cast<u32x4*>(lds + swz(q >> 3, q & 7)) = reg[i];
    }
}

// No-op for the main loops' `after_issue` hook.
struct NoHook {
    __device__ __forceinline__ void operator()() const {}
};

// ---------------------------------------------------------------------------
// int8 main loop: acc[FM][FN] = A[m0.., :] * B[n0.., :]^T
// The MFMA takes the B fragment as its first operand, so it produces the
// transposed 16 x 16 tile: lane l, element e of acc[i][j] holds output row
// i*16 + l%16 and column j*16 + 4*(l/16) + e of the wave tile (four
// consecutive columns per lane, stored with one vector store).
// ---------------------------------------------------------------------------
template <class C, class F = NoHook>
__device__ __forceinline__ void mainloop_i8(const int8_t* __restrict__ A, const int8_t* __restrict__ B,
                                            int64_t M, int64_t N, int64_t K, int64_t m0, int64_t n0,
                                            uint8_t* smem, v4i (&acc)[C::FM][C::FN], F&& after_issue = F{}) {
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int wm = wave / C::WN, wn = wave % C::WN;
    const uint8_t* Ab = reinterpret_cast<const uint8_t*>(A);
    const uint8_t* Bb = reinterpret_cast<const uint8_t*>(B);
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) acc[i][j] = v4i{0, 0, 0, 0};

    const int nk = (int)((K + C::BK - 1) / C::BK);
    const rsrc_t rsa = make_rsrc(Ab + m0 * K, (M - m0) * K);
    const rsrc_t rsb = make_rsrc(Bb + n0 * K, (N - n0) * K);
    const uint32_t ld = (uint32_t)K, kbytes = (uint32_t)K;
    u32x4 ra[C::A_CH], rb[C::B_CH];
    g2r<C::A_CH, C::THREADS>(rsa, ld, 0, kbytes, ra);
    g2r<C::B_CH, C::THREADS>(rsb, ld, 0, kbytes, rb);
    after_issue();
    r2s<C::A_CH, C::THREADS>(smem, ra);
    r2s<C::B_CH, C::THREADS>(smem + C::LDS_A, rb);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        uint8_t* sa = smem + (kt & 1) * (C::LDS_A + C::LDS_B);
        uint8_t* sb = sa + C::LDS_A;
        const bool more = kt + 1 < nk;
        if (more) {
            g2r<C::A_CH, C::THREADS>(rsa, ld, (uint32_t)(kt + 1) * C::BK, kbytes, ra);
            g2r<C::B_CH, C::THREADS>(rsb, ld, (uint32_t)(kt + 1) * C::BK, kbytes, rb);
        }
#pragma unroll
        for (int s = 0; s < C::BK / 64; ++s) {
            const int c = s * 4 + (lane >> 4);
            v4i fa[C::FM], fb[C::FN];
#pragma unroll
            for (int i = 0; i < C::FM; ++i) {
                const int r = wm * C::TM + i * 16 + (lane & 15);
                fa[i] = *reinterpret_cast<const v4i*>(sa + swz(r, c));
            }
#pragma unroll
            for (int j = 0; j < C::FN; ++j) {
                const int r = wn * C::TN + j * 16 + (lane & 15);
                fb[j] = *reinterpret_cast<const v4i*>(sb + swz(r, c));
            }
#pragma unroll
            for (int i = 0; i < C::FM; ++i)
#pragma unroll
                for (int j = 0; j < C::FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fb[j], fa[i], acc[i][j], 0, 0, 0);
        }
        if (more) {
            uint8_t* na = smem + ((kt + 1) & 1) * (C::LDS_A + C::LDS_B);
            r2s<C::A_CH, C::THREADS>(na, ra);
            r2s<C::B_CH, C::THREADS>(na + C::LDS_A, rb);
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// int8 main loop with direct global -> LDS loads (gfx950 buffer_load ... lds).
// WM x WN waves, wave tile (BM/WM) x (BN/WN).  K advances 64 bytes per stage;
// four LDS stages, three in flight.  A DMA instruction writes 64 lanes x 16
// bytes = 1 KB of LDS at consecutive addresses, so the XOR swizzle of the
// stage layout (chunk c of row r stored at chunk c ^ ((r >> 1) & 3), which
// makes the 16-byte fragment reads of 8 consecutive rows hit 8 different bank
// groups) is produced by choosing which global chunk each lane fetches.  The
// waits are explicit: s_waitcnt vmcnt(n) for this wave's stage-kt loads, then
// a bare s_barrier (a __syncthreads would also drain the younger stages).
// With two waves per SIMD (8 waves) one wave's LDS reads and barrier wait
// overlap the other's MFMAs, so the loop itself is not software-pipelined.
// ---------------------------------------------------------------------------
template <int BM_, int BN_, int WM_, int WN_>
struct CfgD {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, NW = WM * WN;
    static constexpr int BK = 64, STAGES = 4, THREADS = 64 * NW;
    static constexpr int TM = BM / WM, TN = BN / WN;
    static constexpr int FM = TM / 16, FN = TN / 16;
    // 1 KB DMA instructions (16 rows) per stage; instruction i is issued by
    // wave i % NW.  A splits evenly over the waves; B may not (then the
    // first B_TOT % NW waves issue one more).
    static constexpr int A_TOT = BM / 16, B_TOT = BN / 16;
    static constexpr int QA = A_TOT / NW, QB = (B_TOT + NW - 1) / NW;
    static constexpr int A_INS = BM / (16 * NW), B_INS = BN / (16 * NW);   // per wave (even splits)
    static constexpr int LDS_A = BM * BK, LDS_B = BN * BK, STAGE = LDS_A + LDS_B;
    static constexpr int LDS = STAGES * STAGE;
    static_assert(BM % 16 == 0 && BN % 16 == 0 && A_TOT % NW == 0, "stage rows must split over waves");
};

__device__ __forceinline__ int swz64(int r, int c) { return r * 64 + ((c ^ ((r >> 1) & 3)) << 4); }

// s_waitcnt immediate waiting for vmcnt <= n only (gfx9 encoding)
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

typedef __attribute__((address_space(3))) void lds_void;

// Workgroup barrier that also keeps the compiler from moving memory accesses
// across it (the DMA writes and the fragment reads of the same LDS stage).
__device__ __forceinline__ void block_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// `after_issue` runs once the first stages' loads are in flight (the caller
// issues its own early loads there).
template <class C, class F = NoHook>
__device__ __forceinline__ void mainloop_i8_dma(rsrc_t rsa, rsrc_t rsb, uint32_t K, uint8_t* smem,
                                                v4i (&acc)[C::FM][C::FN], F&& after_issue = F{}) {
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int wm = wave / C::WN, wn = wave % C::WN;
    constexpr bool B_EVEN = C::B_TOT % C::NW == 0;
    constexpr int PL = C::QA + C::B_TOT / C::NW, PH = C::QA + C::QB;   // loads per stage of a wave
    const bool bhi = B_EVEN || wave < C::B_TOT % C::NW;                // this wave issues QB B loads
    uint32_t oa[C::QA], ca[C::QA], ob[C::QB], cb[C::QB];
#pragma unroll
    for (int q = 0; q < C::QA; ++q) {
        const int P = (q * C::NW + wave) * 64 + lane;        // physical 16-byte chunk of the stage
        const int r = P >> 2, c = (P & 3) ^ ((r >> 1) & 3);
        oa[q] = (uint32_t)r * K + c * 16;
        ca[q] = c * 16;
    }
#pragma unroll
    for (int q = 0; q < C::QB; ++q) {
        const int P = (q * C::NW + wave) * 64 + lane;
        const int r = P >> 2, c = (P & 3) ^ ((r >> 1) & 3);
        ob[q] = (uint32_t)r * K + c * 16;
        cb[q] = c * 16;
    }
    const int nk = (int)((K + C::BK - 1) / C::BK);
    auto issue = [&](int kt) __attribute__((always_inline)) {
        uint8_t* st = smem + (kt % C::STAGES) * C::STAGE;
        const uint32_t k0 = (uint32_t)kt * C::BK;
#pragma unroll
        for (int q = 0; q < C::QA; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_void*)(st + (q * C::NW + wave) * 1024), 16,
                                                     k0 + ca[q] < K ? oa[q] + k0 : kOOB, 0, 0, 0);
#pragma unroll
        for (int q = 0; q < C::QB; ++q)
            if (B_EVEN || q < C::QB - 1 || bhi)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_void*)(st + C::LDS_A + (q * C::NW + wave) * 1024),
                                                         16, k0 + cb[q] < K ? ob[q] + k0 : kOOB, 0, 0, 0);
    };
    // wait until at most `ahead` younger stages of this wave's loads are in flight
    auto wait_stage = [&](int ahead) __attribute__((always_inline)) {
        if (bhi) {
            if (ahead >= 2)
                __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * PH));
            else if (ahead == 1)
                __builtin_amdgcn_s_waitcnt(vmcnt_imm(PH));
            else
                __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        } else {
            if (ahead >= 2)
                __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * PL));
            else if (ahead == 1)
                __builtin_amdgcn_s_waitcnt(vmcnt_imm(PL));
            else
                __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        }
    };
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) acc[i][j] = v4i{0, 0, 0, 0};
    issue(0);
    if (nk > 1) issue(1);
    if (nk > 2) issue(2);
    after_issue();

    // Stage kt + 3 reuses the buffer of stage kt - 1.  Every wave's reads of
    // that stage completed before its MFMAs of iteration kt - 1 (which consume
    // them), hence before it arrived at the barrier of iteration kt.
    const int c = lane >> 4;
    for (int kt = 0; kt < nk; ++kt) {
        wait_stage((kt + 2 < nk - 1 ? kt + 2 : nk - 1) - kt);        // stages issued after kt
        block_barrier();
        if (kt + 3 < nk) issue(kt + 3);
        const uint8_t* sa = smem + (kt % C::STAGES) * C::STAGE;
        const uint8_t* sb = sa + C::LDS_A;
        v4i fa[C::FM];
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
            fa[i] = *reinterpret_cast<const v4i*>(sa + swz64(wm * C::TM + i * 16 + (lane & 15), c));
        // B fragments one ahead of their MFMAs, so that each fragment's LDS
        // latency hides behind the previous fragment's MFMAs: the scheduling
        // groups fix the order [A reads, B0, B1] [MFMA x FM] ([B j+1] [MFMA x FM])...
        v4i fb[C::FN];
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
            fb[j] = *reinterpret_cast<const v4i*>(sb + swz64(wn * C::TN + j * 16 + (lane & 15), c));
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
            for (int i = 0; i < C::FM; ++i)
                acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fb[j], fa[i], acc[i][j], 0, 0, 0);
        if constexpr (C::FN > 4) {
            __builtin_amdgcn_sched_group_barrier(0x100, C::FM + 2, 0);     // DS reads: A, B0, B1
            __builtin_amdgcn_sched_group_barrier(0x008, C::FM, 0);         // MFMAs of B0
#pragma unroll
            for (int j = 1; j + 1 < C::FN; ++j) {
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);         // read B j+1
                __builtin_amdgcn_sched_group_barrier(0x008, C::FM, 0);     // MFMAs of B j
            }
            __builtin_amdgcn_sched_group_barrier(0x008, C::FM, 0);         // MFMAs of the last B
        }
    }
    __syncthreads();
}

template <class C>
struct IsDma { static constexpr bool value = false; };
template <int BM_, int BN_, int WM_, int WN_>
struct IsDma<CfgD<BM_, BN_, WM_, WN_>> { static constexpr bool value = true; };

template <class C, class F = NoHook>
__device__ __forceinline__ void mainloop_any(const int8_t* __restrict__ A, const int8_t* __restrict__ B, int64_t M,
                                             int64_t N, int64_t K, int64_t m0, int64_t n0, uint8_t* smem,
                                             v4i (&acc)[C::FM][C::FN], F&& after_issue = F{}) {
    if constexpr (IsDma<C>::value) {
        const rsrc_t rsa = make_rsrc(A + m0 * K, (M - m0) * K);
        const rsrc_t rsb = make_rsrc(B + n0 * K, (N - n0) * K);
        mainloop_i8_dma<C>(rsa, rsb, (uint32_t)K, smem, acc, after_issue);
    } else {
        mainloop_i8<C>(A, B, M, N, K, m0, n0, smem, acc, after_issue);
    }
}

template <class C>
__global__ __launch_bounds__(C::THREADS) void k_gemm_i8_i32(const int8_t* __restrict__ A,
                                                            const int8_t* __restrict__ B, int64_t M,
                                                            int64_t K, int64_t N, int32_t* __restrict__ Cout,
                                                            int tiles_m, int tiles_n) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[C::LDS];
    int tm, tn;
    tile_of_block(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * C::BM, n0 = (int64_t)tn * C::BN;
    v4i acc[C::FM][C::FN];
    mainloop_any<C>(A, B, M, N, K, m0, n0, smem, acc);
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int wm = wave / C::WN, wn = wave % C::WN;
    const bool vec = (N & 3) == 0;
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
        const int64_t row = m0 + wm * C::TM + i * 16 + (lane & 15);
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
            const int64_t col = n0 + wn * C::TN + j * 16 + 4 * (lane >> 4);
            if (row >= M) continue;
            if (vec) {
                if (col < N) *reinterpret_cast<v4i*>(Cout + row * N + col) = acc[i][j];
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (col + e < N) Cout[row * N + col + e] = acc[i][j][e];
            }
        }
    }
}

__device__ __forceinline__ void store_out(void* out, int dtype, int64_t off, float v) {
    if (dtype == 0)
        static_cast<float*>(out)[off] = v;
    else if (dtype == 1)
        static_cast<uint16_t*>(out)[off] = f2h(v);
    else
        static_cast<uint16_t*>(out)[off] = f2bf(v);
}

// Four consecutive outputs v[0..3] at out[off .. off + 3]; `vec` means off is
// a multiple of 4 and all four are in range, else only the first n are.
__device__ __forceinline__ void store_out4(void* out, int dtype, int64_t off, const v4f& v, bool vec, int n) {
    if (vec) {
        // (two packed conversions per four values, v_cvt_pk_f16_f32 / v_cvt_pk_bf16_f32)
        if (dtype == 0)
            *reinterpret_cast<v4f*>(static_cast<float*>(out) + off) = v;
        else if (dtype == 1)
            *reinterpret_cast<v4h*>(static_cast<uint16_t*>(out) + off) = __builtin_convertvector(v, v4h);
        else
            *reinterpret_cast<v4bf*>(static_cast<uint16_t*>(out) + off) = __builtin_convertvector(v, v4bf);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (e < n) store_out(out, dtype, off + e, v[e]);
    }
}

// tsn: output columns per tile (the tile computes C::BN >= tsn columns and
// stores the first tsn; tsn = C::BN except for the one-round wide tiles).
template <class C>
__global__ __launch_bounds__(C::THREADS) void k_gemm_i8_mixed(const int8_t* __restrict__ Xq,
                                                              const int8_t* __restrict__ Wq, int64_t M,
                                                              int64_t K, int64_t N, MixedEpilogue ep,
                                                              int tiles_m, int tiles_n, int tsn) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[C::LDS];
    int tm, tn;
    tile_of_block(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * C::BM, n0 = (int64_t)tn * tsn;
    const int64_t nlim = n0 + tsn < N ? n0 + tsn : N;     // columns this tile stores: [n0, nlim)
    v4i acc[C::FM][C::FN];
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int wm = wave / C::WN, wn = wave % C::WN;
    const int64_t rb = m0 + wm * C::TM, cb = n0 + wn * C::TN;

    // The epilogue's scales and the outlier count are loaded before the main
    // loop so their latency hides behind it (with many column fragments the
    // channel scales are loaded after it: registers are short).
    constexpr bool LATE = C::FN > 4;
    const rsrc_t rsw = make_rsrc(ep.s_w + cb, (N - cb) * 4);
    const rsrc_t rsx = make_rsrc(ep.s_x + rb, (M - rb) * 4);
    const int cnt = (int)bload4(make_rsrc(ep.count, 4), 0);
    float sw[C::FN][4], sxv[C::FM];
    auto load_scales = [&]() __attribute__((always_inline)) {
        if constexpr (!LATE) {
#pragma unroll
            for (int j = 0; j < C::FN; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sw[j][e] = __builtin_bit_cast(float, bload4(rsw, (uint32_t)(j * 16 + 4 * (lane >> 4) + e) * 4));
        }
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
            sxv[i] = __builtin_bit_cast(float, bload4(rsx, (uint32_t)(i * 16 + (lane & 15)) * 4));
    };
    if constexpr (!LATE) load_scales();

    // Up to PRE outlier columns: the list is read here with the scales, and
    // the gather of this thread's row(s) of X or w~ is issued in the main
    // loop's hook, behind the first stages' loads; the values wait in registers.
    // (Not with many column fragments, whose accumulators leave no registers:
    // those columns are staged after the main loop.)
    constexpr int PRE = LATE ? 0 : OUTLIER_PREFETCH;
    constexpr int PR = (C::BM + C::BN + C::THREADS - 1) / C::THREADS;   // gathered rows per thread
    const rsrc_t rxo = make_rsrc(ep.X + m0 * K, (M - m0) * K * 2);
    const rsrc_t rwo = ep.W16 ? make_rsrc(ep.W16 + n0 * K, (N - n0) * K * 2) : make_rsrc(ep.Wq + n0 * K, (N - n0) * K);
    const rsrc_t rsn = make_rsrc(ep.s_w + n0, (N - n0) * 4);
    uint32_t pk[PRE > 0 ? PRE : 1], pv[PR][PRE > 0 ? PRE : 1];
    {
        const rsrc_t ridx = make_rsrc(ep.idx, (int64_t)PRE * 4);
#pragma unroll
        for (int u = 0; u < PRE; ++u) pk[u] = bload4(ridx, (uint32_t)u * 4);
    }
    // gather row p of the block: X rows [0, BM), then W rows
    auto prefetch = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int pr = 0; pr < PR; ++pr) {
            const int prow = threadIdx.x + pr * C::THREADS;
            const bool pisx = prow < C::BM;
            const uint32_t prr = pisx ? prow : prow - C::BM;
            const bool any = cnt > 0 && cnt <= PRE && prow < C::BM + C::BN;
#pragma unroll
            for (int u = 0; u < PRE; ++u) {
                const bool ok = any && u < cnt;
                if (pisx)
                    pv[pr][u] = bload2(rxo, ok ? (prr * (uint32_t)K + pk[u]) * 2 : kOOB);
                else if (ep.W16)
                    pv[pr][u] = bload2(rwo, ok ? (prr * (uint32_t)K + pk[u]) * 2 : kOOB);
                else
                    pv[pr][u] = bload1(rwo, ok ? prr * (uint32_t)K + pk[u] : kOOB);
            }
        }
    };
    mainloop_any<C>(Xq, Wq, M, N, K, m0, n0, smem, acc, prefetch);
    // LATE: the channel scales of the tile's columns go to LDS (after the
    // outlier staging area), read per fragment in the epilogue
    constexpr int SWE_OFF = ((C::BM + C::BN) * (96 + 8) * 2 + (96 + C::BN) * 4 + 15) / 16 * 16;
    float* swe = reinterpret_cast<float*>(smem + SWE_OFF);
    if constexpr (LATE) {
        static_assert(SWE_OFF + C::BN * 4 <= C::LDS, "epilogue scales exceed LDS");
        load_scales();
        for (int r = threadIdx.x; r < C::BN; r += C::THREADS)
            swe[r] = __builtin_bit_cast(float, bload4(rsn, (uint32_t)r * 4));
        // visible to the epilogue through the barriers below (staging) or this one
        __syncthreads();
    }

    // Epilogue, one 16-row fragment at a time: dequantize C * s_x[m] * s_w[n],
    // then add the fp16 outlier product on v_mfma_f32_16x16x32_f16 (operands
    // in the same transposed order as the int8 main loop) with the
    // dequantized tile as the accumulator input.  The block gathers X[m0.., h]
    // and w~[n0.., h] for up to OCAP outlier columns into LDS (free after the
    // main loop), zero-padded to a multiple of 32; more columns take further
    // passes.  One thread owns one row of X or W and loads only real columns.
    constexpr int OCAP = 96;
    constexpr int OST = OCAP + 8;                             // padded row stride (halves)
    _Float16* xo = reinterpret_cast<_Float16*>(smem);         // [BM][OST], then [BN][OST] for w~
    // One pass of up to OCAP outlier columns into LDS.  The pass's column
    // list (and the weight rows' scales) go to LDS first.  X rows come from
    // the compact outlier rows (contiguous 16-byte loads) when the row
    // quantizer wrote them, else they are gathered like the weight rows: a
    // thread owns one column of a 32-column slab and RSTEP-spaced rows, and
    // issues 8 gathers before it writes any, so a pass costs a few load
    // latencies (the accumulators are live here, so registers are scarce).
    constexpr int RSTEP = C::THREADS / 32;
    constexpr int GB = 8;                                     // gathers in flight per thread
    int* hidx = reinterpret_cast<int*>(smem + (C::BM + C::BN) * OST * 2);
    float* swl = reinterpret_cast<float*>(hidx + OCAP);
    static_assert((C::BM + C::BN) * OST * 2 + (OCAP + C::BN) * 4 <= C::LDS, "outlier staging exceeds LDS");
    // (the row quantizer writes the compact rows for every nonzero count;
    // configurations that prefetch up to PRE columns gather those themselves)
    const bool use_xo = ep.Xo != nullptr && cnt > PRE && cnt <= XO_CAP;
    auto stage = [&](int hs) __attribute__((always_inline)) {
        const int hn = cnt - hs < OCAP ? cnt - hs : OCAP;
        const int hp = (hn + 31) & ~31;
        {
            const rsrc_t ridx = make_rsrc(ep.idx + hs, (int64_t)hn * 4);
            for (int h = threadIdx.x; h < hp; h += C::THREADS) hidx[h] = (int)bload4(ridx, (uint32_t)h * 4);
            if (!ep.W16)
                for (int r = threadIdx.x; r < C::BN; r += C::THREADS)
                    swl[r] = __builtin_bit_cast(float, bload4(rsn, (uint32_t)r * 4));
        }
        if (use_xo) {
            const rsrc_t rxc = make_rsrc(ep.Xo + m0 * XO_CAP, (M - m0) * XO_CAP * 2);
            const int c = threadIdx.x & 3;
            for (int hq = 0; hq < hp; hq += 32) {
                const int h = hq + 8 * c;
#pragma unroll
                for (int r0 = 0; r0 < C::BM; r0 += C::THREADS / 4) {
                    const int r = r0 + (threadIdx.x >> 2);
                    if (r < C::BM) {
                        u32x4 v = bload16(rxc, (uint32_t)(r * XO_CAP + hs + h) * 2);
#pragma unroll
                        for (int d = 0; d < 4; ++d) {
                            const uint32_t lo = h + 2 * d < hn ? 0xffffu : 0u;
                            const uint32_t hi = h + 2 * d + 1 < hn ? 0xffff0000u : 0u;
                            v[d] &= lo | hi;
                        }
                        *reinterpret_cast<u32x4*>(xo + r * OST + h) = v;
                    }
                }
            }
        }
        __syncthreads();                                      // the column list
        // the (row, column) pairs of the real columns, GB per thread and
        // batch, all issued before any is written: a pass with up to
        // GB * THREADS pairs costs one load latency
        const int r0 = use_xo ? C::BM : 0;                       // rows to gather: [r0, BM + BN)
        const int npair = (C::BM + C::BN - r0) * hn;
        for (int pb = 0; pb < npair; pb += GB * C::THREADS) {
            uint32_t v[GB];
            int pr[GB], ph[GB];
#pragma unroll
            for (int u = 0; u < GB; ++u) {
                const int pi = pb + (int)threadIdx.x + u * C::THREADS;
                const bool ok = pi < npair;
                const int q = ok ? pi : 0;
                const int rq = q / hn;
                pr[u] = ok ? r0 + rq : -1;
                ph[u] = q - rq * hn;
                const uint32_t k = (uint32_t)hidx[ph[u]];
                const int r = r0 + rq;
                const bool isx = r < C::BM;
                const uint32_t rr = isx ? r : r - C::BM;
                if (isx)
                    v[u] = bload2(rxo, ok ? (rr * (uint32_t)K + k) * 2 : kOOB);
                else if (ep.W16)
                    v[u] = bload2(rwo, ok ? (rr * (uint32_t)K + k) * 2 : kOOB);
                else
                    v[u] = bload1(rwo, ok ? rr * (uint32_t)K + k : kOOB);
            }
#pragma unroll
            for (int u = 0; u < GB; ++u) {
                const int r = pr[u];
                if (r >= 0) {
                    uint16_t hv = (uint16_t)v[u];
                    if (r >= C::BM && !ep.W16) hv = f2h(swl[r - C::BM] * (float)(int8_t)(uint8_t)v[u]);
                    xo[r * OST + ph[u]] = __builtin_bit_cast(_Float16, hv);
                }
            }
        }
        // zero padding of the gathered rows up to the 32-column slab
        if (hp > hn) {
            const int pw = hp - hn;
            for (int q = threadIdx.x; q < (C::BM + C::BN - r0) * pw; q += C::THREADS) {
                const int rq = q / pw;
                xo[(r0 + rq) * OST + hn + (q - rq * pw)] = __builtin_bit_cast(_Float16, (uint16_t)0);
            }
        }
    };
    if (PRE > 0 && cnt > 0 && cnt <= PRE) {
#pragma unroll
        for (int pr = 0; pr < PR; ++pr) {
            const int prow = threadIdx.x + pr * C::THREADS;
            if (prow < C::BM + C::BN) {                     // the prefetched columns, zero-padded to 32
                const bool pisx = prow < C::BM;
                const float pswr = pisx || ep.W16 ? 0.0f
                                                  : __builtin_bit_cast(float, bload4(rsn, (uint32_t)(prow - C::BM) * 4));
#pragma unroll
                for (int u = 0; u < 32; ++u) {
                    uint16_t hv = 0;
                    if (u < PRE && u < cnt) {
                        hv = (uint16_t)pv[pr][u < PRE ? u : 0];
                        if (!pisx && !ep.W16) hv = f2h(pswr * (float)(int8_t)(uint8_t)pv[pr][u < PRE ? u : 0]);
                    }
                    xo[prow * OST + u] = __builtin_bit_cast(_Float16, hv);
                }
            }
        }
        __syncthreads();
    } else if (cnt > PRE && cnt <= OCAP) {
        stage(0);
        __syncthreads();
    }
    const _Float16* wo = xo + C::BM * OST;
    const bool vec = ((ep.ldo | N | tsn) & 3) == 0;
    static_for<C::FM>([&](auto I) __attribute__((always_inline)) {
        constexpr int i = decltype(I)::value;
        const float sx = sxv[i];
        v4f cf[C::FN];
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
            v4f s4;
            if constexpr (LATE)
                s4 = *reinterpret_cast<const v4f*>(swe + wn * C::TN + j * 16 + 4 * (lane >> 4));
            else
                s4 = v4f{sw[j][0], sw[j][1], sw[j][2], sw[j][3]};
#pragma unroll
            for (int e = 0; e < 4; ++e) cf[j][e] = (float)acc[i][j][e] * sx * s4[e];
        }
        for (int hs = 0; hs < cnt; hs += OCAP) {
            if (cnt > OCAP) {                                 // gather this pass (block-uniform)
                __syncthreads();
                stage(hs);
                __syncthreads();
            }
            const int hn = cnt - hs < OCAP ? cnt - hs : OCAP;
            for (int h0 = 0; h0 < hn; h0 += 32) {
                const int r = wm * C::TM + i * 16 + (lane & 15);
                const v8h ao = *reinterpret_cast<const v8h*>(xo + r * OST + h0 + (lane >> 4) * 8);
#pragma unroll
                for (int j = 0; j < C::FN; ++j) {
                    const int c = wn * C::TN + j * 16 + (lane & 15);
                    const v8h bo = *reinterpret_cast<const v8h*>(wo + c * OST + h0 + (lane >> 4) * 8);
                    cf[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bo, ao, cf[j], 0, 0, 0);
                }
            }
        }
        const int64_t row = rb + i * 16 + (lane & 15);
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
            const int64_t col = cb + j * 16 + 4 * (lane >> 4);
            if (row < M && col < nlim)
                store_out4(ep.out, ep.out_dtype, row * ep.ldo + col, cf[j], vec,
                           (int)(nlim - col < 4 ? nlim - col : 4));
        }
    });
}

// ---------------------------------------------------------------------------
// int8 GEMM with zero-point (asymmetric) dequantization:
//   sum_k (xq - z_x[m]) (wq - z_w[n]) = C - z_x[m] a[n] - z_w[n] r_x[m],
//   a[n] = r_w[n] - K z_w[n],  r_x / r_w = row sums of the codes,
// evaluated in int32 (exact while the result fits, K <= 32768), then
// out = that * s_x[m] * s_w[n].  ZW = false: symmetric weight (z_w = 0).
// tsn: output columns per tile, as for k_gemm_i8_mixed.
// ---------------------------------------------------------------------------
template <class C, bool ZW>
__global__ __launch_bounds__(C::THREADS) void k_gemm_i8_asym(const int8_t* __restrict__ Xq,
                                                             const int8_t* __restrict__ Wq, int64_t M, int64_t K,
                                                             int64_t N, AsymEpilogue ep, int tiles_m, int tiles_n,
                                                             int tsn) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[C::LDS];
    int tm, tn;
    tile_of_block(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * C::BM, n0 = (int64_t)tn * tsn;
    const int64_t nlim = n0 + tsn < N ? n0 + tsn : N;     // columns this tile stores: [n0, nlim)
    v4i acc[C::FM][C::FN];
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int wm = wave / C::WN, wn = wave % C::WN;
    const int64_t rb = m0 + wm * C::TM, cb = n0 + wn * C::TN;
    // Per-column and per-row terms, loaded before the main loop; with many
    // column fragments (registers are short) they are loaded after it, the
    // column terms of the tile into LDS, read per fragment.
    constexpr bool LATE = C::FN > 4;
    constexpr int CT = LATE ? 1 : C::FN;
    const rsrc_t rsx = make_rsrc(ep.s_x + rb, (M - rb) * 4);
    const rsrc_t rzx = make_rsrc(ep.z_x + rb, (M - rb) * 4);
    const rsrc_t rrx = make_rsrc(ZW ? ep.r_x + rb : ep.z_x, ZW ? (M - rb) * 4 : 0);
    float sw[CT][4], sxv[C::FM];
    int32_t an[CT][4], zwv[ZW ? CT : 1][4], zxv[C::FM], rxv[ZW ? C::FM : 1];
    auto load_rows = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < C::FM; ++i) {
            const uint32_t off = (uint32_t)(i * 16 + (lane & 15)) * 4;
            sxv[i] = __builtin_bit_cast(float, bload4(rsx, off));
            zxv[i] = (int32_t)bload4(rzx, off);
            if constexpr (ZW) rxv[i] = (int32_t)bload4(rrx, off);
        }
    };
    if constexpr (!LATE) {
        const rsrc_t rsw = make_rsrc(ep.s_w + cb, (N - cb) * 4);
        const rsrc_t rrw = make_rsrc(ep.r_w + cb, (N - cb) * 4);
        const rsrc_t rzw = make_rsrc(ZW ? ep.z_w + cb : ep.r_w, ZW ? (N - cb) * 4 : 0);
#pragma unroll
        for (int j = 0; j < CT; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t off = (uint32_t)(j * 16 + 4 * (lane >> 4) + e) * 4;
                sw[j][e] = __builtin_bit_cast(float, bload4(rsw, off));
                const int32_t z = ZW ? (int32_t)bload4(rzw, off) : 0;
                an[j][e] = (int32_t)bload4(rrw, off) - (int32_t)K * z;
                if constexpr (ZW) zwv[j][e] = z;
            }
        load_rows();
    }
    mainloop_any<C>(Xq, Wq, M, N, K, m0, n0, smem, acc);
    // LATE: s_w, a and z_w of the tile's C::BN columns, LDS being free after
    // the main loop (it ends with a barrier)
    float* swe = reinterpret_cast<float*>(smem);
    int32_t* ane = reinterpret_cast<int32_t*>(smem) + C::BN;
    int32_t* zwe = reinterpret_cast<int32_t*>(smem) + 2 * C::BN;
    if constexpr (LATE) {
        static_assert(3 * C::BN * 4 <= C::LDS, "epilogue terms exceed LDS");
        load_rows();
        const rsrc_t rsn = make_rsrc(ep.s_w + n0, (N - n0) * 4);
        const rsrc_t rrn = make_rsrc(ep.r_w + n0, (N - n0) * 4);
        const rsrc_t rzn = make_rsrc(ZW ? ep.z_w + n0 : ep.r_w, ZW ? (N - n0) * 4 : 0);
        for (int r = threadIdx.x; r < C::BN; r += C::THREADS) {
            const uint32_t off = (uint32_t)r * 4;
            const int32_t z = ZW ? (int32_t)bload4(rzn, off) : 0;
            swe[r] = __builtin_bit_cast(float, bload4(rsn, off));
            ane[r] = (int32_t)bload4(rrn, off) - (int32_t)K * z;
            zwe[r] = z;
        }
        __syncthreads();
    }
    const bool vec = ((ep.ldo | N | tsn) & 3) == 0;
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
        const int64_t row = rb + i * 16 + (lane & 15);
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
            v4f s4;
            v4i a4, z4;
            if constexpr (LATE) {
                const int t = wn * C::TN + j * 16 + 4 * (lane >> 4);
                s4 = *reinterpret_cast<const v4f*>(swe + t);
                a4 = *reinterpret_cast<const v4i*>(ane + t);
                z4 = *reinterpret_cast<const v4i*>(zwe + t);
            } else {
                const int jj = LATE ? 0 : j;
                s4 = v4f{sw[jj][0], sw[jj][1], sw[jj][2], sw[jj][3]};
                a4 = v4i{an[jj][0], an[jj][1], an[jj][2], an[jj][3]};
                if constexpr (ZW) z4 = v4i{zwv[jj][0], zwv[jj][1], zwv[jj][2], zwv[jj][3]};
                else z4 = v4i{0, 0, 0, 0};
            }
            v4f cf;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // wrap-around int32 arithmetic: exact whenever the result fits
                uint32_t c = (uint32_t)acc[i][j][e] - (uint32_t)zxv[i] * (uint32_t)a4[e];
                if constexpr (ZW) c -= (uint32_t)z4[e] * (uint32_t)rxv[i];
                cf[e] = (float)(int32_t)c * sxv[i] * s4[e];
            }
            const int64_t col = cb + j * 16 + 4 * (lane >> 4);
            if (row < M && col < nlim)
                store_out4(ep.out, ep.out_dtype, row * ep.ldo + col, cf, vec,
                           (int)(nlim - col < 4 ? nlim - col : 4));
        }
    }
}

using CfgBig = CfgD<256, 256, 2, 4>;   // 8 waves, wave tile 128 x 64, LDS-DMA stages
using CfgTail = CfgD<128, 256, 2, 4>;  // 8 waves, wave tile 64 x 64, LDS-DMA stages
using CfgMid = Cfg<128, 128, 2, 2>;    // 4 waves, wave tile 64 x 64 (register-staged)
using CfgMidR = CfgMid;
using CfgSmall = Cfg<64, 64, 2, 2>;    // 4 waves, wave tile 32 x 32

template <class C>
static dim3 grid_of(int64_t M, int64_t N, int& tm, int& tn) {
    tm = (int)((M + C::BM - 1) / C::BM);
    tn = (int)((N + C::BN - 1) / C::BN);
    return dim3((unsigned)(tm * tn));
}

// The largest tile that still gives every one of the 256 CUs a block.
static int pick_cfg(int64_t M, int64_t N) {
    const int64_t big = ((M + 255) / 256) * ((N + 255) / 256);
    const int64_t mid = ((M + 127) / 128) * ((N + 127) / 128);
    if (big >= 256) return 2;
    if (mid >= 256) return 1;
    return 0;
}

hipError_t launch_gemm_i8_i32(const int8_t* A, const int8_t* B, int64_t M, int64_t K, int64_t N, int32_t* C,
                              hipStream_t st) {
    int tm, tn;
    switch (pick_cfg(M, N)) {
        case 2: {
            dim3 g = grid_of<CfgBig>(M, N, tm, tn);
            hipLaunchKernelGGL(k_gemm_i8_i32<CfgBig>, g, dim3(CfgBig::THREADS), 0, st, A, B, M, K, N, C, tm, tn);
            break;
        }
        case 1: {
            dim3 g = grid_of<CfgMid>(M, N, tm, tn);
            hipLaunchKernelGGL(k_gemm_i8_i32<CfgMid>, g, dim3(CfgMid::THREADS), 0, st, A, B, M, K, N, C, tm, tn);
            break;
        }
        default: {
            dim3 g = grid_of<CfgSmall>(M, N, tm, tn);
            hipLaunchKernelGGL(k_gemm_i8_i32<CfgSmall>, g, dim3(CfgSmall::THREADS), 0, st, A, B, M, K, N, C, tm,
                               tn);
        }
    }
    return hipGetLastError();
}

// Output columns [0, split) get 256 x 256 tiles in whole rounds over the 256
// CUs, the rest a second launch of 128 x 256 tiles: without it the last
// partial round of big tiles leaves most CUs idle.
// Returns 0 when no split helps.
static int64_t tail_split(int64_t M, int64_t N) {
    const int64_t tm = (M + 255) / 256, tn = (N + 255) / 256, nb = tm * tn;
    if (nb <= 256 || nb % 256 == 0) return 0;
    const int64_t cols = (nb / 256) * 256 / tm;               // whole tile columns in the full rounds
    const int64_t split = cols * 256;
    return cols >= 1 && split < N ? split : 0;
}

// One-round wide tiles: when 256 x 256 tiles would leave a partial second
// round, 256-row tiles computing 352 columns (wave tile 64 x 176) with a
// column stride tsn <= 352 chosen so that all tiles fit one round over the
// 256 CUs -- e.g. 2048 x 11008: 8 x 32 tiles of 256 x 344, against 1.34
// rounds of 256 x 256.  Returns the stride, or 0 when this does not apply.
using CfgWide = CfgD<256, 352, 4, 2>;  // 8 waves, wave tile 64 x 176, LDS-DMA stages
static int wide_stride(int64_t M, int64_t N) {
    const int64_t tm = (M + 255) / 256;
    if (tm > 256 || ((M + 255) / 256) * ((N + 255) / 256) <= 256) return 0;
    const int64_t tn = 256 / tm;                              // tile columns that fit the round
    const int64_t tsn = ((N + tn - 1) / tn + 7) / 8 * 8;      // stride, a multiple of 8
    return tsn <= CfgWide::BN ? (int)tsn : 0;
}

// ---------------------------------------------------------------------------
// Decode-size (M <= 16) int8 GEMM with the mixed epilogue: the weight stream
// of the fused decode kernel, fed with codes that a quantizer already made.
// 16 output channels per 512-thread workgroup; wave w multiplies the 64-byte
// K steps w, w + 8, ..., each weight load covering 16 rows x 512 contiguous
// bytes, the token codes loaded the same way (from L2: every workgroup reads
// them).  Batches of GV_BATCH steps per wave, two in flight; the MFMAs are
// unconditional (steps past K, tokens past M and channels past N load zeros).
// Everything the epilogue reads that does not depend on the products -- the
// outlier count, the scales and the first GV_OC outlier columns of X and w~
// -- is requested before the weight stream, so only the partial-tile sum,
// the dequantization and the outlier FMAs remain after it.  Threads t < 256
// (token t / 16, channel t % 16) dequantize by s_x[m] s_w[n] and add the
// fp16 outlier product, summed in list order.
// ---------------------------------------------------------------------------
constexpr int GV_WAVES = 8, GV_THREADS = 64 * GV_WAVES, GV_BATCH = 8, GV_OC = 128;
constexpr int GV_PP = GV_OC * 16 / (GV_THREADS / 2);              // gathered pairs per thread and pass
constexpr int GV_ALDS = 65536;                                    // codes staged in LDS up to M K bytes

// ALDS: the codes (M K <= GV_ALDS, K % 1024 == 0, K <= 8192, so at most two
// batches per wave) come into LDS once per
// workgroup by LDS-DMA, rows padded by 16 bytes (the 16 token rows of a
// fragment read hit distinct banks), instead of every wave loading its own
// fragments: that halves the requests in flight beside the weight stream.
template <bool ALDS>
__global__ __launch_bounds__(GV_THREADS) void k_gemv_i8_mixed(const int8_t* __restrict__ Xq,
                                                              const int8_t* __restrict__ Wq, int M, int64_t K,
                                                              int64_t N, MixedEpilogue ep) {
    __shared__ int red[GV_WAVES][256];
    __shared__ float xo_s[GV_OC][16], wo_s[GV_OC][16];
    __shared__ __attribute__((aligned(16))) uint8_t aq[ALDS ? GV_ALDS + 16 * 16 : 1];
    const int lda = (int)K + 16;
    const int lane = threadIdx.x & 63, wave = wave_id(), t = threadIdx.x;
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    const int m = t >> 4, ch = t & 15;                            // the epilogue's token and channel (t < 256)
    const int64_t n = n0 + ch;
    const rsrc_t rsa = make_rsrc(Xq, (int64_t)M * K);             // tokens past M read zeros
    if constexpr (ALDS) {
        // chunk q = 1 KB of row q / (K / 1024): one DMA instruction, 16 bytes per lane
        const int cpr = (int)(K >> 10), tc = M * cpr;
#pragma unroll
        for (int j = 0; j < GV_ALDS / 1024 / GV_WAVES; ++j) {
            const int q = wave + GV_WAVES * j;
            if (q < tc) {
                const int r = q / cpr, c = q - r * cpr;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_void*)(aq + r * lda + 1024 * c), 16,
                                                         (uint32_t)(r * K + 1024 * c + 16 * lane), 0, 0, 0);
            }
        }
    }

    // the epilogue's inputs: the first pass's column list (requested first,
    // so that waiting for it does not wait for the weights), the count and
    // the scales, then, behind the first weight batch, the first pass of
    // outlier operands -- waves 0-3 gather X[r][k] (2 bytes), waves 4-7 the
    // source of w~, W16[n0 + r][k] (2 bytes) or Wq[n0 + r][k] (1 byte); pair q
    // of a wave group is column q / 16, row q % 16; each element is read as
    // the aligned word holding it
    const int tt = t & (GV_THREADS / 2 - 1), gr = tt & 15;        // this thread's gathered row
    uint32_t kk[GV_PP], graw[GV_PP], gsh[GV_PP];
    // the column list of a pass, read without the count (the list buffer
    // holds K entries; entries past the count are never used)
    auto load_idx = [&](int hs) __attribute__((always_inline)) {
        const rsrc_t ridx = make_rsrc(ep.idx ? ep.idx + hs : nullptr, ep.idx ? (K - hs) * 4 : 0);
#pragma unroll
        for (int u = 0; u < GV_PP; ++u) kk[u] = bload4(ridx, (uint32_t)((tt + u * (GV_THREADS / 2)) >> 4) * 4);
    };
    load_idx(0);
    const int cntv = (int)bload4(make_rsrc(ep.count, 4), 0);    // made uniform after the products
    const float sx = __builtin_bit_cast(float, bload4(make_rsrc(ep.s_x, (int64_t)M * 4), t < 256 ? (uint32_t)m * 4 : kOOB));
    const rsrc_t rsn = make_rsrc(ep.s_w + n0, (N - n0) * 4);
    const float sw = __builtin_bit_cast(float, bload4(rsn, (uint32_t)ch * 4));
    const bool xw = wave < GV_WAVES / 2;                          // this wave gathers X (else the weight)
    const rsrc_t rsx = make_rsrc(ep.X, (int64_t)M * K * 2);
    const rsrc_t rwo = ep.W16 ? make_rsrc(ep.W16 + n0 * K, (N - n0) * K * 2) : make_rsrc(ep.Wq + n0 * K, (N - n0) * K);
    const rsrc_t rg = xw ? rsx : rwo;                             // wave-uniform
    const uint32_t esz = xw || ep.W16 ? 2u : 1u;
    const bool rok = !xw || gr < M;
    const float swr = __builtin_bit_cast(float, bload4(rsn, (uint32_t)gr * 4));   // scale of weight row gr
    auto gather = [&](int hs, int cnt) __attribute__((always_inline)) {
        const int hn = cnt - hs < GV_OC ? cnt - hs : GV_OC;
#pragma unroll
        for (int u = 0; u < GV_PP; ++u) {
            const int h = (tt + u * (GV_THREADS / 2)) >> 4;
            const uint32_t o = ((uint32_t)gr * (uint32_t)K + kk[u]) * esz;         // byte offset of the element
            graw[u] = bload4(rg, h < hn && rok ? (o & ~3u) : kOOB);
            gsh[u] = (o & 3u) * 8;
        }
    };
    auto stage = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < GV_PP; ++u) {
            const int h = (tt + u * (GV_THREADS / 2)) >> 4;
            const uint32_t v = graw[u] >> gsh[u];
            if (xw)
                xo_s[h][gr] = h2f((uint16_t)v);
            else
                wo_s[h][gr] = ep.W16 ? h2f((uint16_t)v) : h2f(f2h(swr * (float)(int8_t)(uint8_t)v));
        }
    };

    // the int32 products
    const int S = (int)((K + 63) >> 6);                           // 64-byte K steps (the last one may be partial)
    const rsrc_t rsw = make_rsrc(Wq + n0 * K, (N - n0) * K);      // channels past N read zeros
    const uint32_t kl = 16u * (uint32_t)(lane >> 4);              // this lane's 16 bytes of a step
    const uint32_t o0 = (uint32_t)(lane & 15) * (uint32_t)K + kl;
    const int nb = (S + GV_WAVES * GV_BATCH - 1) / (GV_WAVES * GV_BATCH);
    v4i wa[GV_BATCH], aa[GV_BATCH], wb[GV_BATCH], ab[GV_BATCH];
    auto issue = [&](int b, v4i (&w)[GV_BATCH], v4i (&a)[GV_BATCH]) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < GV_BATCH; ++j) {
            const int s = wave + GV_WAVES * (b * GV_BATCH + j);
            const bool ok = s < S && 64u * (uint32_t)s + kl < (uint32_t)K;
            w[j] = __builtin_bit_cast(v4i, bload16(rsw, ok ? o0 + 64u * (uint32_t)s : kOOB));
            if constexpr (!ALDS) a[j] = __builtin_bit_cast(v4i, bload16(rsa, ok ? o0 + 64u * (uint32_t)s : kOOB));
        }
    };
    // ALDS: this wave's fragments of batch b from the staged codes (rows past
    // M repeat row M - 1: their products land in tokens that are not stored;
    // steps past K meet all-zero weight fragments)
    const int arow = (lane & 15) < M ? (lane & 15) : M - 1;
    auto afrag = [&](int b, v4i (&a)[GV_BATCH]) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < GV_BATCH; ++j) {
            const int s = wave + GV_WAVES * (b * GV_BATCH + j);
            const int off = arow * lda + 64 * (s < S ? s : 0) + (int)kl;
            a[j] = *reinterpret_cast<const v4i*>(aq + off);
        }
    };
    auto mult = [&](const v4i (&w)[GV_BATCH], const v4i (&a)[GV_BATCH], v4i& acc) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < GV_BATCH; ++j) acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[j], w[j], acc, 0, 0, 0);
    };
    // No branches around the loads or the MFMAs: a batch past the end loads
    // zeros (and its MFMAs add nothing), so the compiler keeps every load of
    // a batch ahead of the previous batch's MFMAs and waits for exact counts.
    v4i acc = v4i{0, 0, 0, 0};
    issue(0, wa, aa);
    __builtin_amdgcn_sched_barrier(0);              // the first weight batch goes out before any wait
    // the first pass's gathers wait only for the list and the count
    // (requested before the weight loads), not for the weights
    gather(0, cntv);
    if constexpr (ALDS) {
        // nb <= 2 here: both batches in flight, then one wait (this barrier
        // also makes every wave's codes visible)
        if (nb > 1) issue(1, wb, ab);
        __syncthreads();
        afrag(0, aa);
        mult(wa, aa, acc);
        if (nb > 1) {
            afrag(1, ab);
            mult(wb, ab, acc);
        }
    } else if (nb == 1) {
        mult(wa, aa, acc);
    } else {
        int b = 0;
        do {                                        // nb >= 2: no guard for the compiler to sink batch 0 behind
            issue(b + 1, wb, ab);
            __builtin_amdgcn_sched_barrier(0);      // the next batch's loads go out before these MFMAs wait
            mult(wa, aa, acc);
            issue(b + 2, wa, aa);
            __builtin_amdgcn_sched_barrier(0);
            mult(wb, ab, acc);
            b += 2;
        } while (b < nb);
    }
    // acc: lane l, element e = token 4 (l / 16) + e, channel l % 16
#pragma unroll
    for (int e = 0; e < 4; ++e) red[wave][(4 * (lane >> 4) + e) * 16 + (lane & 15)] = acc[e];
    stage();
    __syncthreads();
    const int cnt = __builtin_amdgcn_readfirstlane(cntv);       // block-uniform
    float v = 0.0f;
    if (t < 256) {
        int32_t c = 0;
#pragma unroll
        for (int w = 0; w < GV_WAVES; ++w) c += red[w][t];
        v = (float)c * sx * sw;
    }
    for (int hs = 0; hs < cnt; hs += GV_OC) {
        if (hs > 0) {                                             // later passes (block-uniform)
            __syncthreads();
            load_idx(hs);
            gather(hs, cnt);
            stage();
            __syncthreads();
        }
        const int hn = cnt - hs < GV_OC ? cnt - hs : GV_OC;
        if (t < 256)
            for (int h = 0; h < hn; ++h) v = v + xo_s[h][m] * wo_s[h][ch];
    }
    if (t < 256 && m < M && n < N) {
        const int64_t o = (int64_t)m * ep.ldo + n;
        if (ep.out_dtype == 0)
            static_cast<float*>(ep.out)[o] = v;
        else if (ep.out_dtype == 1)
            static_cast<uint16_t*>(ep.out)[o] = f2h(v);
        else
            static_cast<uint16_t*>(ep.out)[o] = f2bf(v);
    }
}

hipError_t launch_gemm_i8_mixed(const int8_t* Xq, const int8_t* Wq, int64_t M, int64_t K, int64_t N,
                                const MixedEpilogue& ep, hipStream_t st) {
    int tm, tn;
    if (M <= 16) {
        const dim3 g((unsigned)((N + 15) / 16));
        // the staged path handles at most two batches per wave: K <= 8192
        if (M * K <= GV_ALDS && K % 1024 == 0 && K <= 2 * GV_WAVES * GV_BATCH * 64)
            hipLaunchKernelGGL(k_gemv_i8_mixed<true>, g, dim3(GV_THREADS), 0, st, Xq, Wq, (int)M, K, N, ep);
        else
            hipLaunchKernelGGL(k_gemv_i8_mixed<false>, g, dim3(GV_THREADS), 0, st, Xq, Wq, (int)M, K, N, ep);
        return hipGetLastError();
    }
    if (pick_cfg(M, N) == 2) {
        if (const int tsn = wide_stride(M, N)) {
            tm = (int)((M + 255) / 256);
            tn = (int)((N + tsn - 1) / tsn);
            hipLaunchKernelGGL(k_gemm_i8_mixed<CfgWide>, dim3((unsigned)(tm * tn)), dim3(CfgWide::THREADS), 0, st,
                               Xq, Wq, M, K, N, ep, tm, tn, tsn);
            return hipGetLastError();
        }
        if (const int64_t split = tail_split(M, N)) {
            dim3 g = grid_of<CfgBig>(M, split, tm, tn);
            hipLaunchKernelGGL(k_gemm_i8_mixed<CfgBig>, g, dim3(CfgBig::THREADS), 0, st, Xq, Wq, M, K, split, ep,
                               tm, tn, CfgBig::BN);
            const int esz = ep.out_dtype == 0 ? 4 : 2;
            MixedEpilogue et = ep;
            et.s_w = ep.s_w + split;
            et.W16 = ep.W16 ? ep.W16 + split * K : nullptr;
            et.Wq = ep.Wq + split * K;
            et.out = static_cast<uint8_t*>(ep.out) + split * esz;
            g = grid_of<CfgTail>(M, N - split, tm, tn);
            hipLaunchKernelGGL(k_gemm_i8_mixed<CfgTail>, g, dim3(CfgTail::THREADS), 0, st, Xq, Wq + split * K, M, K,
                               N - split, et, tm, tn, CfgTail::BN);
            return hipGetLastError();
        }
    }
    switch (pick_cfg(M, N)) {
        case 2: {
            dim3 g = grid_of<CfgBig>(M, N, tm, tn);
            hipLaunchKernelGGL(k_gemm_i8_mixed<CfgBig>, g, dim3(CfgBig::THREADS), 0, st, Xq, Wq, M, K, N, ep, tm,
                               tn, CfgBig::BN);
            break;
        }
        case 1: {
            dim3 g = grid_of<CfgMid>(M, N, tm, tn);
            hipLaunchKernelGGL(k_gemm_i8_mixed<CfgMid>, g, dim3(CfgMid::THREADS), 0, st, Xq, Wq, M, K, N, ep, tm,
                               tn, CfgMid::BN);
            break;
        }
        default: {
            dim3 g = grid_of<CfgSmall>(M, N, tm, tn);
            hipLaunchKernelGGL(k_gemm_i8_mixed<CfgSmall>, g, dim3(CfgSmall::THREADS), 0, st, Xq, Wq, M, K, N, ep,
                               tm, tn, CfgSmall::BN);
        }
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// W4A4: operands are packed int4 rows of K/2 bytes.  A stage holds 256 K
// elements (128 bytes) per row; one MFMA step covers 64 elements, i.e. 8
// packed bytes per lane (lane l: row l % 16, bytes 8 (l / 16) of the step).
// ---------------------------------------------------------------------------
__device__ __forceinline__ v4i unpack_hi_nibbles(u32x2 w) {
    // element 2j of word w0 -> byte j of d0 (x16), element 2j+1 -> byte j of d1
    v4i d;
    d[0] = (int)((w[0] << 4) & 0xF0F0F0F0u);
    d[1] = (int)(w[0] & 0xF0F0F0F0u);
    d[2] = (int)((w[1] << 4) & 0xF0F0F0F0u);
    d[3] = (int)(w[1] & 0xF0F0F0F0u);
    return d;
}

constexpr int W4_SW_LDS = 4096;                 // floats of per-group weight scales kept in LDS

// Slot of column c's scale for group g in a block's [group][column] table of
// per-group weight scales: the columns are XOR-swizzled in 4-float quads by
// the group, so the fill (consecutive threads take consecutive groups of one
// column) spreads over the LDS banks and quads stay contiguous for 16-byte reads.
template <int BN>
__device__ __forceinline__ int sw_slot(int g, int c) {
    static_assert(BN % 64 == 0, "column quads to swizzle");
    constexpr int MASK = (BN / 4 < 32 ? BN / 4 : 32) - 1;
    return g * BN + (c ^ ((g & MASK) << 2));
}

template <class C, int G, bool STORE_ACC>
__global__ __launch_bounds__(C::THREADS) void k_gemm_w4a4(const uint32_t* __restrict__ Xp,
                                                          const float* __restrict__ s_x,
                                                          const uint32_t* __restrict__ Wp,
                                                          const float* __restrict__ s_w, int64_t M, int64_t K,
                                                          int64_t N, void* __restrict__ out, int out_dtype,
                                                          int tiles_m, int tiles_n) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[C::LDS];
    __shared__ float sws[STORE_ACC ? 1 : W4_SW_LDS];   // s_w[n0 + c][g] * 2^-8 as [g][c]
    constexpr int KS = 256;                      // K elements per stage
    constexpr int STEPS = KS / 64;               // MFMA steps per stage
    constexpr int SPG = G / 64;                  // MFMA steps per group
    int tm, tn;
    tile_of_block(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * C::BM, n0 = (int64_t)tn * C::BN;
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int wm = wave / C::WN, wn = wave % C::WN;
    const int64_t kbytes = K / 2, ng = K / G;
    const uint8_t* Ab = reinterpret_cast<const uint8_t*>(Xp);
    const uint8_t* Bb = reinterpret_cast<const uint8_t*>(Wp);
    const rsrc_t rsa = make_rsrc(Ab + m0 * kbytes, (M - m0) * kbytes);
    const rsrc_t rsb = make_rsrc(Bb + n0 * kbytes, (N - n0) * kbytes);
    const uint32_t ld = (uint32_t)kbytes;

    // per-group weight scales of this block's columns, staged once in LDS
    // when they fit (else read per group from L2)
    const bool sw_in_lds = !STORE_ACC && ng * C::BN <= W4_SW_LDS;
    const rsrc_t rsw = make_rsrc(s_w + (STORE_ACC ? 0 : n0 * ng), STORE_ACC ? 0 : (N - n0) * ng * 4);
    if (sw_in_lds) {
        // all loads issued before the first write: one memory latency, not one per element
        constexpr int PER = (W4_SW_LDS + C::THREADS - 1) / C::THREADS;
        const int total = (int)ng * C::BN;
        float v[PER];
#pragma unroll
        for (int it = 0; it < PER; ++it) {
            const int t = threadIdx.x + it * C::THREADS;             // coalesced over g
            v[it] = __builtin_bit_cast(float, bload4(rsw, (uint32_t)(t < total ? t : 0) * 4));
        }
#pragma unroll
        for (int it = 0; it < PER; ++it) {
            const int t = threadIdx.x + it * C::THREADS;
            const int cc = t / (int)ng, g = t - cc * (int)ng;
            if (t < total) sws[sw_slot<C::BN>(g, cc)] = v[it] * 0x1p-8f;
        }
    }

    v4f f[C::FM][C::FN];
    v4i acc[C::FM][C::FN];
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
            f[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
            acc[i][j] = v4i{0, 0, 0, 0};
        }
    int ccol[C::FN];                               // block-local column of each fragment
#pragma unroll
    for (int j = 0; j < C::FN; ++j) ccol[j] = wn * C::TN + j * 16 + (lane & 15);

    const int nk = (int)((kbytes + C::BK - 1) / C::BK);
    u32x4 ra[C::A_CH], rb[C::B_CH];
    g2r<C::A_CH, C::THREADS>(rsa, ld, 0, (uint32_t)kbytes, ra);
    g2r<C::B_CH, C::THREADS>(rsb, ld, 0, (uint32_t)kbytes, rb);
    r2s<C::A_CH, C::THREADS>(smem, ra);
    r2s<C::B_CH, C::THREADS>(smem + C::LDS_A, rb);
    __syncthreads();
    int step = 0;                                 // global MFMA step index (64 K each)
    const int nsteps = (int)(K / 64);
    for (int kt = 0; kt < nk; ++kt) {
        uint8_t* sa = smem + (kt & 1) * (C::LDS_A + C::LDS_B);
        uint8_t* sb = sa + C::LDS_A;
        const bool more = kt + 1 < nk;
        if (more) {
            g2r<C::A_CH, C::THREADS>(rsa, ld, (uint32_t)(kt + 1) * C::BK, (uint32_t)kbytes, ra);
            g2r<C::B_CH, C::THREADS>(rsb, ld, (uint32_t)(kt + 1) * C::BK, (uint32_t)kbytes, rb);
        }
#pragma unroll
        for (int s = 0; s < STEPS; ++s, ++step) {
            if (step < nsteps) {
                const int byte = s * 32 + (lane >> 4) * 8;          // within the 128-byte row
                const int c = byte >> 4, within = byte & 15;
                v4i fa[C::FM], fb[C::FN];
#pragma unroll
                for (int i = 0; i < C::FM; ++i) {
                    const int r = wm * C::TM + i * 16 + (lane & 15);
                    fa[i] = unpack_hi_nibbles(*reinterpret_cast<const u32x2*>(sa + swz(r, c) + within));
                }
#pragma unroll
                for (int j = 0; j < C::FN; ++j) {
                    const int r = wn * C::TN + j * 16 + (lane & 15);
                    fb[j] = unpack_hi_nibbles(*reinterpret_cast<const u32x2*>(sb + swz(r, c) + within));
                }
#pragma unroll
                for (int i = 0; i < C::FM; ++i)
#pragma unroll
                    for (int j = 0; j < C::FN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
                if ((step + 1) % SPG == 0) {
                    const int g = step / SPG;
                    if constexpr (STORE_ACC) {
                        int32_t* accp = static_cast<int32_t*>(out);
#pragma unroll
                        for (int i = 0; i < C::FM; ++i)
#pragma unroll
                            for (int j = 0; j < C::FN; ++j) {
                                const int64_t col = n0 + ccol[j];
#pragma unroll
                                for (int e = 0; e < 4; ++e) {
                                    const int64_t row = m0 + wm * C::TM + i * 16 + 4 * (lane >> 4) + e;
                                    if (row < M && col < N) accp[(row * N + col) * ng + g] = acc[i][j][e] >> 8;
                                }
                                acc[i][j] = v4i{0, 0, 0, 0};
                            }
                    } else {
                        float swj[C::FN];
#pragma unroll
                        for (int j = 0; j < C::FN; ++j)
                            swj[j] = sw_in_lds ? sws[sw_slot<C::BN>(g, ccol[j])]
                                               : __builtin_bit_cast(float, bload4(rsw, (uint32_t)(ccol[j] * ng + g) * 4)) *
                                                     0x1p-8f;
#pragma unroll
                        for (int i = 0; i < C::FM; ++i)
#pragma unroll
                            for (int j = 0; j < C::FN; ++j) {
#pragma unroll
                                for (int e = 0; e < 4; ++e)
                                    f[i][j][e] = __builtin_fmaf((float)acc[i][j][e], swj[j], f[i][j][e]);
                                acc[i][j] = v4i{0, 0, 0, 0};
                            }
                    }
                }
            }
        }
        if (more) {
            uint8_t* na = smem + ((kt + 1) & 1) * (C::LDS_A + C::LDS_B);
            r2s<C::A_CH, C::THREADS>(na, ra);
            r2s<C::B_CH, C::THREADS>(na + C::LDS_A, rb);
        }
        __syncthreads();
    }
    if constexpr (!STORE_ACC) {
        const rsrc_t rsx = make_rsrc(s_x + m0, (M - m0) * 4);
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int rl = wm * C::TM + i * 16 + 4 * (lane >> 4) + e;
                const float sx = __builtin_bit_cast(float, bload4(rsx, (uint32_t)rl * 4));
                const int64_t row = m0 + rl;
#pragma unroll
                for (int j = 0; j < C::FN; ++j) {
                    const int64_t col = n0 + ccol[j];
                    if (row < M && col < N) store_out(out, out_dtype, row * N + col, sx * f[i][j][e]);
                }
            }
    }
}

// ---------------------------------------------------------------------------
// W4A4 on the LDS-DMA pipeline: eight waves, wave tile 64 x 64, K advances 64
// packed bytes (128 elements, two MFMA steps) per stage through four LDS
// stages.  A8 (W4A8): the activation operand is int8 codes instead, 128 bytes
// per row and stage (eight 16-byte chunks, XOR-swizzled by row % 8), and each
// fragment's bytes are permuted (v_perm_b32) into the even/odd element order
// the weight's nibble unpack produces, so both operands share one k order;
// the products then carry 16 (weight in the high nibble) instead of 256.  A
// lane's fragment of one step is 8 packed bytes of row l % 16, unpacked into
// the high nibbles: bytes 32 s + 8 (l / 16) of the stage for G = 64, and for
// G >= 128 half s of the 16 bytes 16 (l / 16) .. + 15, read once per stage
// (one 16-byte LDS read instead of two 8-byte ones, which conflict).  The block's
// per-group weight scales (x 2^-8) are staged in LDS as [group][column] when
// they fit.  Operands enter the MFMA in the transposed order of the int8 path
// (lane l, element e: row l % 16, column 4 (l / 16) + e of a fragment).
// ---------------------------------------------------------------------------
constexpr int W4D_SW_LDS = 8192;                 // floats of per-group weight scales kept in LDS

// Accumulator start value of a group: the int32 MFMA sum is added to the bit
// pattern of 1.5 * 2^23, whose binade [2^23, 2^24) has a spacing of 1, so for
// |sum| <= 2^22 the accumulator reads as the float 1.5 * 2^23 + sum and one
// exact subtraction gives float(sum) -- no int-to-float conversion.
constexpr int32_t kAccMagic = 0x4B400000;
constexpr float kAccMagicF = 12582912.0f;

// Chunk swizzle of 128-byte LDS rows (W4A8 activation stages): a 16-byte
// fragment read takes one chunk of 16 consecutive rows, and rows r and r + 8
// (also two rows apart in a 256-byte bank window) get different chunks.
__device__ __forceinline__ int swz128(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// The even/odd order of unpack_hi_nibbles for 16 int8 codes read in order.
__device__ __forceinline__ v4i perm_even_odd(const u32x4& a) {
    return v4i{(int)__builtin_amdgcn_perm(a[1], a[0], 0x06040200u), (int)__builtin_amdgcn_perm(a[1], a[0], 0x07050301u),
               (int)__builtin_amdgcn_perm(a[3], a[2], 0x06040200u), (int)__builtin_amdgcn_perm(a[3], a[2], 0x07050301u)};
}

template <class C, bool A8>
struct W4Stage {
    static_assert(C::A_INS * 16 * C::NW == C::BM && C::B_INS * 16 * C::NW == C::BN, "even stage split");
    static constexpr int A_ROW = A8 ? 128 : 64;                 // activation bytes per row and stage
    static constexpr int LDS_A = C::BM * A_ROW;
    static constexpr int A_INS = A8 ? 2 * C::A_INS : C::A_INS;  // 1 KB DMA instructions per wave
    static constexpr int STAGE = LDS_A + C::LDS_B;
    static constexpr int LDS = C::STAGES * STAGE;
};

// ZX: zero-point activations (codes stored as q - 8, zero-points z_x in
// [0, 15]): the epilogue subtracts (z_x[m] - 8) c_w[n] before the row scale,
// c_w[n] = sum_g s_w[n][g] sum_{k in g} qw[n][k] (launch_w4_column_terms).
template <class C, int G, bool STORE_ACC, bool A8, bool ZX, bool SWL>
__device__ __forceinline__ void w4a4_dma_body(const uint32_t* __restrict__ Xp, const float* __restrict__ s_x,
                                              const uint32_t* __restrict__ Wp, const float* __restrict__ s_w,
                                              int64_t M, int64_t K, int64_t N, void* __restrict__ out,
                                              int out_dtype, int tiles_m, int tiles_n, uint8_t* smem, float* sws,
                                              const int32_t* __restrict__ z_x = nullptr,
                                              const float* __restrict__ c_w = nullptr) {
    constexpr int SPG = G / 64;                       // MFMA steps per group
    // G >= 128: K % G == 0 makes every stage whole, and both steps of a stage
    // fall in one group, so the stage's k order may differ from the packed
    // order as long as both operands take the same one (int32 sums are exact).
    // (The per-group stores of STORE_ACC leave no registers for it.)
    constexpr bool WIDE = SPG >= 2 && !STORE_ACC;
    using S = W4Stage<C, A8>;
    constexpr float SCALE = A8 ? 0x1p-4f : 0x1p-8f;   // the nibble shift(s) in each product
    int tm, tn;
    tile_of_block(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * C::BM, n0 = (int64_t)tn * C::BN;
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int wm = wave / C::WN, wn = wave % C::WN;
    const uint32_t kbytes = (uint32_t)(K / 2);        // packed weight bytes per row
    const uint32_t abytes = A8 ? (uint32_t)K : kbytes;   // activation bytes per row
    const int64_t ng = K / G;
    const rsrc_t rsa = make_rsrc(reinterpret_cast<const uint8_t*>(Xp) + m0 * abytes, (M - m0) * abytes);
    const rsrc_t rsb = make_rsrc(reinterpret_cast<const uint8_t*>(Wp) + n0 * kbytes, (N - n0) * kbytes);

    // SWL: the block's scales staged in LDS (the launcher checks that they fit)
    static_assert(!(SWL && STORE_ACC), "no scales with STORE_ACC");
    constexpr bool sw_in_lds = SWL;
    const rsrc_t rsw = make_rsrc(s_w + (STORE_ACC ? 0 : n0 * ng), STORE_ACC ? 0 : (N - n0) * ng * 4);

    uint32_t oa[S::A_INS], ca[S::A_INS], ob[C::B_INS], cb[C::B_INS];
#pragma unroll
    for (int q = 0; q < S::A_INS; ++q) {
        const int P = (wave * S::A_INS + q) * 64 + lane;
        int r, c;
        if constexpr (A8) {
            r = P >> 3;
            c = (P & 7) ^ swz128(r);
        } else {
            r = P >> 2;
            c = (P & 3) ^ ((r >> 1) & 3);
        }
        oa[q] = (uint32_t)r * abytes + c * 16;
        ca[q] = c * 16;
    }
#pragma unroll
    for (int q = 0; q < C::B_INS; ++q) {
        const int P = (wave * C::B_INS + q) * 64 + lane;
        const int r = P >> 2, c = (P & 3) ^ ((r >> 1) & 3);
        ob[q] = (uint32_t)r * kbytes + c * 16;
        cb[q] = c * 16;
    }
    constexpr int PER_STAGE = S::A_INS + C::B_INS;
    const int nk = (int)((kbytes + C::BK - 1) / C::BK);
    const int nsteps = (int)(K / 64);
    auto issue = [&](int kt) __attribute__((always_inline)) {
        uint8_t* st = smem + (kt % C::STAGES) * S::STAGE;
        const uint32_t k0 = (uint32_t)kt * C::BK;
        const uint32_t a0 = (uint32_t)kt * S::A_ROW;
#pragma unroll
        for (int q = 0; q < S::A_INS; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_void*)(st + (wave * S::A_INS + q) * 1024), 16,
                                                     a0 + ca[q] < abytes ? oa[q] + a0 : kOOB, 0, 0, 0);
#pragma unroll
        for (int q = 0; q < C::B_INS; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_void*)(st + S::LDS_A + (wave * C::B_INS + q) * 1024),
                                                     16, k0 + cb[q] < kbytes ? ob[q] + k0 : kOOB, 0, 0, 0);
    };

    v4i acc[C::FM][C::FN];
    v4f f[C::FM][C::FN];
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
            acc[i][j] = v4i{0, 0, 0, 0};
            f[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
        }
    issue(0);
    if (nk > 1) issue(1);
    if (nk > 2) issue(2);
    // the block's scales, staged while the first stages' loads are in flight
    if constexpr (sw_in_lds) {
        // all loads issued before the first write: one memory latency, not one per element
        constexpr int PER = W4D_SW_LDS / C::THREADS;
        const int total = (int)ng * C::BN;
        float v[PER];
#pragma unroll
        for (int it = 0; it < PER; ++it) {
            const int t = threadIdx.x + it * C::THREADS;                // coalesced over g
            v[it] = __builtin_bit_cast(float, bload4(rsw, (uint32_t)(t < total ? t : 0) * 4));
        }
#pragma unroll
        for (int it = 0; it < PER; ++it) {
            const int t = threadIdx.x + it * C::THREADS;
            const int cc = t / (int)ng, g = t - cc * (int)ng;
            if (t < total) sws[sw_slot<C::BN>(g, cc)] = v[it] * SCALE;
        }
    }
    __syncthreads();
    // f += (accumulator - magic) * (group g's scale), per output
    auto dequant = [&](int g) __attribute__((always_inline)) {
        v4f swj[C::FN];
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
            const int cl = wn * C::TN + j * 16 + 4 * (lane >> 4);   // block-local column
            if constexpr (sw_in_lds) {
                swj[j] = *reinterpret_cast<const v4f*>(sws + sw_slot<C::BN>(g, cl));
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    swj[j][e] = __builtin_bit_cast(float, bload4(rsw, (uint32_t)((cl + e) * ng + g) * 4)) * SCALE;
            }
        }
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int j = 0; j < C::FN; ++j) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    // (a named copy: clang's __builtin_bit_cast of a vector element
                    // expression reads element 0)
                    const int32_t a = acc[i][j][e];
                    f[i][j][e] = __builtin_fmaf(__builtin_bit_cast(float, a) - kAccMagicF, swj[j][e], f[i][j][e]);
                }
                if constexpr (SPG > 2) acc[i][j] = v4i{kAccMagic, kAccMagic, kAccMagic, kAccMagic};
            }
    };
    if constexpr (!STORE_ACC && SPG > 2) {
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int j = 0; j < C::FN; ++j) acc[i][j] = v4i{kAccMagic, kAccMagic, kAccMagic, kAccMagic};
    }
    for (int kt = 0; kt < nk; ++kt) {
        const int ahead = (kt + 2 < nk - 1 ? kt + 2 : nk - 1) - kt;   // stages issued after kt
        if (ahead >= 2)
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * PER_STAGE));
        else if (ahead == 1)
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(PER_STAGE));
        else
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        block_barrier();
        if (kt + 3 < nk) issue(kt + 3);
        const uint8_t* sa = smem + (kt % C::STAGES) * S::STAGE;
        const uint8_t* sb = sa + S::LDS_A;
        // WIDE: one 16-byte read per packed fragment covers the stage; step
        // s2 takes its 8-byte half s2 (elements 32 (l / 16) + 16 s2 .. + 15).
        u32x4 wa[WIDE && !A8 ? C::FM : 1], wb[WIDE ? C::FN : 1];
        if constexpr (WIDE) {
#pragma unroll
            for (int j = 0; j < C::FN; ++j)
                wb[j] = *reinterpret_cast<const u32x4*>(sb + swz64(wn * C::TN + j * 16 + (lane & 15), lane >> 4));
            if constexpr (!A8) {
#pragma unroll
                for (int i = 0; i < C::FM; ++i)
                    wa[i] = *reinterpret_cast<const u32x4*>(sa + swz64(wm * C::TM + i * 16 + (lane & 15), lane >> 4));
            }
        }
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const int step = 2 * kt + s2;
            if (!WIDE && step >= nsteps) break;
            const int byte = s2 * 32 + (lane >> 4) * 8;
            const int c = byte >> 4, within = byte & 15;
            v4i fa[C::FM], fb[C::FN];
#pragma unroll
            for (int i = 0; i < C::FM; ++i) {
                const int r = wm * C::TM + i * 16 + (lane & 15);
                if constexpr (A8) {
                    // elements 16 c8 .. 16 c8 + 15, the ones the weight fragment holds
                    const int c8 = WIDE ? 2 * (lane >> 4) + s2 : 4 * s2 + (lane >> 4);
                    fa[i] = perm_even_odd(*reinterpret_cast<const u32x4*>(sa + r * 128 + ((c8 ^ swz128(r)) * 16)));
                } else if constexpr (WIDE) {
                    fa[i] = unpack_hi_nibbles(u32x2{wa[i][2 * s2], wa[i][2 * s2 + 1]});
                } else {
                    fa[i] = unpack_hi_nibbles(*reinterpret_cast<const u32x2*>(sa + swz64(r, c) + within));
                }
            }
#pragma unroll
            for (int j = 0; j < C::FN; ++j) {
                if constexpr (WIDE)
                    fb[j] = unpack_hi_nibbles(u32x2{wb[j][2 * s2], wb[j][2 * s2 + 1]});
                else
                    fb[j] = unpack_hi_nibbles(
                        *reinterpret_cast<const u32x2*>(sb + swz64(wn * C::TN + j * 16 + (lane & 15), c) + within));
            }
            // A group of at most two steps starts at a step known at compile
            // time (step = 2 kt + s2): its first MFMA takes the start value (zero,
            // or kAccMagic where the dequant reads the sum as a float) instead of
            // resetting the accumulators after each dequant.
            const bool fresh = SPG <= 2 && (SPG == 1 || s2 == 0);
            const v4i acc0 = STORE_ACC ? v4i{0, 0, 0, 0} : v4i{kAccMagic, kAccMagic, kAccMagic, kAccMagic};
#pragma unroll
            for (int i = 0; i < C::FM; ++i)
#pragma unroll
                for (int j = 0; j < C::FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fb[j], fa[i], fresh ? acc0 : acc[i][j], 0, 0, 0);
            if ((step + 1) % SPG == 0) {
                const int g = step / SPG;
                if constexpr (STORE_ACC) {
                    int32_t* accp = static_cast<int32_t*>(out);
#pragma unroll
                    for (int i = 0; i < C::FM; ++i) {
                        const int64_t row = m0 + wm * C::TM + i * 16 + (lane & 15);
#pragma unroll
                        for (int j = 0; j < C::FN; ++j) {
                            const int64_t col = n0 + wn * C::TN + j * 16 + 4 * (lane >> 4);
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                if (row < M && col + e < N)
                                    accp[(row * N + col + e) * ng + g] = acc[i][j][e] >> (A8 ? 4 : 8);
                            if constexpr (SPG > 2) acc[i][j] = v4i{0, 0, 0, 0};
                        }
                    }
                } else {
                    dequant(g);
                }
            }
        }
    }
    // the epilogue's row and column terms, loaded together ahead of their use
    float sx[C::FM], zx[C::FM];
    v4f cw[ZX ? C::FN : 1];
    if constexpr (!STORE_ACC) {
        const rsrc_t rsx = make_rsrc(s_x + m0, (M - m0) * 4);
        const rsrc_t rzx = make_rsrc(ZX ? z_x + m0 : nullptr, ZX ? (M - m0) * 4 : 0);
#pragma unroll
        for (int i = 0; i < C::FM; ++i) {
            const int rl = wm * C::TM + i * 16 + (lane & 15);
            sx[i] = __builtin_bit_cast(float, bload4(rsx, (uint32_t)rl * 4));
            zx[i] = ZX ? (float)((int32_t)bload4(rzx, (uint32_t)rl * 4) - 8) : 0.0f;
        }
        if constexpr (ZX) {
            const rsrc_t rcw = make_rsrc(c_w + n0, (N - n0) * 4);
#pragma unroll
            for (int j = 0; j < C::FN; ++j) {
                const int cl = wn * C::TN + j * 16 + 4 * (lane >> 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) cw[j][e] = __builtin_bit_cast(float, bload4(rcw, (uint32_t)(cl + e) * 4));
            }
        }
    }
    if constexpr (!STORE_ACC) {
        const bool vec = (N & 3) == 0;
#pragma unroll
        for (int i = 0; i < C::FM; ++i) {
            const int rl = wm * C::TM + i * 16 + (lane & 15);
            const int64_t row = m0 + rl;
#pragma unroll
            for (int j = 0; j < C::FN; ++j) {
                const int64_t col = n0 + wn * C::TN + j * 16 + 4 * (lane >> 4);
                v4f o;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if constexpr (ZX)
                        o[e] = sx[i] * __builtin_fmaf(-zx[i], cw[j][e], f[i][j][e]);
                    else
                        o[e] = sx[i] * f[i][j][e];
                }
                if (row < M && col < N) store_out4(out, out_dtype, row * N + col, o, vec, (int)(N - col < 4 ? N - col : 4));
            }
        }
    }
}

template <class C, int G, bool STORE_ACC, bool SWL>
__global__ __launch_bounds__(C::THREADS) void k_gemm_w4a4_dma(const uint32_t* __restrict__ Xp,
                                                              const float* __restrict__ s_x,
                                                              const uint32_t* __restrict__ Wp,
                                                              const float* __restrict__ s_w, int64_t M, int64_t K,
                                                              int64_t N, void* __restrict__ out, int out_dtype,
                                                              int tiles_m, int tiles_n) {
    // one LDS object, the stages and then the scale table: with a second
    // __shared__ array the compiler makes each fragment read wait for every
    // stage load in flight, which serializes the pipeline
    __shared__ __attribute__((aligned(16))) uint8_t smem[C::LDS + (SWL ? 4 * W4D_SW_LDS : 0)];
    float* sws = reinterpret_cast<float*>(smem + C::LDS);
    w4a4_dma_body<C, G, STORE_ACC, false, false, SWL>(Xp, s_x, Wp, s_w, M, K, N, out, out_dtype, tiles_m, tiles_n,
                                                      smem, sws);
}

// W4A4 with zero-point activations.
template <class C, int G, bool SWL>
__global__ __launch_bounds__(C::THREADS) void k_gemm_w4a4z_dma(const uint32_t* __restrict__ Xp,
                                                               const float* __restrict__ s_x,
                                                               const int32_t* __restrict__ z_x,
                                                               const uint32_t* __restrict__ Wp,
                                                               const float* __restrict__ s_w,
                                                               const float* __restrict__ c_w, int64_t M, int64_t K,
                                                               int64_t N, void* __restrict__ out, int out_dtype,
                                                               int tiles_m, int tiles_n) {
    // one LDS object, the stages and then the scale table: with a second
    // __shared__ array the compiler makes each fragment read wait for every
    // stage load in flight, which serializes the pipeline
    __shared__ __attribute__((aligned(16))) uint8_t smem[C::LDS + (SWL ? 4 * W4D_SW_LDS : 0)];
    float* sws = reinterpret_cast<float*>(smem + C::LDS);
    w4a4_dma_body<C, G, false, false, true, SWL>(Xp, s_x, Wp, s_w, M, K, N, out, out_dtype, tiles_m, tiles_n, smem,
                                                 sws, z_x, c_w);
}

// W4A8: int8 activation codes Xq [M x K] against the packed int4 weight.
template <class C, int G, bool STORE_ACC, bool SWL>
__global__ __launch_bounds__(C::THREADS) void k_gemm_w4a8_dma(const int8_t* __restrict__ Xq,
                                                              const float* __restrict__ s_x,
                                                              const uint32_t* __restrict__ Wp,
                                                              const float* __restrict__ s_w, int64_t M, int64_t K,
                                                              int64_t N, void* __restrict__ out, int out_dtype,
                                                              int tiles_m, int tiles_n) {
    // one LDS object, the stages and then the scale table: with a second
    // __shared__ array the compiler makes each fragment read wait for every
    // stage load in flight, which serializes the pipeline
    __shared__ __attribute__((aligned(16))) uint8_t smem[W4Stage<C, true>::LDS + (SWL ? 4 * W4D_SW_LDS : 0)];
    float* sws = reinterpret_cast<float*>(smem + W4Stage<C, true>::LDS);
    w4a4_dma_body<C, G, STORE_ACC, true, false, SWL>(reinterpret_cast<const uint32_t*>(Xq), s_x, Wp, s_w, M, K, N,
                                                     out, out_dtype, tiles_m, tiles_n, smem, sws);
}

// ---------------------------------------------------------------------------
// W4 GEMMs with groups smaller than one MFMA step (G = 8, 16, 32: a 64-deep
// MFMA would sum over several groups).  Each group's int32 sum is formed on
// the VALU: v_dot8_i32_i4 (eight signed nibble products per instruction)
// for int4 activations; for int8 activations (A8) v_dot4_i32_i8 on the codes
// in even / odd element order against the weight nibbles moved into the high
// half of each byte (products x 16, the 2^-4 is exact in the dequant).  64 x 64
// outputs per 256-thread block, 4 x 4 per thread; K in chunks of 64 elements
// staged in LDS with the chunk's per-group weight scales.
//   out[m][n] = s_x[m] (sum_g s_w[n][g] acc_g[m][n] - (ZX ? (z_x[m] - 8) c_w[n] : 0))
// or, with STORE_ACC, acc_g[m][n] into acc [M x N x K/G] (int32).
// ---------------------------------------------------------------------------
template <int G, bool A8, bool ZX, bool STORE_ACC>
__global__ __launch_bounds__(256) void k_gemm_w4_small_g(const uint8_t* __restrict__ Xa, const float* __restrict__ s_x,
                                                         const int32_t* __restrict__ z_x,
                                                         const uint32_t* __restrict__ Wp,
                                                         const float* __restrict__ s_w, const float* __restrict__ c_w,
                                                         int64_t M, int64_t K, int64_t N, void* __restrict__ out,
                                                         int out_dtype) {
    static_assert(G == 8 || G == 16 || G == 32, "groups below one MFMA step");
    constexpr int KC = 64;                            // K elements per chunk
    constexpr int AW = A8 ? KC / 4 : KC / 8;          // activation words per row and chunk
    constexpr int WW = KC / 8;                        // weight words per row and chunk
    constexpr int NGC = KC / G;                       // groups per chunk
    __shared__ uint32_t As[64][AW + 1];
    __shared__ uint32_t Bs[64][WW + 1];
    __shared__ float Ss[64][NGC + 1];
    const int64_t m0 = (int64_t)blockIdx.y * 64, n0 = (int64_t)blockIdx.x * 64;
    const int t = threadIdx.x, tx = t & 15, ty = t >> 4;
    const int64_t ng = K / G;
    const uint32_t abytes = (uint32_t)(A8 ? K : K / 2), wbytes = (uint32_t)(K / 2);
    const rsrc_t ra = make_rsrc(Xa + m0 * abytes, (M - m0) * abytes);
    const rsrc_t rw = make_rsrc(reinterpret_cast<const uint8_t*>(Wp) + n0 * wbytes, (N - n0) * wbytes);
    const rsrc_t rs = make_rsrc(STORE_ACC ? nullptr : s_w + n0 * ng, STORE_ACC ? 0 : (N - n0) * ng * 4);
    float f[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) f[r][c] = 0.0f;
    for (int64_t kc = 0; kc < K; kc += KC) {
        // stage the chunk: 16-byte loads, bytes past the row's end read zero
        const uint32_t ka = (uint32_t)(A8 ? kc : kc / 2), kw = (uint32_t)(kc / 2);
        for (int q = t; q < 64 * (AW / 4); q += 256) {
            const int r = q / (AW / 4), c4 = q % (AW / 4);
            const uint32_t o = ka + 16 * c4;
            const u32x4 v = bload16(ra, o < abytes ? (uint32_t)r * abytes + o : kOOB);
#pragma unroll
            for (int d = 0; d < 4; ++d) As[r][4 * c4 + d] = v[d];
        }
        for (int q = t; q < 64 * (WW / 4); q += 256) {
            const int r = q / (WW / 4), c4 = q % (WW / 4);
            const uint32_t o = kw + 16 * c4;
            const u32x4 v = bload16(rw, o < wbytes ? (uint32_t)r * wbytes + o : kOOB);
#pragma unroll
            for (int d = 0; d < 4; ++d) Bs[r][4 * c4 + d] = v[d];
        }
        if constexpr (!STORE_ACC) {
            for (int q = t; q < 64 * NGC; q += 256) {
                const int c = q / NGC, gg = q % NGC;
                const int64_t g = kc / G + gg;
                Ss[c][gg] = g < ng ? __builtin_bit_cast(float, bload4(rs, (uint32_t)(c * ng + g) * 4)) : 0.0f;
            }
        }
        __syncthreads();
#pragma unroll
        for (int gg = 0; gg < NGC; ++gg) {
            int acc[4][4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[r][c] = 0;
#pragma unroll
            for (int w = 0; w < G / 8; ++w) {            // weight words of the group
                const int wi = gg * (G / 8) + w;
                uint32_t b[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) b[c] = Bs[4 * tx + c][wi];
                if constexpr (A8) {
                    uint32_t be[4], bo[4];
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        be[c] = (b[c] << 4) & 0xF0F0F0F0u;   // elements 0, 2, 4, 6 (x 16)
                        bo[c] = b[c] & 0xF0F0F0F0u;          // elements 1, 3, 5, 7 (x 16)
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const uint32_t a0 = As[4 * ty + r][2 * wi], a1 = As[4 * ty + r][2 * wi + 1];
                        const int ae = (int)__builtin_amdgcn_perm(a1, a0, 0x06040200u);
                        const int ao = (int)__builtin_amdgcn_perm(a1, a0, 0x07050301u);
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            acc[r][c] = __builtin_amdgcn_sdot4(ae, (int)be[c], acc[r][c], false);
                            acc[r][c] = __builtin_amdgcn_sdot4(ao, (int)bo[c], acc[r][c], false);
                        }
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int a = (int)As[4 * ty + r][wi];
#pragma unroll
                        for (int c = 0; c < 4; ++c) acc[r][c] = __builtin_amdgcn_sdot8(a, (int)b[c], acc[r][c], false);
                    }
                }
            }
            const int64_t g = kc / G + gg;
            if constexpr (STORE_ACC) {
                if (g < ng) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int64_t m = m0 + 4 * ty + r;
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            const int64_t n = n0 + 4 * tx + c;
                            if (m < M && n < N)
                                static_cast<int32_t*>(out)[(m * N + n) * ng + g] = A8 ? acc[r][c] >> 4 : acc[r][c];
                        }
                    }
                }
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        f[r][c] = __builtin_fmaf(Ss[4 * tx + c][gg] * (A8 ? 0x1p-4f : 1.0f), (float)acc[r][c], f[r][c]);
            }
        }
        __syncthreads();
    }
    if constexpr (!STORE_ACC) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t m = m0 + 4 * ty + r;
            if (m >= M) continue;
            const float sx = s_x[m];
            const float zp = ZX ? (float)(z_x[m] - 8) : 0.0f;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int64_t n = n0 + 4 * tx + c;
                if (n >= N) continue;
                float v = f[r][c];
                if constexpr (ZX) v = __builtin_fmaf(-zp, c_w[n], v);
                store_out(out, out_dtype, m * N + n, sx * v);
            }
        }
    }
}

template <bool A8, bool ZX, bool STORE_ACC>
static hipError_t launch_w4_small_g(const uint8_t* Xa, const float* s_x, const int32_t* z_x, const uint32_t* Wp,
                                    const float* s_w, const float* c_w, int64_t M, int64_t K, int64_t N, int G,
                                    void* out, int out_dtype, hipStream_t st) {
    const dim3 grid((unsigned)((N + 63) / 64), (unsigned)((M + 63) / 64));
    switch (G) {
        case 8:
            hipLaunchKernelGGL((k_gemm_w4_small_g<8, A8, ZX, STORE_ACC>), grid, dim3(256), 0, st, Xa, s_x, z_x, Wp, s_w,
                               c_w, M, K, N, out, out_dtype);
            break;
        case 16:
            hipLaunchKernelGGL((k_gemm_w4_small_g<16, A8, ZX, STORE_ACC>), grid, dim3(256), 0, st, Xa, s_x, z_x, Wp,
                               s_w, c_w, M, K, N, out, out_dtype);
            break;
        case 32:
            hipLaunchKernelGGL((k_gemm_w4_small_g<32, A8, ZX, STORE_ACC>), grid, dim3(256), 0, st, Xa, s_x, z_x, Wp,
                               s_w, c_w, M, K, N, out, out_dtype);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

using CfgW4 = CfgD<128, 256, 2, 4>;     // 8 waves, wave tile 64 x 64, LDS-DMA stages

// Whether a CfgW4 block's per-group weight scales fit the LDS table.
static bool w4_scales_fit(int64_t K, int G) { return (K / G) * CfgW4::BN <= W4D_SW_LDS; }

template <int G, bool STORE_ACC>
static void w4a4_dispatch(const uint32_t* Xp, const float* s_x, const uint32_t* Wp, const float* s_w, int64_t M,
                          int64_t K, int64_t N, void* out, int out_dtype, hipStream_t st) {
    int tm, tn;
    if (((M + 127) / 128) * ((N + 255) / 256) >= 256) {
        dim3 g = grid_of<CfgW4>(M, N, tm, tn);
        if (!STORE_ACC && w4_scales_fit(K, G))
            hipLaunchKernelGGL((k_gemm_w4a4_dma<CfgW4, G, STORE_ACC, !STORE_ACC>), g, dim3(CfgW4::THREADS), 0, st, Xp,
                               s_x, Wp, s_w, M, K, N, out, out_dtype, tm, tn);
        else
            hipLaunchKernelGGL((k_gemm_w4a4_dma<CfgW4, G, STORE_ACC, false>), g, dim3(CfgW4::THREADS), 0, st, Xp, s_x,
                               Wp, s_w, M, K, N, out, out_dtype, tm, tn);
    } else if (((M + 127) / 128) * ((N + 127) / 128) >= 256) {
        dim3 g = grid_of<CfgMidR>(M, N, tm, tn);
        hipLaunchKernelGGL((k_gemm_w4a4<CfgMidR, G, STORE_ACC>), g, dim3(CfgMidR::THREADS), 0, st, Xp, s_x, Wp, s_w,
                           M, K, N, out, out_dtype, tm, tn);
    } else {
        dim3 g = grid_of<CfgSmall>(M, N, tm, tn);
        hipLaunchKernelGGL((k_gemm_w4a4<CfgSmall, G, STORE_ACC>), g, dim3(CfgSmall::THREADS), 0, st, Xp, s_x, Wp,
                           s_w, M, K, N, out, out_dtype, tm, tn);
    }
}

hipError_t launch_gemm_w4a4(const uint32_t* Xp, const float* s_x, const uint32_t* Wp, const float* s_w,
                            int64_t M, int64_t K, int64_t N, int G, void* out, int out_dtype, hipStream_t st) {
    switch (G) {
        case 64: w4a4_dispatch<64, false>(Xp, s_x, Wp, s_w, M, K, N, out, out_dtype, st); break;
        case 128: w4a4_dispatch<128, false>(Xp, s_x, Wp, s_w, M, K, N, out, out_dtype, st); break;
        case 256: w4a4_dispatch<256, false>(Xp, s_x, Wp, s_w, M, K, N, out, out_dtype, st); break;
        default:
            return launch_w4_small_g<false, false, false>(reinterpret_cast<const uint8_t*>(Xp), s_x, nullptr, Wp, s_w,
                                                          nullptr, M, K, N, G, out, out_dtype, st);
    }
    return hipGetLastError();
}

template <int G>
static void w4a4z_dispatch(const uint32_t* Xp, const float* s_x, const int32_t* z_x, const uint32_t* Wp,
                           const float* s_w, const float* c_w, int64_t M, int64_t K, int64_t N, void* out,
                           int out_dtype, hipStream_t st) {
    int tm, tn;
    dim3 g = grid_of<CfgW4>(M, N, tm, tn);
    if (w4_scales_fit(K, G))
        hipLaunchKernelGGL((k_gemm_w4a4z_dma<CfgW4, G, true>), g, dim3(CfgW4::THREADS), 0, st, Xp, s_x, z_x, Wp, s_w,
                           c_w, M, K, N, out, out_dtype, tm, tn);
    else
        hipLaunchKernelGGL((k_gemm_w4a4z_dma<CfgW4, G, false>), g, dim3(CfgW4::THREADS), 0, st, Xp, s_x, z_x, Wp, s_w,
                           c_w, M, K, N, out, out_dtype, tm, tn);
}

hipError_t launch_gemm_w4a4_asym(const uint32_t* Xp, const float* s_x, const int32_t* z_x, const uint32_t* Wp,
                                 const float* s_w, const float* c_w, int64_t M, int64_t K, int64_t N, int G,
                                 void* out, int out_dtype, hipStream_t st) {
    switch (G) {
        case 64: w4a4z_dispatch<64>(Xp, s_x, z_x, Wp, s_w, c_w, M, K, N, out, out_dtype, st); break;
        case 128: w4a4z_dispatch<128>(Xp, s_x, z_x, Wp, s_w, c_w, M, K, N, out, out_dtype, st); break;
        case 256: w4a4z_dispatch<256>(Xp, s_x, z_x, Wp, s_w, c_w, M, K, N, out, out_dtype, st); break;
        default:
            return launch_w4_small_g<false, true, false>(reinterpret_cast<const uint8_t*>(Xp), s_x, z_x, Wp, s_w, c_w, M,
                                                         K, N, G, out, out_dtype, st);
    }
    return hipGetLastError();
}

template <int G, bool STORE_ACC>
static void w4a8_dispatch(const int8_t* Xq, const float* s_x, const uint32_t* Wp, const float* s_w, int64_t M,
                          int64_t K, int64_t N, void* out, int out_dtype, hipStream_t st) {
    int tm, tn;
    dim3 g = grid_of<CfgW4>(M, N, tm, tn);
    if (!STORE_ACC && w4_scales_fit(K, G))
        hipLaunchKernelGGL((k_gemm_w4a8_dma<CfgW4, G, STORE_ACC, !STORE_ACC>), g, dim3(CfgW4::THREADS), 0, st, Xq,
                           s_x, Wp, s_w, M, K, N, out, out_dtype, tm, tn);
    else
        hipLaunchKernelGGL((k_gemm_w4a8_dma<CfgW4, G, STORE_ACC, false>), g, dim3(CfgW4::THREADS), 0, st, Xq, s_x, Wp,
                           s_w, M, K, N, out, out_dtype, tm, tn);
}

hipError_t launch_gemm_w4a8(const int8_t* Xq, const float* s_x, const uint32_t* Wp, const float* s_w, int64_t M,
                            int64_t K, int64_t N, int G, void* out, int out_dtype, hipStream_t st) {
    switch (G) {
        case 64: w4a8_dispatch<64, false>(Xq, s_x, Wp, s_w, M, K, N, out, out_dtype, st); break;
        case 128: w4a8_dispatch<128, false>(Xq, s_x, Wp, s_w, M, K, N, out, out_dtype, st); break;
        case 256: w4a8_dispatch<256, false>(Xq, s_x, Wp, s_w, M, K, N, out, out_dtype, st); break;
        default:
            return launch_w4_small_g<true, false, false>(reinterpret_cast<const uint8_t*>(Xq), s_x, nullptr, Wp, s_w,
                                                         nullptr, M, K, N, G, out, out_dtype, st);
    }
    return hipGetLastError();
}

hipError_t launch_gemm_w4a8_group_acc(const int8_t* Xq, const uint32_t* Wp, int64_t M, int64_t K, int64_t N, int G,
                                      int32_t* acc, hipStream_t st) {
    switch (G) {
        case 64: w4a8_dispatch<64, true>(Xq, nullptr, Wp, nullptr, M, K, N, acc, 0, st); break;
        case 128: w4a8_dispatch<128, true>(Xq, nullptr, Wp, nullptr, M, K, N, acc, 0, st); break;
        case 256: w4a8_dispatch<256, true>(Xq, nullptr, Wp, nullptr, M, K, N, acc, 0, st); break;
        default:
            return launch_w4_small_g<true, false, true>(reinterpret_cast<const uint8_t*>(Xq), nullptr, nullptr, Wp,
                                                        nullptr, nullptr, M, K, N, G, acc, 0, st);
    }
    return hipGetLastError();
}

hipError_t launch_gemm_w4a4_group_acc(const uint32_t* Xp, const uint32_t* Wp, int64_t M, int64_t K, int64_t N,
                                      int G, int32_t* acc, hipStream_t st) {
    switch (G) {
        case 64: w4a4_dispatch<64, true>(Xp, nullptr, Wp, nullptr, M, K, N, acc, 0, st); break;
        case 128: w4a4_dispatch<128, true>(Xp, nullptr, Wp, nullptr, M, K, N, acc, 0, st); break;
        case 256: w4a4_dispatch<256, true>(Xp, nullptr, Wp, nullptr, M, K, N, acc, 0, st); break;
        default:
            return launch_w4_small_g<false, false, true>(reinterpret_cast<const uint8_t*>(Xp), nullptr, nullptr, Wp,
                                                         nullptr, nullptr, M, K, N, G, acc, 0, st);
    }
    return hipGetLastError();
}


template <bool ZW>
static void launch_asym_cfgs(const int8_t* Xq, const int8_t* Wq, int64_t M, int64_t K, int64_t N,
                             const AsymEpilogue& ep, hipStream_t st) {
    int tm, tn;
    if (pick_cfg(M, N) == 2) {
        if (const int tsn = wide_stride(M, N)) {
            tm = (int)((M + 255) / 256);
            tn = (int)((N + tsn - 1) / tsn);
            hipLaunchKernelGGL((k_gemm_i8_asym<CfgWide, ZW>), dim3((unsigned)(tm * tn)), dim3(CfgWide::THREADS), 0,
                               st, Xq, Wq, M, K, N, ep, tm, tn, tsn);
            return;
        }
        if (const int64_t split = tail_split(M, N)) {
            dim3 g = grid_of<CfgBig>(M, split, tm, tn);
            hipLaunchKernelGGL((k_gemm_i8_asym<CfgBig, ZW>), g, dim3(CfgBig::THREADS), 0, st, Xq, Wq, M, K, split,
                               ep, tm, tn, CfgBig::BN);
            const int esz = ep.out_dtype == 0 ? 4 : 2;
            AsymEpilogue et = ep;
            et.s_w = ep.s_w + split;
            et.r_w = ep.r_w + split;
            et.z_w = ep.z_w ? ep.z_w + split : nullptr;
            et.out = static_cast<uint8_t*>(ep.out) + split * esz;
            g = grid_of<CfgTail>(M, N - split, tm, tn);
            hipLaunchKernelGGL((k_gemm_i8_asym<CfgTail, ZW>), g, dim3(CfgTail::THREADS), 0, st, Xq, Wq + split * K,
                               M, K, N - split, et, tm, tn, CfgTail::BN);
            return;
        }
    }
    switch (pick_cfg(M, N)) {
        case 2: {
            dim3 g = grid_of<CfgBig>(M, N, tm, tn);
            hipLaunchKernelGGL((k_gemm_i8_asym<CfgBig, ZW>), g, dim3(CfgBig::THREADS), 0, st, Xq, Wq, M, K, N, ep,
                               tm, tn, CfgBig::BN);
            break;
        }
        case 1: {
            dim3 g = grid_of<CfgMid>(M, N, tm, tn);
            hipLaunchKernelGGL((k_gemm_i8_asym<CfgMid, ZW>), g, dim3(CfgMid::THREADS), 0, st, Xq, Wq, M, K, N, ep,
                               tm, tn, CfgMid::BN);
            break;
        }
        default: {
            dim3 g = grid_of<CfgSmall>(M, N, tm, tn);
            hipLaunchKernelGGL((k_gemm_i8_asym<CfgSmall, ZW>), g, dim3(CfgSmall::THREADS), 0, st, Xq, Wq, M, K, N,
                               ep, tm, tn, CfgSmall::BN);
        }
    }
}

hipError_t launch_gemm_i8_asym(const int8_t* Xq, const int8_t* Wq, int64_t M, int64_t K, int64_t N,
                               const AsymEpilogue& ep, hipStream_t st) {
    if (ep.z_w)
        launch_asym_cfgs<true>(Xq, Wq, M, K, N, ep, st);
    else
        launch_asym_cfgs<false>(Xq, Wq, M, K, N, ep, st);
    return hipGetLastError();
}

}  // namespace qa
