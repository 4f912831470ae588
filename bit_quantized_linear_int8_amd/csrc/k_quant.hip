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
//
// All global reads are raw buffer loads (hardware range check, zeros outside)
// so every load of a wave is issued before the first one is waited for.
#include "qa_device.hpp"
#include "qa_launch.hpp"

namespace qa {

// ---------------------------------------------------------------------------
// Outlier columns.  A block owns a strip of 64 columns (one 128-byte line per
// row: 8 lanes x 16 bytes) and a segment of rows; a wave instruction reads 8
// full lines.  The column max runs on the sign-cleared fp16 bit patterns
// (magnitudes of fp16 values order like their bits) with packed 16-bit max,
// folded across lanes and waves.  Column j is an outlier when its max exceeds
// the threshold; lane 0 writes the strip's 64 outlier bits as one 64-bit
// word of this row segment's partial flag set (plain stores: no atomics, no
// clearing), and the column max of the segment when the caller asks for it.
// Consumers OR the partial words (and max the partial column maxima).
// ---------------------------------------------------------------------------
constexpr int OC_STRIP = 64;
constexpr int OC_UNR = 8;                       // loads in flight per lane
constexpr int OC_PASS = 256 * 64;               // columns compacted per pass

constexpr int OC_SEG_MAX = 8;                  // row segments of the scan (partial flag sets)

template <bool WANT_MAX>
__global__ __launch_bounds__(256) void k_outlier_scan(const uint16_t* __restrict__ X, int64_t M, int64_t K,
                                                      float tau, unsigned long long* __restrict__ flags_p,
                                                      uint32_t* __restrict__ cmax_p) {
    __shared__ uint32_t red[4][32];
    const int t = threadIdx.x, lane = t & 63, wave = wave_id();
    const int64_t c0 = (int64_t)blockIdx.x * OC_STRIP;
    const int64_t nw = (K + 63) / 64;
    const int seg = blockIdx.y, nseg = gridDim.y;
    const int chunk = lane & 7, rsub = lane >> 3;
    const uint32_t coff = (c0 + chunk * 8 + 8 <= K) ? (uint32_t)chunk * 16 : kOOB;
    uint32_t m[4] = {0u, 0u, 0u, 0u};
    // this segment's row blocks: rb = 256 (seg + nseg j)
    for (int64_t rb = (int64_t)seg * 32 * OC_UNR; rb < M; rb += (int64_t)nseg * 32 * OC_UNR) {
        const int64_t nr = M - rb < 32 * OC_UNR ? M - rb : 32 * OC_UNR;
        const rsrc_t rs = make_rsrc(X + rb * K + c0, (nr * K - c0) * 2);   // rows past the block read zeros
        u32x4 v[OC_UNR];
#pragma unroll
        for (int u = 0; u < OC_UNR; ++u) {
            const uint32_t r = (uint32_t)(u * 32 + wave * 8 + rsub);
            v[u] = bload16(rs, coff == kOOB ? kOOB : r * (uint32_t)K * 2 + coff);
        }
#pragma unroll
        for (int u = 0; u < OC_UNR; ++u)
#pragma unroll
            for (int d = 0; d < 4; ++d) m[d] = pk_max_u16(m[d], v[u][d] & 0x7fff7fffu);
    }
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int o = 8; o < 64; o <<= 1) m[d] = pk_max_u16(m[d], (uint32_t)__shfl_xor((int)m[d], o, QA_WAVE));
    if (rsub == 0) {
#pragma unroll
        for (int d = 0; d < 4; ++d) red[wave][chunk * 4 + d] = m[d];
    }
    __syncthreads();
    if (wave == 0) {
        // lane j: column c0 + j.  Every (strip, segment) slot is overwritten, so
        // the scratch needs no clearing between calls.
        const int w = lane >> 1;
        const uint32_t a = pk_max_u16(pk_max_u16(red[0][w], red[1][w]), pk_max_u16(red[2][w], red[3][w]));
        const float cm = h2f((uint16_t)((lane & 1) ? (a >> 16) : (a & 0xffffu)));
        const int64_t col = c0 + lane;
        const unsigned long long bits = __ballot(col < K && cm > tau);
        if (lane == 0) flags_p[(int64_t)seg * nw + blockIdx.x] = bits;
        if (WANT_MAX && col < K) cmax_p[(int64_t)seg * K + col] = __builtin_bit_cast(uint32_t, cm);
    }
}

// Ascending outlier list from the flag words: thread t owns columns
// [t C, t C + C) of each pass of up to 16384 columns, so one block-wide scan of
// the per-thread counts places every outlier.  Optionally writes the byte
// mask and the column max.  Run by one block of 256 threads.
// `word(w)` returns flag word w (the OR of the scan's partial words).
template <class WordF>
__device__ void outlier_compact(WordF word, const uint32_t* __restrict__ cmax_p, int nseg, int64_t K,
                                uint8_t* __restrict__ mask, int32_t* __restrict__ idx, int32_t* __restrict__ count,
                                float* __restrict__ colmax_out, int* wsum) {
    const int t = threadIdx.x, lane = t & 63, wave = wave_id();
    int running = 0;
    for (int64_t pb = 0; pb < K; pb += OC_PASS) {
        const int64_t pk = K - pb < OC_PASS ? K - pb : OC_PASS;
        const int C = (int)((pk + 255) / 256);                // <= 64 columns per thread
        const int64_t cb = pb + (int64_t)t * C;
        // the (at most two) flag words covering [cb, cb + C)
        const int64_t w0 = cb >> 6;
        const unsigned long long f0 = word(w0), f1 = word(w0 + 1);
        const int sh = (int)(cb & 63);
        unsigned long long fl = sh ? ((f0 >> sh) | (f1 << (64 - sh))) : f0;
        int64_t lim = pb + pk - cb;                            // valid columns of this thread
        lim = lim < 0 ? 0 : (lim > C ? C : lim);
        fl = lim >= 64 ? fl : (fl & ((1ull << lim) - 1ull));
        if (mask || colmax_out) {
            for (int i = 0; i < (int)lim; ++i) {
                const int64_t col = cb + i;
                if (mask) mask[col] = (uint8_t)((fl >> i) & 1ull);
                if (colmax_out) {
                    uint32_t cm = 0u;                  // magnitudes: bits order like values
#pragma unroll
                    for (int sg = 0; sg < OC_SEG_MAX; ++sg)
                        if (sg < nseg) cm = max(cm, cmax_p[(int64_t)sg * K + col]);
                    colmax_out[col] = __builtin_bit_cast(float, cm);
                }
            }
        }
        const int cnt = __popcll(fl);
        int x = cnt;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(x, d, QA_WAVE);
            if (lane >= d) x += y;
        }
        if (lane == 63) wsum[wave] = x;
        __syncthreads();
        int off = running + x - cnt;
        for (int w = 0; w < wave; ++w) off += wsum[w];
        while (fl) {
            const int i = __builtin_ctzll(fl);
            fl &= fl - 1ull;
            idx[off++] = (int32_t)(cb + i);
        }
        running += wsum[0] + wsum[1] + wsum[2] + wsum[3];
        __syncthreads();
    }
    if (t == 0) *count = running;
}

__global__ __launch_bounds__(256) void k_outlier_finalize(const unsigned long long* __restrict__ flags_p,
                                                          const uint32_t* __restrict__ cmax_p, int nseg, int64_t K,
                                                          uint8_t* __restrict__ mask, int32_t* __restrict__ idx,
                                                          int32_t* __restrict__ count, float* __restrict__ colmax_out) {
    __shared__ int wsum[4];
    const int64_t nw = (K + 63) / 64;
    const rsrc_t rf = make_rsrc(flags_p, (int64_t)nseg * nw * 8);
    auto word = [&](int64_t w) -> unsigned long long {
        unsigned long long f = 0ull;
#pragma unroll
        for (int sg = 0; sg < OC_SEG_MAX; ++sg) {             // all loads in flight at once
            const u32x2 a = bload8(rf, w < nw && sg < nseg ? (uint32_t)(sg * nw + w) * 8 : kOOB);
            f |= a[0] | ((unsigned long long)a[1] << 32);
        }
        return f;
    };
    outlier_compact(word, cmax_p, nseg, K, mask, idx, count, colmax_out, wsum);
}

// Row segments of the scan: about 512 workgroups (strips x segments), at most
// OC_SEG_MAX segments and one per 256 rows.
static int outlier_segments(int64_t M, int64_t K) {
    const int64_t strips = (K + 63) / 64;
    int64_t segs = (512 + strips - 1) / strips;
    const int64_t by_rows = M > 0 ? (M + 255) / 256 : 1;
    if (segs > by_rows) segs = by_rows;
    if (segs > OC_SEG_MAX) segs = OC_SEG_MAX;
    return segs < 1 ? 1 : (int)segs;
}

// partial flags [OC_SEG_MAX x ceil(K/64)] u64, then partial column max [OC_SEG_MAX x K] u32
size_t outlier_scratch_bytes(int64_t K) {
    return (size_t)OC_SEG_MAX * ((size_t)((K + 63) / 64) * 8 + (size_t)K * 4) + 64;
}

static int outlier_scan(const uint16_t* X, int64_t M, int64_t K, float tau, void* scratch, bool want_max,
                        hipStream_t st) {
    unsigned long long* flags_p = static_cast<unsigned long long*>(scratch);
    const int64_t nw = (K + 63) / 64;
    uint32_t* cmax_p = reinterpret_cast<uint32_t*>(flags_p + OC_SEG_MAX * nw);
    const int segs = outlier_segments(M, K);
    dim3 grid((unsigned)nw, (unsigned)segs);
    if (want_max)
        hipLaunchKernelGGL(k_outlier_scan<true>, grid, dim3(256), 0, st, X, M, K, tau, flags_p, cmax_p);
    else
        hipLaunchKernelGGL(k_outlier_scan<false>, grid, dim3(256), 0, st, X, M, K, tau, flags_p, cmax_p);
    return segs;
}

hipError_t launch_outlier_cols(const uint16_t* X, int64_t M, int64_t K, float tau, uint8_t* mask,
                               int32_t* idx, int32_t* count, float* colmax, void* scratch, hipStream_t st) {
    const int segs = outlier_scan(X, M, K, tau, scratch, colmax != nullptr, st);
    unsigned long long* flags_p = static_cast<unsigned long long*>(scratch);
    const uint32_t* cmax_p = reinterpret_cast<const uint32_t*>(flags_p + OC_SEG_MAX * ((K + 63) / 64));
    hipLaunchKernelGGL(k_outlier_finalize, dim3(1), dim3(256), 0, st, flags_p, cmax_p, segs, K, mask, idx, count,
                       colmax);
    return hipGetLastError();
}

hipError_t launch_outlier_flags(const uint16_t* X, int64_t M, int64_t K, float tau, void* scratch, int* segs,
                                hipStream_t st) {
    *segs = outlier_scan(X, M, K, tau, scratch, false, st);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Top-k decomposition: the outlier set is the k columns with the largest
// column maximum, equal maxima taken in ascending column order.  One block
// of 1024 threads, after the scan above with no threshold.  The maxima are
// fp16 magnitudes, so a 15-bit key (the sign-cleared fp16 pattern, which
// orders like the value) identifies each; the block merges the segments'
// partial maxima into LDS keys (K <= TOPK_MAXK), finds the k-th largest key
// by a two-pass radix select (bits 14..8, then 7..0) with one histogram per
// wave (same-bin LDS atomics then only collide inside a wave), ranks the
// ties in column order with a block scan, and writes the selection as
// segment 0's flag words (the scan left the other segments' words zero), so
// the flag consumers see exactly the top-k set.  Thread t owns the TC
// consecutive columns [t TC, t TC + TC), TC = K / 1024 rounded up to a power
// of two, so a flag word is assembled from 64 / TC threads.
// FROMX (M <= 16 rows, M K <= 2^17): no scan before it; the block takes the column maxima
// from X itself (sign-cleared fp16 patterns, max over the rows) and leaves
// them as segment 0's partial maxima, as the scan would have.
// ---------------------------------------------------------------------------
constexpr int TOPK_MAXK = 32768;
constexpr int TOPK_THREADS = 1024;
constexpr int TOPK_WAVES = TOPK_THREADS / 64;
constexpr int TOPK_FROMX_ROWS = 16;
constexpr int64_t TOPK_FROMX_ELEMS = 16 * 8192;       // one CU reads at most 256 KB of X

template <bool FROMX>
__global__ __launch_bounds__(TOPK_THREADS) void k_topk_select(unsigned long long* __restrict__ flags_p,
                                                              uint32_t* __restrict__ cmax_p, int nseg,
                                                              int64_t K, int64_t k, const uint16_t* __restrict__ X,
                                                              int M) {
    __shared__ uint16_t keys[TOPK_MAXK];
    __shared__ uint32_t hist[TOPK_WAVES][256];
    __shared__ unsigned long long wout[TOPK_MAXK / 64];
    __shared__ uint32_t wsum[TOPK_WAVES];
    __shared__ uint32_t sel[2];                         // digit found, count above it
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int64_t nw = (K + 63) / 64;
    if constexpr (FROMX) {
        // four columns per thread and pass, all rows' loads in flight at once
        const rsrc_t rx = make_rsrc(X, (int64_t)M * K * 2);
        for (int64_t j0 = 0; j0 < K; j0 += 4 * TOPK_THREADS) {
            uint32_t v[4][TOPK_FROMX_ROWS];
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int i = 0; i < TOPK_FROMX_ROWS; ++i) {
                    const int64_t j = j0 + u * TOPK_THREADS + t;
                    v[u][i] = bload2(rx, i < M && j < K ? (uint32_t)(i * K + j) * 2 : kOOB);
                }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                uint32_t m = 0u;
#pragma unroll
                for (int i = 0; i < TOPK_FROMX_ROWS; ++i) m = max(m, v[u][i] & 0x7fffu);
                const int64_t j = j0 + u * TOPK_THREADS + t;
                if (j < K) {
                    const float cm = h2f((uint16_t)m);
                    keys[j] = f2h(cm);                  // the same key the scan + merge give
                    cmax_p[j] = __builtin_bit_cast(uint32_t, cm);
                }
            }
        }
    }
    // merge the segments: four columns per thread and pass, all 4 x OC_SEG_MAX
    // loads in flight before the first is used (out-of-range ones read 0)
    const rsrc_t rc = make_rsrc(cmax_p, (int64_t)nseg * K * 4);
    for (int64_t j0 = 0; !FROMX && j0 < K; j0 += 4 * TOPK_THREADS) {
        uint32_t v[4][OC_SEG_MAX];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int sg = 0; sg < OC_SEG_MAX; ++sg) {
                const int64_t j = j0 + u * TOPK_THREADS + t;
                v[u][sg] = bload4(rc, sg < nseg && j < K ? (uint32_t)(sg * K + j) * 4 : kOOB);
            }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            uint32_t m = 0u;
#pragma unroll
            for (int sg = 0; sg < OC_SEG_MAX; ++sg) m = max(m, v[u][sg]);
            const int64_t j = j0 + u * TOPK_THREADS + t;
            if (j < K) keys[j] = f2h(__builtin_bit_cast(float, m));   // exact: m is an fp16 magnitude
        }
    }
    for (int64_t w = t; w < nw; w += TOPK_THREADS) wout[w] = 0ull;
    int tc = 1;                                          // columns per thread, a power of two
    while ((int64_t)tc * TOPK_THREADS < K) tc <<= 1;
    const int64_t c0 = (int64_t)t * tc;
    // k-th largest key: digits fixed so far in `prefix` (under `pmask`)
    uint32_t prefix = 0u, pmask = 0u, remaining = (uint32_t)k;
    for (int pass = 0; pass < 2 && k > 0; ++pass) {
        const int shift = pass == 0 ? 8 : 0;
        for (int i = lane; i < 256; i += 64) hist[wave][i] = 0u;
        __syncthreads();
        for (int c = 0; c < tc; ++c) {
            const int64_t j = c0 + c;
            if (j < K) {
                const uint32_t key = keys[j];
                if ((key & pmask) == prefix) atomicAdd(&hist[wave][(key >> shift) & 255u], 1u);
            }
        }
        __syncthreads();
        if (wave == 0) {
            // lane l holds digits 255 - 4l .. 252 - 4l, summed over the waves;
            // inclusive sums from the top digit down
            uint32_t h[4], cs = 0u;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t a = 0u;
#pragma unroll
                for (int w = 0; w < TOPK_WAVES; ++w) a += hist[w][255 - 4 * lane - i];
                h[i] = a;
                cs += a;
            }
            uint32_t incl = cs;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t y = (uint32_t)__shfl_up((int)incl, o, QA_WAVE);
                if (lane >= o) incl += y;
            }
            uint32_t above = incl - cs;                 // count in digits above this lane's four
            if (above < remaining && remaining <= incl) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (above + h[i] >= remaining) {
                        sel[0] = 255u - 4u * lane - i;
                        sel[1] = above;
                        break;
                    }
                    above += h[i];
                }
            }
        }
        __syncthreads();
        prefix |= sel[0] << shift;
        pmask |= 255u << shift;
        remaining -= sel[1];
        __syncthreads();
    }
    // remaining = how many columns equal to the k-th key are taken (lowest first)
    const uint32_t kth = prefix;
    uint32_t ties = 0u;
    for (int c = 0; c < tc; ++c) {
        const int64_t j = c0 + c;
        ties += (k > 0 && j < K && keys[j] == kth) ? 1u : 0u;
    }
    uint32_t x = ties;                                   // exclusive scan in column order
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = (uint32_t)__shfl_up((int)x, o, QA_WAVE);
        if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    uint32_t before = x - ties;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    unsigned long long bits = 0ull;                      // this thread's columns, bit c = column c0 + c
    for (int c = 0; c < tc; ++c) {
        const int64_t j = c0 + c;
        if (k <= 0 || j >= K) continue;
        const uint32_t key = keys[j];
        bool take = key > kth;
        if (key == kth) {
            take = before < remaining;
            ++before;
        }
        if (take) bits |= 1ull << c;
    }
    if (bits) atomicOr(&wout[c0 >> 6], bits << (c0 & 63));
    __syncthreads();
    for (int64_t w = t; w < nw; w += TOPK_THREADS) flags_p[w] = wout[w];
}

hipError_t launch_outlier_topk_flags(const uint16_t* X, int64_t M, int64_t K, int64_t k, void* scratch, int* segs,
                                     hipStream_t st) {
    unsigned long long* flags_p = static_cast<unsigned long long*>(scratch);
    uint32_t* cmax_p = reinterpret_cast<uint32_t*>(flags_p + OC_SEG_MAX * ((K + 63) / 64));
    if (M <= TOPK_FROMX_ROWS && M * K <= TOPK_FROMX_ELEMS) {   // one launch: column maxima from X in the block
        *segs = 1;
        hipLaunchKernelGGL(k_topk_select<true>, dim3(1), dim3(TOPK_THREADS), 0, st, flags_p, cmax_p, 1, K, k, X,
                           (int)M);
    } else {
        *segs = outlier_scan(X, M, K, __builtin_inff(), scratch, true, st);
        hipLaunchKernelGGL(k_topk_select<false>, dim3(1), dim3(TOPK_THREADS), 0, st, flags_p, cmax_p, *segs, K, k,
                           X, (int)M);
    }
    return hipGetLastError();
}

hipError_t launch_outlier_topk(const uint16_t* X, int64_t M, int64_t K, int64_t k, uint8_t* mask, int32_t* idx,
                               int32_t* count, float* colmax, void* scratch, hipStream_t st) {
    int segs = 1;
    hipError_t e = launch_outlier_topk_flags(X, M, K, k, scratch, &segs, st);
    if (e != hipSuccess) return e;
    unsigned long long* flags_p = static_cast<unsigned long long*>(scratch);
    const uint32_t* cmax_p = reinterpret_cast<const uint32_t*>(flags_p + OC_SEG_MAX * ((K + 63) / 64));
    hipLaunchKernelGGL(k_outlier_finalize, dim3(1), dim3(256), 0, st, flags_p, cmax_p, segs, K, mask, idx, count,
                       colmax);
    return hipGetLastError();
}

int64_t topk_max_columns() { return TOPK_MAXK; }

// Column absolute maxima (the activation and weight statistics of the
// SmoothQuant migration): the scan above with no threshold, then one thread
// per column maxes the segments' partial maxima (and the caller's running
// maximum when accumulating; non-negative floats order like their bits).
__global__ __launch_bounds__(256) void k_colmax_merge(const uint32_t* __restrict__ cmax_p, int nseg, int64_t K,
                                                      float* __restrict__ colmax, int accumulate) {
    const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (j >= K) return;
    uint32_t m = accumulate ? __builtin_bit_cast(uint32_t, colmax[j]) : 0u;
#pragma unroll
    for (int sg = 0; sg < OC_SEG_MAX; ++sg)
        if (sg < nseg) m = max(m, cmax_p[(int64_t)sg * K + j]);
    colmax[j] = __builtin_bit_cast(float, m);
}

hipError_t launch_col_absmax(const uint16_t* A, int64_t rows, int64_t K, float* colmax, bool accumulate,
                             void* scratch, hipStream_t st) {
    const int segs = outlier_scan(A, rows, K, __builtin_inff(), scratch, true, st);
    const uint32_t* cmax_p =
        reinterpret_cast<const uint32_t*>(static_cast<unsigned long long*>(scratch) + OC_SEG_MAX * ((K + 63) / 64));
    hipLaunchKernelGGL(k_colmax_merge, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, st, cmax_p, segs, K, colmax,
                       accumulate ? 1 : 0);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Row-wise int8 quantization, 8 elements (16 bytes) per lane and chunk.
// NC > 0 keeps the row in registers (K <= 512 * NC), split over the WPR waves
// of the row (part p owns chunks p 64 NC / WPR + l + 64 i in lane l), which
// combine the row maximum through LDS; NC == 0 is one wave per row and reads
// the row twice (absmax pass, then quantize pass).
//
// Masks: MASK_BYTES -- caller's byte per column (nonzero = masked), applied per
// value; MASK_FLAGS -- outlier flag bits: every workgroup ORs the outlier
// scan's nseg partial flag sets into one bit per column in LDS, and a byte of
// it (one 8-column chunk) selects 16-bit keep words from a 256-entry table in
// LDS, ANDed into the fp16 bits.  In MASK_FLAGS mode block 0 also writes the
// ascending outlier list and its count; in MASK_NONE mode a non-null `count`
// is set to 0 (no outliers).
// ---------------------------------------------------------------------------
enum { MASK_NONE = 0, MASK_BYTES = 1, MASK_FLAGS = 2 };

// masked elements -> 0 (before the absmax and the quantizer)
__device__ __forceinline__ void apply_mask(float* x, u32x2 mk) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
        if ((mk[j >> 2] >> (8 * (j & 3))) & 0xffu) x[j] = 0.0f;
}

__device__ __forceinline__ float absmax8(const float* x) {
    float a = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) a = fmaxf(a, __builtin_fabsf(x[j]));
    return a;
}

// static (affine) codes: clip(rint(x / s) + z, qmin, qmax); masked -> clip(z)
__device__ __forceinline__ u32x2 codes8_static(const float* x, u32x2 mk, float s, int z, int qmin, int qmax) {
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        int code;
        if ((mk[j >> 2] >> (8 * (j & 3))) & 0xffu) {
            code = clampi(z, qmin, qmax);
        } else {
            double t = (double)__builtin_rintf(x[j] / s) + (double)z;
            t = t < (double)qmin ? (double)qmin : (t > (double)qmax ? (double)qmax : t);
            code = (int)t;
        }
        w[j >> 2] |= ((uint32_t)code & 0xffu) << (8 * (j & 3));
    }
    return u32x2{w[0], w[1]};
}

constexpr int RQ_FLAG_WORDS = 2048;             // merged flag words in LDS: K <= 131072

template <int NC, bool STATIC, int MASK, int WPR>
__global__ __launch_bounds__(256) void k_rowquant_i8(const uint16_t* __restrict__ X, int64_t rows, int64_t K,
                                                     const uint8_t* __restrict__ mask, int nseg, int qmin, int qmax,
                                                     const float* __restrict__ s_in, const int32_t* __restrict__ z_in,
                                                     int8_t* __restrict__ q, float* __restrict__ s_out,
                                                     int32_t* __restrict__ idx, int32_t* __restrict__ count,
                                                     uint16_t* __restrict__ xo) {
    __shared__ u32x4 lut[MASK == MASK_FLAGS ? 256 : 1];
    // (a row held in registers has K <= 8192: at most 128 flag words)
    __shared__ unsigned long long flw[MASK == MASK_FLAGS ? (NC > 0 ? 128 : RQ_FLAG_WORDS) : 1];
    __shared__ uint32_t wpre[MASK == MASK_FLAGS && NC > 0 ? 128 : 1];
    __shared__ uint32_t wtot[4];
    __shared__ int wsum[4];
    __shared__ uint32_t pmx[WPR > 1 ? 4 : 1];
    static_assert(WPR == 1 || ((WPR == 2 || WPR == 4) && NC >= WPR), "waves per row need a row held in registers");
    constexpr int NCW = NC / WPR;                     // chunks per lane of this wave
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int64_t row = (int64_t)blockIdx.x * (4 / WPR) + wave / WPR;
    const int part = wave % WPR;                      // which part of the row
    const bool live = row < rows;
    // chunk i of this lane: the wave's part of the row, lane-interleaved
    auto cho = [&](int i) -> int64_t { return (int64_t)part * 64 * NCW + lane + 64 * i; };
    const int64_t nch = K >> 3;
    const rsrc_t rx = make_rsrc(X + (live ? row : 0) * K, live ? K * 2 : 0);
    // With the row held in registers (K <= 8192: at most 128 flag words, one
    // per thread) the flag words are requested first and the row right after
    // them; loads retire in order, so the flag merge waits only for the flag
    // words, and the block barrier behind it waits only for LDS traffic.  Each
    // wave then waits for its own row alone, not for the slowest of the block.
    constexpr bool EARLY = MASK == MASK_FLAGS && NC > 0;
    u32x2 fpre[EARLY ? OC_SEG_MAX : 1];
    if constexpr (EARLY) {
        const int64_t nw = (K + 63) / 64;
        const rsrc_t rf = make_rsrc(mask, (int64_t)nseg * nw * 8);
        const bool mine = (int64_t)threadIdx.x < nw;
#pragma unroll
        for (int sg = 0; sg < OC_SEG_MAX; ++sg)
            fpre[sg] = bload8(rf, mine && sg < nseg ? (uint32_t)(sg * nw + threadIdx.x) * 8 : kOOB);
        __builtin_amdgcn_sched_barrier(0);
    }
    u32x4 vpre[NC > 0 ? NCW : 1];
    if constexpr (NC > 0) {
#pragma unroll
        for (int i = 0; i < NCW; ++i) vpre[i] = bload16(rx, (uint32_t)cho(i) * 16);
    }
    if constexpr (MASK == MASK_FLAGS) {
        const uint32_t b = threadIdx.x;              // keep words of an 8-bit outlier pattern
        u32x4 k;
#pragma unroll
        for (int d = 0; d < 4; ++d)
            k[d] = (((b >> (2 * d)) & 1u) ? 0u : 0xffffu) | (((b >> (2 * d + 1)) & 1u) ? 0u : 0xffff0000u);
        lut[b] = k;
        const int64_t nw = (K + 63) / 64;
        const rsrc_t rf = make_rsrc(mask, (int64_t)nseg * nw * 8);
        // thread t merges the flag words [t per, (t + 1) per)
        const int64_t per = (nw + 255) / 256, w0 = (int64_t)threadIdx.x * per, w1 = w0 + per < nw ? w0 + per : nw;
        uint32_t own = 0u;
        if constexpr (EARLY) {
            // merged in every thread (threads past the last word read zeros),
            // so the loads above are not moved into a branch behind the row's
            unsigned long long f = 0ull;
#pragma unroll
            for (int sg = 0; sg < OC_SEG_MAX; ++sg) f |= fpre[sg][0] | ((unsigned long long)fpre[sg][1] << 32);
            own = (uint32_t)__popcll(f);
            if (w0 < w1) flw[w0] = f;
        } else {
            for (int64_t w = w0; w < w1; ++w) {
                unsigned long long f = 0ull;
#pragma unroll
                for (int sg = 0; sg < OC_SEG_MAX; ++sg) {         // all loads in flight at once
                    const u32x2 a = bload8(rf, sg < nseg ? (uint32_t)(sg * nw + w) * 8 : kOOB);
                    f |= a[0] | ((unsigned long long)a[1] << 32);
                }
                flw[w] = f;
                own += (uint32_t)__popcll(f);
            }
        }
        if constexpr (NC > 0) {
            if (xo) {
                // rank of each flag word's first column in the outlier list,
                // within its owner wave (the waves' totals are added when read)
                uint32_t x = own;
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) {
                    const uint32_t y = (uint32_t)__shfl_up((int)x, o, QA_WAVE);
                    if (lane >= o) x += y;
                }
                if (lane == 63) wtot[wave_id()] = x;
                uint32_t run = x - own;
                for (int64_t w = w0; w < w1; ++w) {
                    wpre[w] = run;
                    run += (uint32_t)__popcll(flw[w]);
                }
            }
        }
        if constexpr (EARLY) {
            lds_only_barrier();                      // the row loads stay in flight
        } else {
            __syncthreads();
        }
        if (blockIdx.x == 0)
            outlier_compact([&](int64_t w) -> unsigned long long { return w < nw ? flw[w] : 0ull; }, nullptr, 0, K,
                            nullptr, idx, count, nullptr, wsum);
    }
    if constexpr (MASK == MASK_NONE)
        if (count && blockIdx.x == 0 && threadIdx.x == 0) *count = 0;
    // (with two waves per row and a dynamic scale, every wave reaches the
    // exchange of the row maximum below first)
    constexpr bool XCHG = WPR > 1 && !STATIC;
    if constexpr (!XCHG)
        if (!live) return;
    const rsrc_t rm = make_rsrc(mask, MASK == MASK_BYTES ? K : 0);
    const uint8_t* flb = reinterpret_cast<const uint8_t*>(flw);
    int8_t* qr = q + row * K;
    float s = 1.0f, r = 1.0f;
    int z = 0;
    if constexpr (STATIC) {
        s = s_in[row];
        z = z_in ? z_in[row] : 0;
    }
    // chunk ch: fp16 bits with MASK_FLAGS already applied, byte mask for MASK_BYTES
    uint32_t fbl = 0u;                                  // flag byte of the last chunk masked
    auto mask_of = [&](int64_t ch, u32x4& v, u32x2& mk) {
        mk = u32x2{0u, 0u};
        if constexpr (MASK == MASK_FLAGS) {
            fbl = ch < nch ? flb[ch] : 0u;
            v &= lut[fbl];
        }
        if constexpr (MASK == MASK_BYTES) mk = bload8(rm, (uint32_t)ch * 8);
    };
    auto load = [&](int64_t ch, u32x4& v, u32x2& mk) {
        v = bload16(rx, (uint32_t)ch * 16);
        mask_of(ch, v, mk);
    };
    if constexpr (NC > 0) {
        u32x4 v[NCW];
        u32x2 mk[NCW];
        uint32_t fbv[NCW];
#pragma unroll
        for (int i = 0; i < NCW; ++i) {
            v[i] = vpre[i];
            mask_of(cho(i), v[i], mk[i]);
            fbv[i] = fbl;
        }
        if constexpr (!STATIC) {
            // the row maximum as a non-negative float's bit pattern (these
            // order like the values), combined over the row's waves
            uint32_t ab;
            if constexpr (MASK == MASK_BYTES) {
                float a = 0.0f;
#pragma unroll
                for (int i = 0; i < NCW; ++i) {
                    float x[8];
                    unpack8(v[i], x);
                    apply_mask(x, mk[i]);
                    a = fmaxf(a, absmax8(x));
                }
                ab = __builtin_bit_cast(uint32_t, wave_max(a));
            } else {
                // on the sign-cleared fp16 patterns (they order like the
                // magnitudes), two per instruction; DPP lane reduction
                uint32_t am = 0u;
#pragma unroll
                for (int i = 0; i < NCW; ++i)
#pragma unroll
                    for (int d = 0; d < 4; ++d) am = pk_max_u16(am, v[i][d] & 0x7fff7fffu);
                ab = __builtin_bit_cast(uint32_t, h2f((uint16_t)wave_max_u32(max(am & 0xffffu, am >> 16))));
            }
            if constexpr (XCHG) {
                if (lane == 0) pmx[wave] = ab & 0x7fffffffu;      // (a -0.0 maximum would order last)
                lds_only_barrier();
                ab = 0u;                                            // every wave of the row, this one included
#pragma unroll
                for (int q = 0; q < WPR; ++q) ab = max(ab, pmx[wave - part + q]);
                if (!live) return;
            }
            const float amax = __builtin_bit_cast(float, ab);
            s = amax == 0.0f ? 1.0f : amax / (float)qmax;
            r = 1.0f / s;
            if (lane == 0 && part == 0) s_out[row] = s;
        }
#pragma unroll
        for (int i = 0; i < NCW; ++i) {
            const int64_t ch = cho(i);
            if (ch < nch) {
                u32x2 c;
                if constexpr (STATIC) {
                    float x[8];
                    unpack8(v[i], x);
                    c = codes8_static(x, mk[i], s, z, qmin, qmax);
                } else if constexpr (MASK == MASK_BYTES) {
                    float x[8];
                    unpack8(v[i], x);
                    apply_mask(x, mk[i]);
                    c = clip_codes(codes8_dyn(x, s, r), qmin);
                } else {
                    c = clip_codes(codes8_dyn_h(v[i], s, r), qmin);
                }
                st_codes8(qr + ch * 8, c);
            }
        }
        if constexpr (MASK == MASK_FLAGS) {
            // this row's outlier values, in list order, into xo[row][0 .. XO_CAP)
            // (after the codes: its LDS reads wait behind their stores)
            const int64_t nw = (K + 63) / 64, per = (nw + 255) / 256;
            const uint32_t t0 = wtot[0], t1 = wtot[1], t2 = wtot[2];
            if (xo && t0 + t1 + t2 + wtot[3] > 0u) {
#pragma unroll
                for (int i = 0; i < NCW; ++i) {
                    const int64_t ch = cho(i);
                    const uint32_t fb = fbv[i];
                    if (fb) {
                        const int64_t w = ch >> 3;
                        const int ow = (int)((w / per) >> 6);          // wave that ranked word w
                        const uint32_t woff = (ow > 0 ? t0 : 0u) + (ow > 1 ? t1 : 0u) + (ow > 2 ? t2 : 0u);
                        const unsigned long long fw = flw[w];
                        const int sh = (int)(ch & 7) * 8;
                        uint32_t rank = wpre[w] + woff + (uint32_t)__popcll(sh ? fw & ((1ull << sh) - 1ull) : 0ull);
                        for (int b = 0; b < 8; ++b) {
                            if ((fb >> b) & 1u) {
                                if (rank < (uint32_t)XO_CAP)
                                    xo[row * XO_CAP + rank] = (uint16_t)(vpre[i][b >> 1] >> (16 * (b & 1)));
                                ++rank;
                            }
                        }
                    }
                }
            }
        }
    } else {
        if constexpr (!STATIC) {
            float amax = 0.0f;
            for (int64_t ch = lane; ch < nch; ch += 64) {
                u32x4 v;
                u32x2 mk;
                load(ch, v, mk);
                float x[8];
                unpack8(v, x);
                if constexpr (MASK == MASK_BYTES) apply_mask(x, mk);
                amax = fmaxf(amax, absmax8(x));
            }
            amax = wave_max(amax);
            s = amax == 0.0f ? 1.0f : amax / (float)qmax;
            r = 1.0f / s;
            if (lane == 0) s_out[row] = s;
        }
        for (int64_t ch = lane; ch < nch; ch += 64) {
            u32x4 v;
            u32x2 mk;
            load(ch, v, mk);
            float x[8];
            unpack8(v, x);
            u32x2 c;
            if constexpr (STATIC) {
                c = codes8_static(x, mk, s, z, qmin, qmax);
            } else {
                if constexpr (MASK == MASK_BYTES) apply_mask(x, mk);
                c = clip_codes(codes8_dyn(x, s, r), qmin);
            }
            st_codes8(qr + ch * 8, c);
        }
    }
}

template <bool STATIC, int MASK>
static void rowquant_dispatch(const uint16_t* X, int64_t rows, int64_t K, const uint8_t* mask, int nseg, int qmin,
                              int qmax, const float* s_in, const int32_t* z_in, int8_t* q, float* s_out, int32_t* idx,
                              int32_t* count, hipStream_t st, uint16_t* xo = nullptr) {
    // several waves per row when the row is held in registers in two or more
    // chunks per lane (more waves in flight, less dependent work per wave):
    // two for 2 to 8 chunks, four for 16 (four measured slightly slower at 8)
    const int64_t nch = K / 8;
    const int wpr = nch > 512 && nch <= 1024 ? 4 : nch > 64 && nch <= 512 ? 2 : 1;
    const dim3 grid((unsigned)((rows + 4 / wpr - 1) / (4 / wpr))), block(256);
#define QA_RQ_W(NC, W) hipLaunchKernelGGL((k_rowquant_i8<NC, STATIC, MASK, W>), grid, block, 0, st, X, rows, K, mask, \
                                          nseg, qmin, qmax, s_in, z_in, q, s_out, idx, count, xo)
#define QA_RQ(NC) QA_RQ_W(NC, (NC >= 16 ? 4 : NC >= 2 ? 2 : 1))
    if (nch <= 64) QA_RQ(1);
    else if (nch <= 128) QA_RQ(2);
    else if (nch <= 256) QA_RQ(4);
    else if (nch <= 512) QA_RQ(8);
    else if (nch <= 1024) QA_RQ(16);
    else QA_RQ(0);
#undef QA_RQ
#undef QA_RQ_W
}

hipError_t launch_rowquant_i8(const uint16_t* X, int64_t rows, int64_t K, const uint8_t* mask, int qmin, int qmax,
                              const float* s_in, const int32_t* z_in, int8_t* q, float* s_out, hipStream_t st) {
    if (s_in)
        rowquant_dispatch<true, MASK_BYTES>(X, rows, K, mask, 0, qmin, qmax, s_in, z_in, q, s_out, nullptr, nullptr,
                                            st);
    else if (mask)
        rowquant_dispatch<false, MASK_BYTES>(X, rows, K, mask, 0, qmin, qmax, s_in, z_in, q, s_out, nullptr, nullptr,
                                             st);
    else
        rowquant_dispatch<false, MASK_NONE>(X, rows, K, mask, 0, qmin, qmax, s_in, z_in, q, s_out, nullptr, nullptr,
                                            st);
    return hipGetLastError();
}

bool rowquant_writes_xo(int64_t K) { return K / 8 <= 1024; }      // rows held in registers (NC > 0)

hipError_t launch_rowquant_i8_flags(const uint16_t* X, int64_t rows, int64_t K, const void* scratch, int nseg,
                                    int8_t* q, float* s_out, int32_t* idx, int32_t* count, uint16_t* xo,
                                    hipStream_t st) {
    rowquant_dispatch<false, MASK_FLAGS>(X, rows, K, static_cast<const uint8_t*>(scratch), nseg, -127, 127, nullptr,
                                         nullptr, q, s_out, idx, count, st, rowquant_writes_xo(K) ? xo : nullptr);
    return hipGetLastError();
}

hipError_t launch_rowquant_i8_no_outliers(const uint16_t* X, int64_t rows, int64_t K, int8_t* q, float* s_out,
                                          int32_t* count, hipStream_t st) {
    rowquant_dispatch<false, MASK_NONE>(X, rows, K, nullptr, 0, -127, 127, nullptr, nullptr, q, s_out, nullptr, count,
                                        st);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Asymmetric (zero-point) row quantization: per row, the min-max grid over
// [lo, hi] = [min(min x, 0), max(max x, 0)]: s = fl32(fl32(hi - lo) / (qmax -
// qmin)) (1.0 when hi == lo), z = clip(qmin - rint(fl32(lo / s))), codes
// clip(rint(fl32(x / s)) + z), and the row sum of the codes (int32).  WPR
// waves per row as in k_rowquant_i8, combining their minima, maxima and code
// sums through LDS (chunks past the row read 0, which is in the range anyway).
// Codes: |x / s| <= (qmax - qmin)(1 + 2^-23) <= 255.0001, so t = fma(x, r, 256)
// with r = fl32(1/s) lies in (0, 512): |x r - x/s| <= 255.0001 * 2^-24, the
// rounding of t adds at most 2^-16 and fl(x/s) is within 2^-17 of x/s, so
// t - 256 is within 4e-5 < 2^-14 of fl(x/s); unless t is that close to
// n + 1/2, rint(t) - 256 = rint(fl(x/s)).  Chunks with such a t take the
// correctly rounded division.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void minmax8(const float* x, float& lo, float& hi) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        lo = fminf(lo, x[j]);
        hi = fmaxf(hi, x[j]);
    }
}

__device__ __forceinline__ u32x2 codes8_asym(const float* x, float s, float r, int z, int qmin, int qmax, int& sum) {
    float n[8];
    float dmax = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float t = __builtin_fmaf(x[j], r, 256.0f);
        n[j] = __builtin_rintf(t);
        dmax = fmaxf(dmax, __builtin_fabsf(t - n[j]));
    }
    if (dmax > 0.5f - 0x1p-14f) {
#pragma unroll
        for (int j = 0; j < 8; ++j) n[j] = __builtin_rintf(x[j] / s) + 256.0f;
    }
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int c = clampi((int)n[j] - 256 + z, qmin, qmax);
        sum += c;
        w[j >> 2] |= ((uint32_t)c & 0xffu) << (8 * (j & 3));
    }
    return u32x2{w[0], w[1]};
}

__device__ __forceinline__ int wave_sum_i32(int v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, QA_WAVE);
    return v;
}

template <int NC, int WPR>
__global__ __launch_bounds__(256) void k_rowquant_i8_asym(const uint16_t* __restrict__ X, int64_t rows, int64_t K,
                                                          int qmin, int qmax, int8_t* __restrict__ q,
                                                          float* __restrict__ s_out, int32_t* __restrict__ z_out,
                                                          int32_t* __restrict__ rowsum) {
    static_assert(WPR == 1 || ((WPR == 2 || WPR == 4) && NC >= WPR), "waves per row need a row held in registers");
    constexpr int NCW = NC / WPR;
    __shared__ uint32_t xr[WPR > 1 ? 3 : 1][4];
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int64_t row = (int64_t)blockIdx.x * (4 / WPR) + wave / WPR;
    const int part = wave % WPR;
    const bool live = row < rows;
    if (WPR == 1 && !live) return;                    // (several waves per row all reach the exchanges)
    const int64_t nch = K >> 3;
    const rsrc_t rx = make_rsrc(X + (live ? row : 0) * K, live ? K * 2 : 0);
    int8_t* qr = q + row * K;
    float lo = 0.0f, hi = 0.0f;
    u32x4 v[NC > 0 ? NCW : 1];
    auto cho = [&](int i) -> int64_t { return (int64_t)part * 64 * NCW + lane + 64 * i; };
    if constexpr (NC > 0) {
#pragma unroll
        for (int i = 0; i < NCW; ++i) v[i] = bload16(rx, (uint32_t)cho(i) * 16);
#pragma unroll
        for (int i = 0; i < NCW; ++i) {
            float x[8];
            unpack8(v[i], x);
            minmax8(x, lo, hi);
        }
    } else {
        for (int64_t ch = lane; ch < nch; ch += 64) {
            float x[8];
            unpack8(bload16(rx, (uint32_t)ch * 16), x);
            minmax8(x, lo, hi);
        }
    }
    hi = wave_max(hi);
    lo = -wave_max(-lo);
    if constexpr (WPR > 1) {
        // hi >= 0 and -lo >= 0: with the sign bit cleared (a part of the row
        // that is all zeros gives -lo = -0.0, whose pattern is 0x80000000)
        // their bit patterns order like the values
        if (lane == 0) {
            xr[0][wave] = __builtin_bit_cast(uint32_t, hi) & 0x7fffffffu;
            xr[1][wave] = __builtin_bit_cast(uint32_t, -lo) & 0x7fffffffu;
        }
        lds_only_barrier();
        uint32_t h = 0u, l = 0u;
#pragma unroll
        for (int w = 0; w < WPR; ++w) {
            h = max(h, xr[0][wave - part + w]);
            l = max(l, xr[1][wave - part + w]);
        }
        hi = __builtin_bit_cast(float, h);
        lo = -__builtin_bit_cast(float, l);
    }
    const float s = hi != lo ? (hi - lo) / (float)(qmax - qmin) : 1.0f;
    const int z = clampi(qmin - (int)__builtin_rintf(lo / s), qmin, qmax);
    const float r = 1.0f / s;
    int sum = 0;
    if constexpr (NC > 0) {
#pragma unroll
        for (int i = 0; i < NCW; ++i) {
            const int64_t ch = cho(i);
            if (live && ch < nch) {
                float x[8];
                unpack8(v[i], x);
                st_codes8(qr + ch * 8, codes8_asym(x, s, r, z, qmin, qmax, sum));
            }
        }
    } else {
        for (int64_t ch = lane; ch < nch; ch += 64) {
            float x[8];
            unpack8(bload16(rx, (uint32_t)ch * 16), x);
            st_codes8(qr + ch * 8, codes8_asym(x, s, r, z, qmin, qmax, sum));
        }
    }
    sum = wave_sum_i32(sum);
    if constexpr (WPR > 1) {
        if (lane == 0) xr[2][wave] = (uint32_t)sum;
        lds_only_barrier();
        sum = 0;
#pragma unroll
        for (int w = 0; w < WPR; ++w) sum += (int)xr[2][wave - part + w];
        if (!live || part != 0) return;
    }
    if (lane == 0) {
        s_out[row] = s;
        z_out[row] = z;
        if (rowsum) rowsum[row] = sum;
    }
}

hipError_t launch_rowquant_i8_asym(const uint16_t* X, int64_t rows, int64_t K, int qmin, int qmax, int8_t* q,
                                   float* s_out, int32_t* z_out, int32_t* rowsum, hipStream_t st) {
    // waves per row as in the symmetric quantizer
    const int64_t nch = K / 8;
    const int wpr = nch > 512 && nch <= 1024 ? 4 : nch > 64 && nch <= 512 ? 2 : 1;
    const dim3 grid((unsigned)((rows + 4 / wpr - 1) / (4 / wpr))), block(256);
#define QA_RA(NC) hipLaunchKernelGGL((k_rowquant_i8_asym<NC, (NC >= 16 ? 4 : NC >= 2 ? 2 : 1)>), grid, block, 0, st, X, \
                                     rows, K, qmin, qmax, q, s_out, z_out, rowsum)
    if (nch <= 64) QA_RA(1);
    else if (nch <= 128) QA_RA(2);
    else if (nch <= 256) QA_RA(4);
    else if (nch <= 512) QA_RA(8);
    else if (nch <= 1024) QA_RA(16);
    else QA_RA(0);
#undef QA_RA
    return hipGetLastError();
}

// Row sums of int8 rows (K % 16 == 0): one wave per row, 16 bytes per lane.
__global__ __launch_bounds__(256) void k_row_sums_i8(const int8_t* __restrict__ A, int64_t rows, int64_t K,
                                                     int32_t* __restrict__ sums) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + wave_id();
    if (row >= rows) return;
    const rsrc_t ra = make_rsrc(A + row * K, K);
    int sum = 0;
    for (int64_t c0 = 0; c0 < K; c0 += 64 * 16 * 4) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = bload16(ra, (uint32_t)(c0 + (u * 64 + lane) * 16));
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int d = 0; d < 4; ++d)
#pragma unroll
                for (int b = 0; b < 4; ++b) sum += (int)(int8_t)(v[u][d] >> (8 * b));
    }
    sum = wave_sum_i32(sum);
    if (lane == 0) sums[row] = sum;
}

hipError_t launch_row_sums_i8(const int8_t* A, int64_t rows, int64_t K, int32_t* sums, hipStream_t st) {
    hipLaunchKernelGGL(k_row_sums_i8, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, A, rows, K, sums);
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

// Code formats of the per-row quantizers below: symmetric int4 (packed),
// symmetric int8, and zero-point int4 (q = clip(rint(x / s) + z, 0, 15),
// packed as the two's complement nibble q - 8).
enum { HQ_I4 = 0, HQ_I8 = 1, HQ_I4Z = 2 };

// Per-row parameters from the row's maximum magnitude `amax` (symmetric) or
// its range [lo, hi] with lo <= 0 <= hi (zero-point, the min-max rule over
// [0, 15]: s = fl32(fl32(hi - lo) / 15), 1.0 when hi == lo, and
// z = clip(-rint(fl32(lo / s)), 0, 15)).
struct RowParams {
    float s, r;
    int z;
};

template <int MODE>
__device__ __forceinline__ RowParams row_params(float amax, float lo, float hi, int qmax) {
    RowParams p;
    p.z = 0;
    if constexpr (MODE == HQ_I4Z) {
        p.s = hi != lo ? (hi - lo) / 15.0f : 1.0f;
        p.z = clampi(-(int)__builtin_rintf(lo / p.s), 0, 15);
    } else {
        p.s = amax == 0.0f ? 1.0f : amax / (float)qmax;
    }
    p.r = 1.0f / p.s;
    return p;
}

// The codes of chunk ch (8 values, |x / s| <= q_max (1 + 2^-23)), clipped
// below at qmin: HQ_I8, eight int8 codes at out + 8 ch; otherwise eight int4
// codes packed into the word out[ch], element j in bits [4j+3:4j].
template <int MODE>
__device__ __forceinline__ uint32_t code_word(const float* x, const RowParams& p, int qmin) {
    if constexpr (MODE == HQ_I4Z) {
        int unused = 0;
        const u32x2 q = codes8_asym(x, p.s, p.r, p.z, 0, 15, unused);
        return pack_nibbles(u32x2{q[0] ^ 0x08080808u, q[1] ^ 0x08080808u});
    } else {
        return pack_codes(x, p.s, p.r, qmin);
    }
}

template <int MODE>
__device__ __forceinline__ void store_codes(void* out, int64_t ch, const float* x, const RowParams& p, int qmin) {
    if constexpr (MODE == HQ_I8)
        reinterpret_cast<u32x2*>(out)[ch] = clip_codes(codes8_dyn(x, p.s, p.r), qmin);
    else
        reinterpret_cast<uint32_t*>(out)[ch] = code_word<MODE>(x, p, qmin);
}

// 4 x 4 transpose inside each quad of lanes: on return lane 4b + j holds in
// w[k] what lane 4b + k held in w[j] (two exchange steps, lane bit 0 with
// register bit 0, then lane bit 1 with register bit 1; DPP quad moves).
__device__ __forceinline__ void quad_transpose(uint32_t* w, int lane) {
    uint32_t a[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)w[r ^ 1], 0xB1, 0xF, 0xF, false);
        a[r] = ((lane ^ r) & 1) ? o : w[r];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a[r ^ 2], 0x4E, 0xF, 0xF, false);
        w[r] = ((lane ^ r) & 2) ? o : a[r];
    }
}

// The magnitudes a row's parameters need, as non-negative fp32 bit patterns
// (which order like the values): amax, or -lo and hi.
__device__ __forceinline__ void range8(const float* x, float& amax, float& nlo, float& hi) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        amax = fmaxf(amax, __builtin_fabsf(x[j]));
        nlo = fmaxf(nlo, -x[j]);
        hi = fmaxf(hi, x[j]);
    }
}

// Per-row scale, row held in registers (NC > 0) or recomputed (NC == 0).
template <int G, int NC, int MODE>
__global__ __launch_bounds__(256) void k_hq4_row(const uint16_t* __restrict__ X, int64_t rows, int64_t K,
                                                 int qmin, int qmax, double c, void* __restrict__ codes,
                                                 float* __restrict__ s_out, int32_t* __restrict__ z_out) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + wave_id();
    if (row >= rows) return;
    const int64_t nch = K >> 3;
    const rsrc_t rx = make_rsrc(X + row * K, K * 2);
    void* pr = reinterpret_cast<uint8_t*>(codes) + row * nch * (MODE == HQ_I8 ? 8 : 4);
    if constexpr (NC > 0) {
        u32x4 v[NC];
#pragma unroll
        for (int i = 0; i < NC; ++i) v[i] = bload16(rx, (uint32_t)(lane + 64 * i) * 16);
        float xs[NC][8];
        float amax = 0.0f, nlo = 0.0f, hi = 0.0f;
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            fwht_chunk<G>(v[i], c, lane, xs[i]);
            range8(xs[i], amax, nlo, hi);
        }
        const RowParams p = row_params<MODE>(wave_max(amax), -wave_max(nlo), wave_max(hi), qmax);
        if (lane == 0) {
            s_out[row] = p.s;
            if (MODE == HQ_I4Z) z_out[row] = p.z;
        }
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const int64_t ch = lane + 64 * i;
            if (ch < nch) store_codes<MODE>(pr, ch, xs[i], p, qmin);
        }
    } else {
        float amax = 0.0f, nlo = 0.0f, hi = 0.0f;
        for (int64_t base = 0; base < nch; base += 64) {
            const int64_t ch = base + lane;
            float xo[8];
            fwht_chunk<G>(bload16(rx, (uint32_t)ch * 16), c, lane, xo);
            range8(xo, amax, nlo, hi);
        }
        const RowParams p = row_params<MODE>(wave_max(amax), -wave_max(nlo), wave_max(hi), qmax);
        if (lane == 0) {
            s_out[row] = p.s;
            if (MODE == HQ_I4Z) z_out[row] = p.z;
        }
        for (int64_t base = 0; base < nch; base += 64) {
            const int64_t ch = base + lane;
            float xo[8];
            fwht_chunk<G>(bload16(rx, (uint32_t)ch * 16), c, lane, xo);
            if (ch < nch) store_codes<MODE>(pr, ch, xo, p, qmin);
        }
    }
}

// Per-row scale with the whole row in registers and the butterfly almost all
// in-lane: K = 512 NC WPR, WPR waves per row (each owns K / WPR contiguous
// elements, whole G-blocks), NC chunks of 8 elements per lane; the WPR waves
// of a row combine their absmax through LDS.
// With CPB = G/8 chunks per G-block, a lane holds
//   LPB == 1 (NC >= CPB): chunks lane*NC .. lane*NC + NC - 1 (whole blocks);
//   LPB  > 1 (NC <  CPB): chunks (lane/LPB)*CPB + lane%LPB + LPB*i of one block,
// so element bits 0-2 are in the chunk, the chunk slots carry the remaining
// in-block bits except the lowest log2(LPB) chunk bits, which sit in the lane
// index and take one DPP quad exchange per bit.  The stages commute and every
// partial sum is exact in fp64, so their order does not matter.
template <int G, int NC, int WPR, int MODE>
__global__ __launch_bounds__(256) void k_hq4_row_reg(const uint16_t* __restrict__ X, int64_t rows, int64_t K,
                                                     int qmin, int qmax, double c, void* __restrict__ codes,
                                                     float* __restrict__ s_out, int32_t* __restrict__ z_out) {
    constexpr int CPB = G / 8;
    constexpr int LPB = CPB > NC ? CPB / NC : 1;
    static_assert(CPB >= 1 && LPB <= 4 && (LPB > 1 ? CPB % NC == 0 : NC % CPB == 0), "unsupported G / NC");
    static_assert(WPR == 1 || WPR == 2 || WPR == 4, "waves per row");
    __shared__ uint32_t red[3][4];
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int64_t row = (int64_t)blockIdx.x * (4 / WPR) + wave / WPR;
    const int part = wave % WPR;                      // which K / WPR slice of the row
    const bool live = row < rows;                     // every wave reaches the barrier below
    const rsrc_t rx = make_rsrc(X + row * K, live ? K * 2 : 0);
    const int64_t ch0 = row * (K >> 3) + part * 64 * NC;
    auto chunk = [&](int i) -> int {
        return LPB == 1 ? lane * NC + i : (lane / LPB) * CPB + (lane % LPB) + LPB * i;
    };
    const uint32_t pbase = (uint32_t)part * 64 * NC * 16;
    u32x4 v[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i) v[i] = bload16(rx, pbase + (uint32_t)chunk(i) * 16);
    double y[NC][8];
#pragma unroll
    for (int i = 0; i < NC; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) y[i][j] = (double)h2f((uint16_t)(v[i][j >> 1] >> (16 * (j & 1))));
    // element bits (strides 1, 2, 4 inside a chunk)
#pragma unroll
    for (int h = 1; h < 8 && h < G; h <<= 1)
#pragma unroll
        for (int i = 0; i < NC; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if ((j & h) == 0) {
                    const double a = y[i][j], b = y[i][j + h];
                    y[i][j] = a + b;
                    y[i][j + h] = a - b;
                }
    // chunk-slot bits
    constexpr int SLOT_SPAN = LPB == 1 ? CPB : NC;
#pragma unroll
    for (int h = 1; h < SLOT_SPAN; h <<= 1)
#pragma unroll
        for (int i = 0; i < NC; ++i)
            if ((i & h) == 0)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const double a = y[i][j], b = y[i + h][j];
                    y[i][j] = a + b;
                    y[i + h][j] = a - b;
                }
    // lane bits: partner lane ^ d; the lower lane keeps a + b, the upper p - y = a - b
#pragma unroll
    for (int d = 1; d < LPB; d <<= 1) {
        const double sg = (lane & d) ? -1.0 : 1.0;
#pragma unroll
        for (int i = 0; i < NC; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const double p = d == 1 ? dpp_xor_f64<1>(y[i][j]) : dpp_xor_f64<2>(y[i][j]);
                y[i][j] = __builtin_fma(sg, y[i][j], p);
            }
    }
    float xs[NC][8];
    float amax = 0.0f, nlo = 0.0f, hi = 0.0f;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
#pragma unroll
        for (int j = 0; j < 8; ++j) xs[i][j] = (float)(y[i][j] * c);
        range8(xs[i], amax, nlo, hi);
    }
    // the maxima are >= 0, so their bit patterns order like their values
    constexpr int NR = MODE == HQ_I4Z ? 3 : 1;
    uint32_t ab[3] = {__builtin_bit_cast(uint32_t, amax), __builtin_bit_cast(uint32_t, nlo),
                      __builtin_bit_cast(uint32_t, hi)};
#pragma unroll
    for (int k = 0; k < NR; ++k) ab[k] = wave_max_u32(ab[k]);
    if constexpr (WPR > 1) {
        if (lane == 0)
#pragma unroll
            for (int k = 0; k < NR; ++k) red[k][wave] = ab[k];
        __syncthreads();
        const int w0 = wave - part;
#pragma unroll
        for (int q = 0; q < WPR; ++q)
#pragma unroll
            for (int k = 0; k < NR; ++k) ab[k] = max(ab[k], red[k][w0 + q]);
    }
    if (!live) return;
    const RowParams p = row_params<MODE>(__builtin_bit_cast(float, ab[0]), -__builtin_bit_cast(float, ab[1]),
                                         __builtin_bit_cast(float, ab[2]), qmax);
    if (lane == 0 && part == 0) {
        s_out[row] = p.s;
        if (MODE == HQ_I4Z) z_out[row] = p.z;
    }
    if constexpr (MODE == HQ_I8 && NC == 4) {
        // eight int8 codes per chunk: the wave's 256 chunks (2 KB) go through
        // LDS so that each of its two stores covers 1 KB of whole lines
        __shared__ u32x2 stg[4][64 * NC];
#pragma unroll
        for (int i = 0; i < NC; ++i) stg[wave][chunk(i)] = clip_codes(codes8_dyn(xs[i], p.s, p.r), qmin);
        __builtin_amdgcn_wave_barrier();
        const u32x4* sv = reinterpret_cast<const u32x4*>(stg[wave]);
        const u32x4 a = sv[lane], b = sv[64 + lane];                  // chunks 2l, 2l + 1 and 128 + 2l, 129 + 2l
        u32x2* pw = static_cast<u32x2*>(codes) + ch0;
        if ((reinterpret_cast<uintptr_t>(codes) & 15u) == 0) {
            __builtin_nontemporal_store(a, reinterpret_cast<u32x4*>(pw + 2 * lane));
            __builtin_nontemporal_store(b, reinterpret_cast<u32x4*>(pw + 128 + 2 * lane));
        } else {
            pw[2 * lane] = u32x2{a[0], a[1]};
            pw[2 * lane + 1] = u32x2{a[2], a[3]};
            pw[128 + 2 * lane] = u32x2{b[0], b[1]};
            pw[129 + 2 * lane] = u32x2{b[2], b[3]};
        }
    } else if constexpr (MODE != HQ_I8 && NC == 4 && (LPB == 4 || LPB == 1)) {
        // four packed words per lane, made contiguous (with LPB == 4 the quad
        // transpose gives lane 4b + j the chunks 16b + 4j .. 16b + 4j + 3), so
        // a wave stores 1 KB of whole lines, streamed out like the int8 codes
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = code_word<MODE>(xs[i], p, qmin);
        if constexpr (LPB == 4) quad_transpose(w, lane);
        uint32_t* pw = static_cast<uint32_t*>(codes) + ch0 + (LPB == 4 ? (lane >> 2) * 16 + (lane & 3) * 4 : lane * 4);
        if ((reinterpret_cast<uintptr_t>(codes) & 15u) == 0) {
            __builtin_nontemporal_store(u32x4{w[0], w[1], w[2], w[3]}, reinterpret_cast<u32x4*>(pw));
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) pw[k] = w[k];
        }
    } else {
#pragma unroll
        for (int i = 0; i < NC; ++i) store_codes<MODE>(codes, ch0 + chunk(i), xs[i], p, qmin);
    }
}

// Per-group scale (G >= 8): the G/8 lanes of a block reduce their absmax.
template <int G>
__global__ __launch_bounds__(256) void k_hq4_group(const uint16_t* __restrict__ X, int64_t rows, int64_t K,
                                                   int qmin, int qmax, double c, uint32_t* __restrict__ packed,
                                                   float* __restrict__ s_out) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + wave_id();
    if (row >= rows) return;
    const int64_t nch = K >> 3;
    const int64_t ngr = K / G;
    const rsrc_t rx = make_rsrc(X + row * K, K * 2);
    uint32_t* pr = packed + row * nch;
    for (int64_t base = 0; base < nch; base += 64) {
        const int64_t ch = base + lane;
        float xo[8];
        fwht_chunk<G>(bload16(rx, (uint32_t)ch * 16), c, lane, xo);
        float amax = group_max(absmax8f(xo), G / 8);
        const float s = amax == 0.0f ? 1.0f : amax / (float)qmax;
        const float r = 1.0f / s;
        if (ch < nch) {
            pr[ch] = pack_codes(xo, s, r, qmin);
            if ((lane & (G / 8 - 1)) == 0) s_out[row * ngr + (ch * 8) / G] = s;
        }
    }
}

// k_hq4_row_reg<G, NC> handles K == 512 NC when G / NC fits its lane mapping.
template <int G, int NC>
constexpr bool hq4_row_reg_ok() {
    return G >= 8 && (G / 8 > NC ? (G / 8) / NC <= 4 && (G / 8) % NC == 0 : NC % (G / 8) == 0);
}

template <int G, int NC, int WPR, int MODE>
static bool hq4_row_reg_try(const uint16_t* X, int64_t rows, int64_t K, int qmin, int qmax, double c,
                            void* codes, float* s, int32_t* z, hipStream_t st) {
    if constexpr (hq4_row_reg_ok<G, NC>()) {
        if (K != 512 * NC * WPR) return false;
        const dim3 grid((unsigned)((rows + 4 / WPR - 1) / (4 / WPR))), block(256);
        hipLaunchKernelGGL((k_hq4_row_reg<G, NC, WPR, MODE>), grid, block, 0, st, X, rows, K, qmin, qmax, c, codes,
                           s, z);
        return true;
    } else {
        return false;
    }
}

template <int G, int MODE = HQ_I4>
static void hq4_dispatch(const uint16_t* X, int64_t rows, int64_t K, bool per_group, int qmin, int qmax,
                         void* codes, float* s, hipStream_t st, int32_t* z = nullptr) {
    const double c = 1.0 / __builtin_sqrt((double)G);
    const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
    if (per_group) {
        if constexpr (G >= 8 && MODE == HQ_I4)
            hipLaunchKernelGGL((k_hq4_group<G>), grid, block, 0, st, X, rows, K, qmin, qmax, c,
                               static_cast<uint32_t*>(codes), s);
        return;
    }
    const int64_t nch = K / 8;
    // two waves per row where the lane mapping allows it (more waves to hide latency)
    if (hq4_row_reg_try<G, 2, 1, MODE>(X, rows, K, qmin, qmax, c, codes, s, z, st) ||
        hq4_row_reg_try<G, 2, 2, MODE>(X, rows, K, qmin, qmax, c, codes, s, z, st) ||
        hq4_row_reg_try<G, 4, 2, MODE>(X, rows, K, qmin, qmax, c, codes, s, z, st) ||
        hq4_row_reg_try<G, 8, 1, MODE>(X, rows, K, qmin, qmax, c, codes, s, z, st) ||
        hq4_row_reg_try<G, 4, 1, MODE>(X, rows, K, qmin, qmax, c, codes, s, z, st) ||
        hq4_row_reg_try<G, 8, 2, MODE>(X, rows, K, qmin, qmax, c, codes, s, z, st))
        return;
#define QA_HQ(NC) \
    hipLaunchKernelGGL((k_hq4_row<G, NC, MODE>), grid, block, 0, st, X, rows, K, qmin, qmax, c, codes, s, z)
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

// Column terms of the zero-point correction (an offline computation on the
// weight), one wave per output channel: lane l sums the signed nibbles of
// groups l, l + 64, ... (exact integers; a group's words are read by one
// lane, consecutive lanes reading consecutive groups), and lane 0 adds the
// products with the fp32 group scales, each exact in fp64, over g ascending.
__global__ __launch_bounds__(256) void k_w4_column_terms(const uint32_t* __restrict__ Wp, const float* __restrict__ s_w,
                                                         int64_t N, int64_t K, int G, float* __restrict__ c) {
    __shared__ int gsum[4][512];
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int64_t n = (int64_t)blockIdx.x * 4 + wave;
    const int64_t words = K / 8, ng = K / G, wpg = G / 8;
    if (n >= N) return;
    const uint32_t* w = Wp + n * words;
    double acc = 0.0;
    for (int64_t g0 = 0; g0 < ng; g0 += 512) {
        const int64_t gn = ng - g0 < 512 ? ng - g0 : 512;
        for (int64_t g = lane; g < gn; g += 64) {
            int sum = 0;
            for (int64_t i = (g0 + g) * wpg; i < (g0 + g + 1) * wpg; ++i) {
                const uint32_t v = w[i];
#pragma unroll
                for (int j = 0; j < 8; ++j) sum += (int)(v << (28 - 4 * j)) >> 28;    // nibble j, sign-extended
            }
            gsum[wave][g] = sum;
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);                 // this wave's LDS writes (lgkmcnt(0))
        __builtin_amdgcn_wave_barrier();
        if (lane == 0)
            for (int64_t g = 0; g < gn; ++g) acc += (double)s_w[n * ng + g0 + g] * (double)gsum[wave][g];
        __builtin_amdgcn_wave_barrier();
    }
    if (lane == 0) c[n] = (float)acc;
}

hipError_t launch_w4_column_terms(const uint32_t* Wp, const float* s_w, int64_t N, int64_t K, int G, float* c,
                                  hipStream_t st) {
    hipLaunchKernelGGL(k_w4_column_terms, dim3((unsigned)((N + 3) / 4)), dim3(256), 0, st, Wp, s_w, N, K, G, c);
    return hipGetLastError();
}

// The same rotation with zero-point int4 codes per row (q - 8 packed, z in [0, 15]).
hipError_t launch_hadamard_quant_i4_asym(const uint16_t* X, int64_t rows, int64_t K, int G, uint32_t* packed,
                                         float* s, int32_t* z, hipStream_t st) {
    switch (G) {
        case 1: hq4_dispatch<1, HQ_I4Z>(X, rows, K, false, 0, 15, packed, s, st, z); break;
        case 2: hq4_dispatch<2, HQ_I4Z>(X, rows, K, false, 0, 15, packed, s, st, z); break;
        case 4: hq4_dispatch<4, HQ_I4Z>(X, rows, K, false, 0, 15, packed, s, st, z); break;
        case 8: hq4_dispatch<8, HQ_I4Z>(X, rows, K, false, 0, 15, packed, s, st, z); break;
        case 16: hq4_dispatch<16, HQ_I4Z>(X, rows, K, false, 0, 15, packed, s, st, z); break;
        case 32: hq4_dispatch<32, HQ_I4Z>(X, rows, K, false, 0, 15, packed, s, st, z); break;
        case 64: hq4_dispatch<64, HQ_I4Z>(X, rows, K, false, 0, 15, packed, s, st, z); break;
        case 128: hq4_dispatch<128, HQ_I4Z>(X, rows, K, false, 0, 15, packed, s, st, z); break;
        case 256: hq4_dispatch<256, HQ_I4Z>(X, rows, K, false, 0, 15, packed, s, st, z); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// The same rotation with per-row int8 codes (W4A8 activations).
hipError_t launch_hadamard_quant_i8(const uint16_t* X, int64_t rows, int64_t K, int G, int qmin, int qmax,
                                    int8_t* q, float* s, hipStream_t st) {
    switch (G) {
        case 1: hq4_dispatch<1, HQ_I8>(X, rows, K, false, qmin, qmax, q, s, st); break;
        case 2: hq4_dispatch<2, HQ_I8>(X, rows, K, false, qmin, qmax, q, s, st); break;
        case 4: hq4_dispatch<4, HQ_I8>(X, rows, K, false, qmin, qmax, q, s, st); break;
        case 8: hq4_dispatch<8, HQ_I8>(X, rows, K, false, qmin, qmax, q, s, st); break;
        case 16: hq4_dispatch<16, HQ_I8>(X, rows, K, false, qmin, qmax, q, s, st); break;
        case 32: hq4_dispatch<32, HQ_I8>(X, rows, K, false, qmin, qmax, q, s, st); break;
        case 64: hq4_dispatch<64, HQ_I8>(X, rows, K, false, qmin, qmax, q, s, st); break;
        case 128: hq4_dispatch<128, HQ_I8>(X, rows, K, false, qmin, qmax, q, s, st); break;
        case 256: hq4_dispatch<256, HQ_I8>(X, rows, K, false, qmin, qmax, q, s, st); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace qa
