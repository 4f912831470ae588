/*
 * qa.h -- C ABI of libqa, quantized linear layers for AMD Instinct MI355X
 * (gfx950, CDNA4).
 *
 * Quantized linear layers of LLM inference:
 *   - LLM.int8() mixed precision: feature columns whose activation magnitude
 *     exceeds a threshold stay in fp16, all other columns are quantized to
 *     int8 with vector-wise absmax scales (per token for X, per output
 *     channel for W), multiplied with int32 accumulation, dequantized by the
 *     outer product of the scales and summed with the fp16 outlier product.
 *   - FlatQuant's Kronecker transform (P = P1 (x) P2) fused with int4
 *     quantization, feeding the same W4A4 GEMM.
 *   - W4A4 group Hadamard: each G-wide block of the K dimension is rotated by
 *     the normalized Hadamard matrix, quantized to int4 (dynamic per-token
 *     scales for X, per-row-per-group scales for W), packed eight per 32-bit
 *     word, multiplied with int32 accumulation per group and dequantized.
 *   - SmoothQuant W8A8: activation columns are divided by per-channel
 *     migration factors and the weight's input channels multiplied by them,
 *     so both quantize to int8 with plain absmax scales (per token or per
 *     tensor for X, per output channel for W) and no fp16 branch.
 *
 * Sources, cited by page title and section:
 *   [AIInfra-Q01]  Infrasys-AI "AIInfra" notes, page 05Quantization01 (模型量化):
 *                  the LLM.int8() method -- outlier detection, "a. 向量级量化",
 *                  "b. INT8 矩阵乘法与反量化", merge of the two parts.
 *                  Its advice for training: decompose the largest-magnitude
 *                  1-2% of feature dimensions instead of about 0.1% (top-k).
 *                  Its FlatQuant section: the apply stage reshapes each token
 *                  to X~ [n1 x n2] and computes X~ x1 P1^T x2 P2 with
 *                  P = P1 (x) P2, fused with dynamic int4 quantization; the
 *                  sizes minimize n1 + n2 (8192 -> 64 x 128).
 *   [Scholia-IQ]   "模型推理量化" (Inference Quantization notes): §4 Scale,
 *                  §5 Outlier, §6 Zero-point (§6.2 affine clip), §7 Granularity.
 *   [GroupRot]     "低比特量化加速：分组旋转方法从W8A8到W4A4的实践与展望":
 *                  §二 normalized Hadamard, §5.1 weight transform and storage,
 *                  §5.2 online activation transform fused with quantization,
 *                  §5.4 packing and int32 accumulation.
 *   [QE2]          "Quantization explained, part 2" (tanjunchen.github.io),
 *                  §1.2: threshold 6.0 on a channel's activation magnitude;
 *                  §4.2: SmoothQuant, the per-input-channel migration
 *                  X W = (X diag(s)^-1)(diag(s) W), s_j = max|X_j|^alpha /
 *                  max|W_j|^(1-alpha); §4.4: factors fixed offline.
 *
 * Conventions shared by every entry point:
 *   - All array arguments are DEVICE pointers allocated and owned by the
 *     caller; the library allocates nothing and keeps no per-call state.
 *   - Matrices are row-major.  X is [M x K] (tokens x in-features), W is
 *     [N x K] (out-features x in-features), the output is [M x N].
 *   - fp16 / bf16 arrays are passed as `const void*` holding IEEE binary16 /
 *     bfloat16 bit patterns.
 *   - `stream` is a hipStream_t (NULL: the default stream).  Every call is
 *     asynchronous and stream-ordered; nothing synchronizes the host.
 *   - Every argument check runs before any HIP call.  On error nothing is
 *     launched and outputs are untouched.  Device faults surface at the
 *     caller's next synchronization.
 *   - Sizes and scalar arguments are checked first.  M == 0 or N == 0 (an
 *     empty batch or layer; rows == 0 for the quantizers) is then a valid
 *     no-op, and the pointers of empty arrays may be NULL.
 *   - Inputs must be finite (NaN / Inf are not checked on the hot path).
 *   - Rounding: scales are fl32(absmax / q_max) with IEEE correctly rounded
 *     division (1.0 when absmax is 0, [Scholia-IQ §4]); codes are
 *     clip(rint(fl32(x / s)) + z, q_min, q_max) with ties to even.
 */
#ifndef QA_H
#define QA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QA_OK = 0,
    QA_ERR_NULL = 1,        /* a required pointer is NULL */
    QA_ERR_SHAPE = 2,       /* negative size, K not a multiple of the required step, bad G */
    QA_ERR_ALIGN = 3,       /* a pointer is not 16-byte aligned */
    QA_ERR_VALUE = 4,       /* q_min > q_max, range outside the code type, NaN threshold, ... */
    QA_ERR_WORKSPACE = 5,   /* workspace smaller than the matching *_workspace() size */
    QA_ERR_UNSUPPORTED = 6, /* a valid request that this library has no kernel for */
    QA_ERR_DEVICE = 7       /* a HIP launch failed; see qa_last_error() */
} qa_status;

typedef enum { QA_F32 = 0, QA_F16 = 1, QA_BF16 = 2 } qa_dtype;

typedef enum { QA_SCALE_PER_ROW = 0, QA_SCALE_PER_GROUP = 1, QA_SCALE_PER_TENSOR = 2 } qa_scale_mode;

/* SmoothQuant side: activations are divided by the factors, weights multiplied. */
typedef enum { QA_SMOOTH_DIVIDE = 0, QA_SMOOTH_MULTIPLY = 1 } qa_smooth_op;

/* Human-readable name of a status code (static string). */
const char* qa_status_string(qa_status s);

/* Detail of the last error raised on the calling thread ("" if none). */
const char* qa_last_error(void);

/* ---------------------------------------------------------------------------
 * Outlier feature columns  [AIInfra-Q01, LLM.int8() detection step; QE2 §1.2]
 *
 * colmax[j] = max_i |X[i][j]| (fp16 widened exactly to fp32).  Column j is an
 * outlier when colmax[j] > threshold (strict; threshold compared in fp32).
 *   X       fp16 [M x K]
 *   mask    u8 [K]: 1 for an outlier column, else 0
 *   idx     i32 [K]: the outlier columns in ascending order in idx[0..count)
 *           (entries from count on are unspecified)
 *   count   i32 [1]: number of outlier columns
 *   colmax  f32 [K] or NULL
 *   scratch device buffer of qa_outlier_cols_workspace(K) bytes (any content)
 * Errors: NULL pointers, M < 0, K <= 0, K > 2^22, K % 8 != 0, X not 16-byte
 * aligned, NaN threshold, small scratch.
 * ------------------------------------------------------------------------- */
size_t qa_outlier_cols_workspace(int64_t K);
qa_status qa_outlier_cols(const void* X_f16, int64_t M, int64_t K, float threshold,
                          uint8_t* mask, int32_t* idx, int32_t* count, float* colmax_or_null,
                          void* scratch, size_t scratch_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Top-k outlier columns  [AIInfra-Q01: decompose the largest-magnitude 1-2%
 * of feature dimensions]
 *
 * Same outputs as qa_outlier_cols, but the set is the k columns with the
 * largest colmax[j] = max_i |X[i][j]|; equal maxima are taken in ascending
 * column order, so exactly k columns are chosen.  k = ceil(p K) decomposes
 * the share p of the dimensions.
 *   scratch qa_outlier_cols_workspace(K) bytes (any content)
 * Errors: as qa_outlier_cols, plus K > 32768 (QA_ERR_SHAPE), k < 0 or
 * k > K (QA_ERR_VALUE).
 * ------------------------------------------------------------------------- */
qa_status qa_outlier_topk(const void* X_f16, int64_t M, int64_t K, int64_t k, uint8_t* mask, int32_t* idx,
                          int32_t* count, float* colmax_or_null, void* scratch, size_t scratch_bytes,
                          void* stream);

/* ---------------------------------------------------------------------------
 * Row-wise int8 quantization  [AIInfra-Q01 "a. 向量级量化"; Scholia-IQ §4,
 * §6.2]
 *
 * One scale per row of X [rows x K] (per token for activations, per output
 * channel for a weight [N x K]).
 *   Dynamic (s_in == NULL): s[r] = absmax over the unmasked columns of row r
 *     divided by q_max (1.0 if that absmax is 0), z = 0, written to s_out[r].
 *     Requires q_max > 0 and z_in == NULL.
 *   Static (s_in != NULL): s = s_in[r] (> 0, finite: not checked),
 *     z = z_in ? z_in[r] : 0; s_out is ignored.
 *   Xq[r][j] = clip(rint(x / s) + z, q_min, q_max); a masked column j
 *     (mask[j] != 0) is skipped by the absmax and receives clip(z).
 *   X       fp16 [rows x K]; mask u8 [K] or NULL; Xq i8 [rows x K]
 * Errors: NULL X / Xq (or s_out in dynamic mode), rows < 0, K <= 0,
 * K > 2^26, K % 8 != 0, X or Xq not 16-byte aligned, q_min > q_max, range outside
 * [-128, 127], dynamic mode with q_max <= 0 or z_in != NULL.
 * ------------------------------------------------------------------------- */
qa_status qa_quantize_rowwise_int8(const void* X_f16, int64_t rows, int64_t K,
                                   const uint8_t* mask_or_null, int32_t q_min, int32_t q_max,
                                   const float* s_in_or_null, const int32_t* z_in_or_null,
                                   int8_t* Xq, float* s_out_or_null, void* stream);

/* ---------------------------------------------------------------------------
 * LLM.int8() mixed-precision linear  [AIInfra-Q01: detection, "a. 向量级量化",
 * "b. INT8 矩阵乘法与反量化", merge; QE2 §1.2]
 *
 *   O       = { j : max_i |X[i][j]| > threshold }            (all M rows)
 *   s_x[m]  = max_{j not in O} |X[m][j]| / 127               (1.0 if 0)
 *   Xq[m][j]= clip(rint(X[m][j] / s_x[m]), -127, 127), 0 for j in O
 *   C[m][n] = sum_k Xq[m][k] * Wq[n][k]                      (int32)
 *   out     = C * s_x[m] * s_w[n] + sum_{h in O} X[m][h] * w~[n][h]
 * with fp16 outlier operands and fp32 accumulation; w~ = W_f16[n][h] when
 * W_f16 is given, else fp16(fl32(s_w[n] * Wq[n][h])).
 *   X       fp16 [M x K]
 *   Wq, s_w the weight quantized per output channel (qa_quantize_rowwise_int8
 *           on W [N x K], q range [-127, 127]): i8 [N x K], f32 [N]
 *   W_f16   fp16 [N x K] or NULL
 *   out     [M x N] of out_dtype (fp32, fp16 or bf16, round to nearest even)
 *   workspace  qa_qlinear_int8_mixed_workspace(M, K) bytes (any content);
 *           holds the outlier mask / list / count, s_x and Xq
 * threshold = +inf gives plain vector-wise W8A8; a negative threshold sends
 * every column through the fp16 product.
 * Errors: NULL pointers, M < 0, N < 0, K <= 0, K % 16 != 0, misaligned
 * pointers, NaN threshold, bad out_dtype, small workspace.
 * ------------------------------------------------------------------------- */
size_t qa_qlinear_int8_mixed_workspace(int64_t M, int64_t K);
qa_status qa_qlinear_int8_mixed(const void* X_f16, int64_t M, int64_t K,
                                const int8_t* Wq, const float* s_w, const void* W_f16_or_null,
                                int64_t N, float threshold, void* out, qa_dtype out_dtype,
                                void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Where the integer stages of an LLM.int8() call sit in its workspace
 * [AIInfra-Q01: detection and "a. 向量级量化"]
 *
 * After qa_qlinear_int8_mixed or qa_qlinear_int8_topk with M, N > 0 has
 * completed on its stream, its workspace holds, at these byte offsets:
 *   offsets[0]  idx    i32 [count]: the outlier columns O, ascending
 *   offsets[1]  count  i32 [1]:     |O|
 *   offsets[2]  s_x    f32 [M]:     the per-token scales
 *   offsets[3]  Xq     i8 [M x K]:  the int8 codes the GEMM consumed
 *                                   (0 in the columns of O)
 * i.e. exactly the values qa_outlier_cols (or qa_outlier_topk) and
 * qa_quantize_rowwise_int8 with that mask produce for the same X.  The
 * offsets depend only on M and K.  offsets: a HOST array of 4 entries.
 * Errors: M <= 0, K <= 0 (QA_ERR_SHAPE), offsets NULL (QA_ERR_NULL).
 * ------------------------------------------------------------------------- */
qa_status qa_qlinear_int8_mixed_offsets(int64_t M, int64_t K, size_t* offsets);

/* ---------------------------------------------------------------------------
 * LLM.int8() mixed linear without a workspace  -- for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.
 *
 * Same arguments, kernels and results as qa_qlinear_int8_mixed, minus the
 * workspace: the call's scratch lives in a static device array of
 * QA_NOALLOC_SCRATCH_BYTES (40 MiB) that every GPU the library runs on holds
 * until the process ends.  The call allocates nothing (no hipMalloc, hipFree
 * or allocating library routine); the caller still provides X, Wq, s_w,
 * W_f16 and out.  Nothing in the scratch needs clearing: every slot a call
 * reads was written earlier in the same call.  All calls on one GPU share
 * that one array, so calls that overlap on one GPU (on different streams,
 * without ordering between them) race and give undefined results; calls on
 * one stream, or otherwise ordered, are safe.  After the call the scratch
 * holds the integer stages at the offsets of qa_qlinear_int8_mixed_offsets
 * (until the next call on that GPU).
 * Errors: as qa_qlinear_int8_mixed, and QA_ERR_WORKSPACE when
 * qa_qlinear_int8_mixed_workspace(M, K) > QA_NOALLOC_SCRATCH_BYTES (e.g.
 * M x K above about 33.5 million); QA_ERR_DEVICE if the scratch's device
 * address cannot be looked up.
 * ------------------------------------------------------------------------- */
#define QA_NOALLOC_SCRATCH_BYTES ((size_t)40 << 20)
qa_status qa_qlinear_int8_mixed_noalloc(const void* X_f16, int64_t M, int64_t K, const int8_t* Wq,
                                        const float* s_w, const void* W_f16_or_null, int64_t N, float threshold,
                                        void* out, qa_dtype out_dtype, void* stream);

/* ---------------------------------------------------------------------------
 * LLM.int8() linear with top-k decomposition  [AIInfra-Q01: decomposition
 * share raised to the top 1-2% of feature dimensions]
 *
 * qa_qlinear_int8_mixed with O = the k columns of qa_outlier_topk instead of
 * the threshold set; everything else (scales, codes, GEMM, fp16 outlier
 * product) is identical.  k = 0 is plain vector-wise W8A8; k = K sends every
 * column through the fp16 product.
 *   workspace  qa_qlinear_int8_topk_workspace(M, K) bytes (any content)
 * Errors: as qa_qlinear_int8_mixed (no threshold), plus K > 32768
 * (QA_ERR_SHAPE), k < 0 or k > K (QA_ERR_VALUE).
 * ------------------------------------------------------------------------- */
size_t qa_qlinear_int8_topk_workspace(int64_t M, int64_t K);
qa_status qa_qlinear_int8_topk(const void* X_f16, int64_t M, int64_t K, int64_t k, const int8_t* Wq,
                               const float* s_w, const void* W_f16_or_null, int64_t N, void* out,
                               qa_dtype out_dtype, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Block Hadamard rotation fused with int4 quantization and packing
 * [GroupRot §二, §5.1, §5.2, §5.4; Scholia-IQ §7.3]
 *
 *   X'[r][b*G + j] = fl32( fl64(1/sqrt(G)) * sum_i X[r][b*G + i] * H[i][j] ),
 *   H[i][j] = (-1)^popcount(i & j) (Sylvester order); the +-1 sum is exact.
 *   PER_ROW:   s[r]    = absmax(X'[r][:]) / q_max                (s: [rows])
 *   PER_GROUP: s[r][b] = absmax(X'[r][bG:(b+1)G]) / q_max        (s: [rows x K/G])
 *   code = clip(rint(X' / s), q_min, q_max); element 8w+i of a row is the
 *   two's-complement nibble in bits [4i+3:4i] of packed[r][w].
 *   G = 1 is the identity rotation.
 *   X       fp16 [rows x K]; packed u32 [rows x K/8]; s f32 as above
 * Errors: NULL pointers, rows < 0, K <= 0, K % 8 != 0, K % G != 0, G not a
 * power of two in [1, 256], PER_GROUP with G < 8, q range outside [-8, 7],
 * q_max <= 0, q_min > q_max, misaligned X / packed.
 * ------------------------------------------------------------------------- */
qa_status qa_hadamard_quant_int4(const void* X_f16, int64_t rows, int64_t K, int32_t G,
                                 qa_scale_mode mode, int32_t q_min, int32_t q_max,
                                 uint32_t* packed, float* s, void* stream);

/* ---------------------------------------------------------------------------
 * W4A4 group-Hadamard linear  [GroupRot §5.2, §5.4]
 *
 *   (Xp, s_x) = qa_hadamard_quant_int4(X, G, PER_ROW, -7, 7)  (on device)
 *   acc_g[m][n] = sum_{k in group g} qx[m][k] * qw[n][k]     (int32)
 *   out[m][n]   = s_x[m] * sum_g s_w[n][g] * acc_g[m][n]
 *   X       fp16 [M x K]
 *   Wp, s_w the offline weight: qa_hadamard_quant_int4(W, G, PER_GROUP, ...)
 *           u32 [N x K/8], f32 [N x K/G]
 *   out     [M x N] of out_dtype
 *   workspace  qa_qlinear_w4a4_workspace(M, K) bytes (any content)
 * Errors: NULL pointers, M < 0, N < 0, K <= 0, G not a power of two in [8, 256],
 * K % G != 0, misaligned pointers, bad out_dtype, small workspace.
 * ------------------------------------------------------------------------- */
size_t qa_qlinear_w4a4_workspace(int64_t M, int64_t K);
qa_status qa_qlinear_w4a4(const void* X_f16, int64_t M, int64_t K, const uint32_t* Wp,
                          const float* s_w, int64_t N, int32_t G, void* out, qa_dtype out_dtype,
                          void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Hadamard rotation + per-row int8 codes  [GroupRot §二, §5.2: the rotation
 * fused with dynamic per-token quantization; Scholia-IQ §2.2: 8-bit
 * activations of W4A8]
 *
 *   X'[r] = X[r] * blockdiag(H_G) / sqrt(G)   (as qa_hadamard_quant_int4)
 *   s[r]  = fl32(max_j |X'[r][j]| / q_max)     (1.0 for an all-zero row)
 *   q[r][j] = clip(rint(fl32(X'[r][j] / s[r])), q_min, q_max)
 *   X fp16 [rows x K]; q i8 [rows x K]; s f32 [rows]
 * Errors: NULL pointers, rows < 0, K <= 0, K % 8 != 0, G not a power of two
 * in [1, 256], K % G != 0, q_min > q_max, q_min < -128, q_max > 127,
 * q_max <= 0, misaligned X (16 bytes) / q (8 bytes) / s.
 * ------------------------------------------------------------------------- */
qa_status qa_hadamard_quant_int8(const void* X_f16, int64_t rows, int64_t K, int32_t G, int32_t q_min,
                                 int32_t q_max, int8_t* q, float* s, void* stream);

/* ---------------------------------------------------------------------------
 * W4A8 group-Hadamard linear  [Scholia-IQ §2.1-§2.2: 4-bit weights, 8-bit
 * activations; "从离群值到平坦线" §4: a transform fitted for W4A4 serves W4A8
 * unchanged; GroupRot §5.2, §5.4]
 *
 *   (Xq, s_x) = qa_hadamard_quant_int8(X, G, -127, 127)   (on device)
 *   acc_g[m][n] = sum_{k in group g} Xq[m][k] * qw[n][k]   (int32)
 *   out[m][n]   = s_x[m] * sum_g s_w[n][g] * acc_g[m][n]
 *   Wp, s_w  the offline W4A4 weight: qa_hadamard_quant_int4(W, G, PER_GROUP,
 *            -7, 7): u32 [N x K/8], f32 [N x K/G]
 *   out      [M x N] of out_dtype
 *   workspace  qa_qlinear_w4a8_workspace(M, K) bytes (any content)
 * Errors: NULL pointers, M < 0, N < 0, K <= 0, G not a power of two in [8, 256],
 * K % G != 0, misaligned pointers, bad out_dtype, small workspace.
 * ------------------------------------------------------------------------- */
size_t qa_qlinear_w4a8_workspace(int64_t M, int64_t K);
qa_status qa_qlinear_w4a8(const void* X_f16, int64_t M, int64_t K, const uint32_t* Wp,
                          const float* s_w, int64_t N, int32_t G, void* out, qa_dtype out_dtype,
                          void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Hadamard rotation + zero-point int4 codes per row  [GroupRot §二, §5.2;
 * Scholia-IQ §6 (q = round(x/s) + z, x^ = s (q - z)), §6.2 (the grid on the
 * data's range, clip to [q_min, q_max])]
 *
 *   X'[r] = X[r] * blockdiag(H_G) / sqrt(G)       (as qa_hadamard_quant_int4)
 *   [lo, hi] = [min(min X'[r], 0), max(max X'[r], 0)]
 *   s[r] = fl32(fl32(hi - lo) / 15)   (1.0 when hi == lo)
 *   z[r] = clip(-rint(fl32(lo / s[r])), 0, 15)
 *   q = clip(rint(fl32(X'[r][j] / s[r])) + z[r], 0, 15), packed eight per
 *   word as the two's complement nibble q - 8 (element 8w+i in bits
 *   [4i+3:4i] of word w)
 *   X fp16 [rows x K]; packed u32 [rows x K/8]; s f32, z i32 [rows]
 * Errors: NULL pointers, rows < 0, K <= 0, K % 8 != 0, G not a power of two
 * in [1, 256], K % G != 0, misaligned pointers.
 * ------------------------------------------------------------------------- */
qa_status qa_hadamard_quant_int4_asym(const void* X_f16, int64_t rows, int64_t K, int32_t G, uint32_t* packed,
                                      float* s, int32_t* z, void* stream);

/* Column terms of a per-group int4 weight (offline, with the weight):
 *   c[n] = fl32(sum_g s_w[n][g] * sum_{k in group g} qw[n][k])   (fp64, g ascending)
 *   Wp u32 [N x K/8], s_w f32 [N x K/G]; c f32 [N]
 * Errors: NULL pointers, N < 0, K <= 0, G not a power of two in [8, 256],
 * K % G != 0, misaligned pointers. */
qa_status qa_w4_column_terms(const uint32_t* Wp, const float* s_w, int64_t N, int64_t K, int32_t G, float* c,
                             void* stream);

/* ---------------------------------------------------------------------------
 * W4A4 linear with zero-point activations  [Scholia-IQ §6, §6.2, §7.3;
 * GroupRot §5.2, §5.4]
 *
 *   (Xp, s_x, z_x) = qa_hadamard_quant_int4_asym(X, G)   (on device)
 *   out[m][n] = s_x[m] * sum_g s_w[n][g] * sum_{k in g} (q[m][k] - z_x[m]) qw[n][k]
 *             = s_x[m] * (sum_g s_w[n][g] sum_{k in g} (q - 8) qw - (z_x[m] - 8) c_w[n])
 *   Wp, s_w  the offline W4A4 weight (qa_hadamard_quant_int4, PER_GROUP)
 *   c_w      qa_w4_column_terms(Wp, s_w, G): f32 [N]
 *   out      [M x N] of out_dtype
 *   workspace  qa_qlinear_w4a4_asym_workspace(M, K) bytes (any content)
 * Errors: NULL pointers, M < 0, N < 0, K <= 0, G not a power of two in [8, 256],
 * K % G != 0, misaligned pointers, bad out_dtype, small workspace.
 * ------------------------------------------------------------------------- */
size_t qa_qlinear_w4a4_asym_workspace(int64_t M, int64_t K);
qa_status qa_qlinear_w4a4_asym(const void* X_f16, int64_t M, int64_t K, const uint32_t* Wp, const float* s_w,
                               const float* c_w, int64_t N, int32_t G, void* out, qa_dtype out_dtype,
                               void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Asymmetric (zero-point) row quantization  [Scholia-IQ §6: q = round(x/s) +
 * z, x^ = s (q - z), z the integer that stands for real 0; §6.2: the grid
 * shifted onto the data's range, q clipped to [q_min, q_max]]
 *
 * Per row r (the pages leave the choice of s and z open; min-max is taken):
 *   lo = min(min_j X[r][j], 0), hi = max(max_j X[r][j], 0)
 *   s  = fl32(fl32(hi - lo) / (q_max - q_min))      (1.0 when hi == lo)
 *   z  = clip(q_min - rint(fl32(lo / s)), q_min, q_max)
 *   q[r][j]   = clip(rint(fl32(X[r][j] / s)) + z, q_min, q_max)
 *   rowsum[r] = sum_j q[r][j]                          (if rowsum != NULL)
 *   X fp16 [rows x K]; q i8 [rows x K]; s_out f32, z_out i32, rowsum i32 [rows]
 * Errors: NULL pointers, rows < 0, K <= 0, K > 2^26, K % 8 != 0, X or q not
 * 16-byte aligned, q_min >= q_max or outside [-128, 127].
 * ------------------------------------------------------------------------- */
qa_status qa_quantize_rowwise_int8_asym(const void* X_f16, int64_t rows, int64_t K, int32_t q_min, int32_t q_max,
                                        int8_t* q, float* s_out, int32_t* z_out, int32_t* rowsum_or_null,
                                        void* stream);

/* Row sums of int8 rows: sums[r] = sum_j A[r][j] (the weight term of the
 * zero-point correction below for a weight quantized without zero-point).
 * Errors: NULL pointers, rows < 0, K <= 0, K > 2^26, K % 16 != 0, A not
 * 16-byte aligned. */
qa_status qa_int8_row_sums(const int8_t* A, int64_t rows, int64_t K, int32_t* sums, void* stream);

/* ---------------------------------------------------------------------------
 * W8A8 linear with zero-point activations  [Scholia-IQ §6, §6.2;
 * AIInfra-Q01 "b. INT8 矩阵乘法与反量化"]
 *
 *   (Xq, s_x, z_x) = qa_quantize_rowwise_int8_asym(X, -128, 127)  (per token,
 *                    on device)
 *   out[m][n] = s_x[m] s_w[n] sum_k (Xq[m][k] - z_x[m]) (Wq[n][k] - z_w[n])
 * evaluated as C - z_x a[n] - z_w[n] r_x[m] with C the int32 GEMM,
 * a[n] = w_rowsum[n] - K z_w[n] and r_x the activation code sums (exact).
 *   Wq i8 [N x K], s_w f32 [N]: the weight (symmetric from
 *           qa_quantize_rowwise_int8, or asymmetric from
 *           qa_quantize_rowwise_int8_asym with z_w = its z_out)
 *   z_w     i32 [N] or NULL (zero-point 0)
 *   w_rowsum  i32 [N]: sum_k Wq[n][k] (rowsum_out of the asymmetric
 *           quantizer, or qa_int8_row_sums)
 *   out     [M x N] of out_dtype
 *   workspace  qa_qlinear_int8_asym_workspace(M, K) bytes (any content)
 * Errors: NULL pointers, M < 0, N < 0, K <= 0, K % 16 != 0, K > 32768 (the
 * integer sum must fit int32), misaligned pointers, bad out_dtype, small
 * workspace.
 * ------------------------------------------------------------------------- */
size_t qa_qlinear_int8_asym_workspace(int64_t M, int64_t K);
qa_status qa_qlinear_int8_asym(const void* X_f16, int64_t M, int64_t K, const int8_t* Wq, const float* s_w,
                               const int32_t* z_w_or_null, const int32_t* w_rowsum, int64_t N, void* out,
                               qa_dtype out_dtype, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Column absolute maxima  [QE2 §4.2: max|X_j| and max|W_j| per input channel]
 *
 *   colmax[j] = max_r |A[r][j]|  (accumulate == 0)
 *   colmax[j] = max(colmax[j], max_r |A[r][j]|)  (accumulate != 0: a running
 *               maximum over calibration batches; colmax must then hold
 *               non-negative finite values, e.g. from an earlier call)
 * For activations A = X [M x K]; for the weight A = W [N x K] gives the
 * maximum over output channels of each input channel.  Exact (fp16 widened).
 *   A       fp16 [rows x K]; colmax f32 [K]
 *   scratch device buffer of qa_col_absmax_workspace(K) bytes (any content)
 * rows == 0 is a no-op.
 * Errors: NULL pointers, rows < 0, K <= 0, K > 2^22, K % 8 != 0, A not
 * 16-byte aligned, small scratch.
 * ------------------------------------------------------------------------- */
size_t qa_col_absmax_workspace(int64_t K);
qa_status qa_col_absmax(const void* A_f16, int64_t rows, int64_t K, float* colmax, int accumulate,
                        void* scratch, size_t scratch_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * SmoothQuant migration factors  [QE2 §4.2]
 *
 *   s[j] = fl32( pow(act_absmax[j], alpha) / pow(w_absmax[j], 1 - alpha) )
 * evaluated in fp64 (alpha widened exactly from fp32); s[j] = 1 when either
 * maximum is 0.  alpha = 0.5 splits the range evenly; alpha = 1 gives
 * s = act_absmax (activation columns scaled to magnitude 1); alpha = 0 gives
 * s = 1 / w_absmax.  The fp64 pow of the device math library may differ from
 * another implementation's by one rounding, so s can differ in the last fp32
 * bit; the smoothing below takes s as given.
 *   act_absmax, w_absmax  f32 [K], non-negative finite
 *   s       f32 [K]
 * Errors: NULL pointers, K < 0, alpha NaN or outside [0, 1].  K == 0 is a
 * no-op.
 * ------------------------------------------------------------------------- */
qa_status qa_smooth_factors(const float* act_absmax, const float* w_absmax, int64_t K, float alpha, float* s,
                            void* stream);

/* ---------------------------------------------------------------------------
 * Smoothing fused with int8 quantization  [QE2 §4.2; Scholia-IQ §4, §7]
 *
 *   a^[r][j] = fl32(A[r][j] / s[j])   (QA_SMOOTH_DIVIDE: activations)
 *   a^[r][j] = fl32(A[r][j] * s[j])   (QA_SMOOTH_MULTIPLY: the weight W [N x K],
 *                                      offline)
 *   QA_SCALE_PER_ROW:    s_out[r] = fl32(max_j |a^[r][j]| / 127)
 *   QA_SCALE_PER_TENSOR: s_out[r] = fl32(max_{r,j} |a^[r][j]| / 127) for every r
 *   (1.0 for an all-zero row / tensor)
 *   q[r][j]  = clip(rint(a^[r][j] / s_out[r]), -127, 127)
 *   A       fp16 [rows x K]; s f32 [K], positive finite; q i8 [rows x K];
 *   s_out   f32 [rows]
 * Errors: NULL pointers, rows < 0, K <= 0, K > 2^26, K % 8 != 0, A or q not
 * 16-byte aligned, bad op, mode not PER_ROW / PER_TENSOR.  rows == 0 is a
 * no-op.
 * ------------------------------------------------------------------------- */
qa_status qa_quantize_smooth_int8(const void* A_f16, int64_t rows, int64_t K, const float* s, qa_smooth_op op,
                                  qa_scale_mode mode, int8_t* q, float* s_out, void* stream);

/* ---------------------------------------------------------------------------
 * SmoothQuant W8A8 linear  [QE2 §4.2, §4.4; AIInfra-Q01 "b. INT8 矩阵乘法与反量化"]
 *
 *   (Xq, s_x) = qa_quantize_smooth_int8(X, s, QA_SMOOTH_DIVIDE, mode)  (on device)
 *   C[m][n]   = sum_k Xq[m][k] * Wq[n][k]                              (int32)
 *   out       = C * s_x[m] * s_w[n]
 *   X       fp16 [M x K]; s f32 [K] (qa_smooth_factors)
 *   Wq, s_w the smoothed weight: qa_quantize_smooth_int8(W, s,
 *           QA_SMOOTH_MULTIPLY, QA_SCALE_PER_ROW): i8 [N x K], f32 [N]
 *   mode    QA_SCALE_PER_ROW (per token) or QA_SCALE_PER_TENSOR for X
 *   out     [M x N] of out_dtype
 *   workspace  qa_qlinear_int8_smooth_workspace(M, K) bytes (any content);
 *           after the call it holds s_x and Xq
 * Decode shapes (K % 256 == 0 with M <= 8 at K <= 4096 or M <= 4 at
 * K <= 8192) run as one kernel that smooths, quantizes and multiplies; the
 * results are the same bits.
 * Errors: NULL pointers, M < 0, N < 0, K <= 0, K % 16 != 0, K > 131072,
 * misaligned pointers, bad mode or out_dtype, small workspace.
 * ------------------------------------------------------------------------- */
size_t qa_qlinear_int8_smooth_workspace(int64_t M, int64_t K);
qa_status qa_qlinear_int8_smooth(const void* X_f16, int64_t M, int64_t K, const float* s, qa_scale_mode mode,
                                 const int8_t* Wq, const float* s_w, int64_t N, void* out, qa_dtype out_dtype,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Kronecker affine transform fused with int4 quantization  [AIInfra-Q01,
 * FlatQuant section: X~ x1 P1^T x2 P2, P = P1 (x) P2, dynamic int4 codes in one
 * kernel]
 *
 * Each row x (K = n1 n2) is read as X~[i][j] = x[i n2 + j] and transformed to
 * X' = P1^T X~ P2 (= x (P1 (x) P2)), mode 1 first, every output one fp32 chain
 * of fused multiply-adds over the contraction index in ascending order:
 *   Y[a][j]  = sum_i P1[i][a] X~[i][j],   X'[a][b] = sum_j Y[a][j] P2[j][b].
 * Then int4 codes of X' as qa_hadamard_quant_int4 makes them (PER_ROW: one
 * scale per row; PER_GROUP: per G-wide group), packed eight per word.
 * Activations take the learned P1, P2; the offline weight takes P1^-T, P2^-T
 * (the same matrices when they are orthogonal), so X' W'^T = X W^T.
 *   X       fp16 [rows x K]; P1 f32 [n1 x n1], P2 f32 [n2 x n2] row-major
 *   packed  u32 [rows x K/8]; s f32 [rows] or [rows x K/G]
 * Sizes with a kernel: (n1, n2) in {(8,8), (8,16), (16,16), (16,32), (32,32),
 * (32,64), (64,64), (64,128)} -- the minimal-sum splits of 64 .. 8192; per
 * group, G a multiple of 8 with a group inside one wave's chunks.
 * Errors: NULL pointers, rows < 0, n1 n2 != K (QA_ERR_SHAPE), no kernel for
 * the sizes (QA_ERR_UNSUPPORTED), bad mode / q range, misaligned pointers.
 * ------------------------------------------------------------------------- */
qa_status qa_kron_quant_int4(const void* X_f16, int64_t rows, int64_t K, int64_t n1, int64_t n2, const float* P1,
                             const float* P2, qa_scale_mode mode, int32_t G, int32_t q_min, int32_t q_max,
                             uint32_t* packed, float* s, void* stream);

/* ---------------------------------------------------------------------------
 * Kronecker factor sizes  [AIInfra-Q01, FlatQuant section (the split of P
 * into P1 (x) P2 minimizes n1 + n2 under n1 n2 = n, n1 <= n2; n = 8192 gives
 * 64 x 128); 从离群值到平坦线：FlatQuant 如何重塑 LLM 的 4-bit 量化格局, §2
 * (4096 as 64 x 64)]
 *
 *   n1 = the largest divisor of n not above sqrt(n), n2 = n / n1: the pair
 *   with n1 n2 = n, n1 <= n2 and the smallest n1 + n2.  Host arithmetic, no
 *   device work.
 *   n           transform width (K), > 0
 *   n1, n2      host int64 outputs
 *   has_kernel  host int32 output, may be NULL: 1 when qa_kron_quant_int4 and
 *               qa_qlinear_kron_w4a4 have a kernel for (n1, n2), else 0
 * Errors: NULL n1 or n2 (QA_ERR_NULL), n <= 0 (QA_ERR_SHAPE); the outputs
 * are untouched on error.
 * ------------------------------------------------------------------------- */
qa_status qa_kron_sizes(int64_t n, int64_t* n1, int64_t* n2, int32_t* has_kernel);

/* ---------------------------------------------------------------------------
 * W4A4 linear with the Kronecker transform  [AIInfra-Q01, FlatQuant section:
 * transform + dynamic int4 of X in one kernel, int4 GEMM with the
 * pre-transformed int4 weight]
 *
 *   (Xp, s_x) = qa_kron_quant_int4(X, n1, n2, P1, P2, PER_ROW, -7, 7)
 *   out[m][n] = s_x[m] sum_g s_w[n][g] sum_{k in g} qx[m][k] qw[n][k]
 *   Wp, s_w  the offline weight: qa_kron_quant_int4(W, n1, n2, P1^-T, P2^-T,
 *            PER_GROUP, G, -7, 7): u32 [N x K/8], f32 [N x K/G]
 *   out      [M x N] of out_dtype
 *   workspace  qa_qlinear_kron_w4a4_workspace(M, K) bytes (any content)
 * Errors: NULL pointers, M < 0, N < 0, G not a power of two in [8, 256], K % G != 0,
 * n1 n2 != K, unsupported sizes, misaligned pointers, bad out_dtype, small
 * workspace.
 * ------------------------------------------------------------------------- */
size_t qa_qlinear_kron_w4a4_workspace(int64_t M, int64_t K);
qa_status qa_qlinear_kron_w4a4(const void* X_f16, int64_t M, int64_t K, int64_t n1, int64_t n2, const float* P1,
                               const float* P2, const uint32_t* Wp, const float* s_w, int64_t N, int32_t G, void* out,
                               qa_dtype out_dtype, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Parity entry points: the integer accumulators of the two GEMMs, stored.
 *
 * qa_gemm_i8_i32  [AIInfra-Q01 "b. INT8 矩阵乘法与反量化"]
 *   C[m][n] = sum_k A[m][k] * B[n][k]; A i8 [M x K], B i8 [N x K],
 *   C i32 [M x N].  The caller keeps |C| < 2^31 (K * 128^2 < 2^31 suffices).
 *   Errors: NULL, M < 0, N < 0, K <= 0, K % 16 != 0, misaligned pointers.
 *
 * qa_gemm_w4a4_group_acc  [GroupRot §5.4]
 *   acc[m][n][g] = sum_{k in group g} qx[m][k] * qw[n][k] from packed int4
 *   Xp u32 [M x K/8], Wp u32 [N x K/8]; acc i32 [M x N x K/G].
 *   Errors: NULL, M < 0, N < 0, K <= 0, G not a power of two in [8, 256],
 *   K % G != 0, misaligned pointers.
 *
 * qa_gemm_w4a8_group_acc  [GroupRot §5.4; Scholia-IQ §2.2]
 *   acc[m][n][g] = sum_{k in group g} Xq[m][k] * qw[n][k] from int8 codes
 *   Xq i8 [M x K] and packed int4 Wp u32 [N x K/8]; acc i32 [M x N x K/G].
 *   Errors as qa_gemm_w4a4_group_acc (Xq 16-byte aligned).
 * ------------------------------------------------------------------------- */
qa_status qa_gemm_i8_i32(const int8_t* A, const int8_t* B, int64_t M, int64_t K, int64_t N,
                         int32_t* C, void* stream);
qa_status qa_gemm_w4a4_group_acc(const uint32_t* Xp, const uint32_t* Wp, int64_t M, int64_t K,
                                 int64_t N, int32_t G, int32_t* acc, void* stream);
qa_status qa_gemm_w4a8_group_acc(const int8_t* Xq, const uint32_t* Wp, int64_t M, int64_t K,
                                 int64_t N, int32_t G, int32_t* acc, void* stream);

/* ---------------------------------------------------------------------------
 * Measurement helper, not part of the method: the single-launch HBM read
 * floor that the decode kernel (one launch streaming the whole int8 weight)
 * is compared with.
 *
 * qa_probe_stream_read
 *   Reads src[0 .. bytes) once with wgs workgroups of 512 threads, each a
 *   contiguous slice; every load instruction moves lane_bytes bytes per lane
 *   (64 * lane_bytes contiguous bytes per wave instruction) and `unroll`
 *   loads per lane are in flight before any is used.  The data are folded
 *   into a value stored to sink[wg * 512 + thread] only if it equals a fixed
 *   constant (so sink is normally left untouched; it must hold wgs * 512
 *   u32).  bytes == 0 launches the same grid with nothing to read (the cost
 *   of the launch itself).
 *   src: device, 16-byte aligned; sink: device u32 [wgs * 512].
 *   Errors: NULL pointers, wgs not in [1, 65536], lane_bytes not 4, 8 or 16,
 *   unroll not 1, 2, 4 or 8, misaligned src.
 * ------------------------------------------------------------------------- */
qa_status qa_probe_stream_read(const void* src, size_t bytes, int32_t wgs, int32_t lane_bytes, int32_t unroll,
                               uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QA_H */
