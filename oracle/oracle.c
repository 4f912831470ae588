/*
 * oracle.c -- plain, slow CPU reference for the quantized linear layer.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load this library.  It shares no code, header, table or
 * helper with the GPU library, and the GPU library never calls it.
 *
 * What it computes (sources are cited by page title and section):
 *
 *   [AIInfra-Q01]  Infrasys-AI "AIInfra" notes, page 05Quantization01
 *                  (模型量化): the LLM.int8() method -- outlier detection by a
 *                  magnitude threshold, "a. 向量级量化" (vector-wise scales),
 *                  "b. INT8 矩阵乘法与反量化" (int32 accumulation, dequant by
 *                  the outer product of the scales), and the merge of the fp16
 *                  outlier product with the int8 part.
 *   [Scholia-IQ]   "模型推理量化" (Inference Quantization notes): §2.1-§2.2
 *                  the WxAy notation (W4A8: 4-bit weights, 8-bit
 *                  activations), §4 Scale
 *                  (s = max|x|/qmax, q = round(x/s), x^ = s*q, all-zero input
 *                  needs a safe scale), §5 Outlier, §6 Zero-point and §6.2
 *                  affine clip q = clip(round(x/s)+z, qmin, qmax), §7.3
 *                  per-group scales.
 *   [GroupRot]     "低比特量化加速：分组旋转方法从W8A8到W4A4的实践与展望":
 *                  §二 normalized Hadamard rotation of G-wide blocks, §5.1
 *                  offline weight transform, §5.2 online activation transform
 *                  fused with dynamic quantization, §5.4 eight int4 per 32-bit
 *                  word and int32 accumulation.
 *   [FlatQuant]    AIInfra 05Quantization01, FlatQuant section (the apply
 *                  stage: X~ = X reshaped to [k x n1 x n2],
 *                  X' = X~ x1 P1^T x2 P2, dynamic int4 codes of X', int4
 *                  GEMM with the offline-transformed weight; Kronecker sizes
 *                  argmin (n1 + n2) with n1 n2 = n, n1 <= n2), and
 *                  "从离群值到平坦线" §2 (4096 = 64 x 64), §4 (a transform
 *                  fitted for W4A4 serves W4A8 unchanged).
 *   [QE2]          "Quantization explained, part 2" (tanjunchen.github.io):
 *                  §1.2, threshold 6.0 on a channel's activation magnitude and
 *                  the 4096-wide row with one value of 70; §4.2 SmoothQuant,
 *                  the per-input-channel migration Y = (X diag(s)^-1)(diag(s) W)
 *                  with s_j = max|X_j|^alpha / max|W_j|^(1-alpha).
 *
 * Arithmetic rules (the pages leave these open; the readings are fixed here):
 *   - fp16 inputs are widened exactly; all float reductions are fp64.
 *   - A scale is s = fl32(absmax / qmax) (IEEE fp32, correctly rounded), or
 *     1.0f when absmax is 0.  A code is clip(rint(fl32(x / s)) + z) with
 *     round-half-to-even.  Build with -ffp-contract=off, no fast-math.
 *   - Outlier column j: max_i |x_ij| > threshold (strict), compared in fp32.
 *   - Hadamard H_G[i][j] = (-1)^popcount(i & j) (Sylvester order), applied on
 *     the right of each G-wide block; the +-1 sum is exact in fp64, then one
 *     fp64 multiply by fl64(1/sqrt(G)) and one rounding to fp32.
 *   - int4 packing: element 8w+i of a row sits in bits [4i+3:4i] of word w,
 *     two's complement.
 *   - Asymmetric (zero-point) parameters, per row: lo = min(min_j x_j, 0),
 *     hi = max(max_j x_j, 0) (the range holds real 0, which z stands for),
 *     s = fl32(fl32(hi - lo) / (qmax - qmin)) (1.0 when hi == lo),
 *     z = clip(qmin - rint(fl32(lo / s)), qmin, qmax); codes by the affine rule.
 *   - Kronecker transform of a row x (X~[i][j] = x[i n2 + j]): X' = P1^T X~ P2,
 *     i.e. x (P1 (x) P2); mode 1 first, each output a chain of fp32 fused
 *     multiply-adds over the contraction index in ascending order, from 0
 *     (the codes are decided on these fp32 values).
 *   - SmoothQuant: s_j = fl32(pow(cx_j, alpha) / pow(cw_j, 1 - alpha)) in
 *     fp64, and s_j = 1 when cx_j or cw_j is 0 (the formula is undefined or
 *     zero there).  Activations become fl32(x / s_j), weights fl32(w * s_j),
 *     one IEEE fp32 operation each, before the absmax quantizer.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_F16 1
#define ORC_BF16 2

/* ---------------------------------------------------------------------------
 * Number formats, from the IEEE 754 definitions.
 * ------------------------------------------------------------------------- */

/* binary16 bit pattern -> exact double. */
double orc_f16_to_f64(uint16_t h)
{
    int sign = h >> 15;
    int e = (h >> 10) & 31;
    int m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);              /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);  /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* double -> bit pattern of a binary format with `mbits` fraction bits and
 * exponent bias `bias`, round to nearest, ties to even.  Used for fp16
 * (10, 15) and bf16 (7, 127). */
static uint32_t orc_round_small_float(double v, int mbits, int bias, int ebits)
{
    uint32_t sign = signbit(v) ? 1u : 0u;
    uint32_t emax_field = (1u << ebits) - 1u;
    uint32_t sign_bit = sign << (mbits + ebits);
    if (isnan(v))
        return sign_bit | (emax_field << mbits) | (1u << (mbits - 1));
    double a = fabs(v);
    /* largest finite value is (2 - 2^-mbits) * 2^(emax); the midpoint to the
     * next power of two rounds up to infinity (its neighbour below is odd). */
    int emax = (int)emax_field - 1 - bias;
    double overflow_mid = ldexp(2.0 - ldexp(1.0, -(mbits + 1)), emax);
    if (a >= overflow_mid)
        return sign_bit | (emax_field << mbits);
    int emin = 1 - bias;
    if (a < ldexp(1.0, emin)) {
        /* subnormal range: integer multiple of 2^(emin - mbits) */
        double q = rint(ldexp(a, mbits - emin));
        return sign_bit | (uint32_t)q;          /* q may reach 2^mbits = min normal */
    }
    int x;
    frexp(a, &x);                               /* a = f * 2^x, f in [0.5, 1) */
    int e = x - 1;                              /* unbiased exponent */
    double q = rint(ldexp(a, mbits - e));       /* in [2^mbits, 2^(mbits+1)] */
    uint32_t bits = ((uint32_t)(e + bias) << mbits) + ((uint32_t)q - (1u << mbits));
    return sign_bit | bits;                     /* a carry into the exponent is correct */
}

uint16_t orc_f64_to_f16(double v) { return (uint16_t)orc_round_small_float(v, 10, 15, 5); }
uint16_t orc_f64_to_bf16(double v) { return (uint16_t)orc_round_small_float(v, 7, 127, 8); }

/* Round `n` doubles to the output dtype (0 fp32, 1 fp16, 2 bf16). */
void orc_round_output(const double* in, int64_t n, int dtype, void* out)
{
    for (int64_t i = 0; i < n; ++i) {
        if (dtype == ORC_F32)
            ((float*)out)[i] = (float)in[i];
        else if (dtype == ORC_F16)
            ((uint16_t*)out)[i] = orc_f64_to_f16(in[i]);
        else
            ((uint16_t*)out)[i] = orc_f64_to_bf16(in[i]);
    }
}

void orc_f16_to_f32_array(const uint16_t* in, int64_t n, float* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = (float)orc_f16_to_f64(in[i]);
}

/* ---------------------------------------------------------------------------
 * Outlier feature columns  [AIInfra-Q01, LLM.int8() detection step;
 * QE2 §1.2: a channel whose activation magnitude exceeds 6.0 is an outlier]
 * ------------------------------------------------------------------------- */
void orc_outlier_cols(const uint16_t* X, int64_t M, int64_t K, float tau,
                      uint8_t* mask, int32_t* idx, int32_t* count, float* colmax)
{
    int32_t n = 0;
    for (int64_t j = 0; j < K; ++j) {
        float cm = 0.0f;
        for (int64_t i = 0; i < M; ++i) {
            float a = fabsf((float)orc_f16_to_f64(X[i * K + j]));
            if (a > cm)
                cm = a;
        }
        if (colmax)
            colmax[j] = cm;
        mask[j] = (cm > tau) ? 1 : 0;
        if (mask[j])
            idx[n++] = (int32_t)j;
    }
    *count = n;
}

/* ---------------------------------------------------------------------------
 * Top-k decomposition  [AIInfra-Q01, advice for training: raise the share of
 * decomposed feature dimensions to the largest-magnitude 1-2%]
 * O = the k columns with the largest max_i |x_ij|, chosen one at a time as
 * the largest remaining maximum, equal maxima in ascending column order.
 * k is clamped to [0, K].  idx lists O in ascending order.
 * ------------------------------------------------------------------------- */
void orc_outlier_topk(const uint16_t* X, int64_t M, int64_t K, int64_t k,
                      uint8_t* mask, int32_t* idx, int32_t* count, float* colmax)
{
    float* cm = (float*)malloc(sizeof(float) * (size_t)(K > 0 ? K : 1));
    int32_t none = 0;
    orc_outlier_cols(X, M, K, INFINITY, mask, idx, &none, cm);    /* column maxima; no column exceeds +inf */
    if (k < 0) k = 0;
    if (k > K) k = K;
    for (int64_t j = 0; j < K; ++j)
        mask[j] = 0;
    for (int64_t r = 0; r < k; ++r) {
        int64_t best = -1;
        for (int64_t j = 0; j < K; ++j)
            if (!mask[j] && (best < 0 || cm[j] > cm[best]))
                best = j;
        mask[best] = 1;
    }
    int32_t n = 0;
    for (int64_t j = 0; j < K; ++j)
        if (mask[j])
            idx[n++] = (int32_t)j;
    *count = n;
    if (colmax)
        memcpy(colmax, cm, sizeof(float) * (size_t)K);
    free(cm);
}

/* ---------------------------------------------------------------------------
 * Quantization of rows, [Scholia-IQ §4, §6.2, §7.3; AIInfra-Q01 "a. 向量级量化"]
 *
 * x is [rows x K] fp32; every `gsize` consecutive columns of a row share one
 * scale (gsize == K: one scale per row).  mask (may be NULL) marks columns
 * that are excluded from the absmax and receive the code that stands for 0.
 * Dynamic mode (s_in == NULL): s = absmax/qmax (1.0 if absmax is 0), z = 0,
 * scales written to s_out [rows x K/gsize].  Static mode: s = s_in[row],
 * z = z_in ? z_in[row] : 0 (gsize must equal K).
 * ------------------------------------------------------------------------- */
static int8_t orc_clip_code(double t, int32_t qmin, int32_t qmax)
{
    if (t < (double)qmin) return (int8_t)qmin;
    if (t > (double)qmax) return (int8_t)qmax;
    return (int8_t)(int32_t)t;
}

void orc_quant_rows_f32(const float* x, int64_t rows, int64_t K, int64_t gsize,
                        const uint8_t* mask, int32_t qmin, int32_t qmax,
                        const float* s_in, const int32_t* z_in,
                        int8_t* q, float* s_out)
{
    int64_t ngroups = K / gsize;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t g = 0; g < ngroups; ++g) {
            const float* xs = x + r * K + g * gsize;
            int8_t* qs = q + r * K + g * gsize;
            float s;
            int32_t z;
            if (s_in) {
                s = s_in[r];
                z = z_in ? z_in[r] : 0;
            } else {
                float a = 0.0f;
                for (int64_t j = 0; j < gsize; ++j) {
                    if (mask && mask[g * gsize + j])
                        continue;
                    float v = fabsf(xs[j]);
                    if (v > a)
                        a = v;
                }
                s = (a == 0.0f) ? 1.0f : a / (float)qmax;
                z = 0;
                s_out[r * ngroups + g] = s;
            }
            for (int64_t j = 0; j < gsize; ++j) {
                if (mask && mask[g * gsize + j]) {
                    qs[j] = orc_clip_code((double)z, qmin, qmax);
                    continue;
                }
                float t = rintf(xs[j] / s);     /* fp32 division, ties to even */
                qs[j] = orc_clip_code((double)t + (double)z, qmin, qmax);
            }
        }
    }
}

/* fp16 rows -> codes (int8 path). */
void orc_quant_rows_f16(const uint16_t* X, int64_t rows, int64_t K, int64_t gsize,
                        const uint8_t* mask, int32_t qmin, int32_t qmax,
                        const float* s_in, const int32_t* z_in,
                        int8_t* q, float* s_out)
{
    float* xf = (float*)malloc(sizeof(float) * (size_t)(rows * K > 0 ? rows * K : 1));
    orc_f16_to_f32_array(X, rows * K, xf);
    orc_quant_rows_f32(xf, rows, K, gsize, mask, qmin, qmax, s_in, z_in, q, s_out);
    free(xf);
}

/* ---------------------------------------------------------------------------
 * Integer GEMM with int32 accumulation  [AIInfra-Q01 "b. INT8 矩阵乘法与反量化"]
 * C[m][n] = sum_k A[m][k] * B[n][k]; A is [M x K], B is [N x K].
 * Summed in int64; returns the number of results that do not fit int32.
 * `rows` (may be NULL) selects the rows of A to compute; C is [nrows x N].
 * ------------------------------------------------------------------------- */
int64_t orc_gemm_i8_i32(const int8_t* A, const int8_t* B, int64_t M, int64_t K, int64_t N,
                        const int64_t* rows, int64_t nrows, int32_t* C)
{
    int64_t bad = 0;
    if (!rows)
        nrows = M;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : bad)
    for (int64_t ri = 0; ri < nrows; ++ri) {
        int64_t m = rows ? rows[ri] : ri;
        const int8_t* a = A + m * K;
        for (int64_t n = 0; n < N; ++n) {
            const int8_t* b = B + n * K;
            int64_t acc = 0;
            for (int64_t k = 0; k < K; ++k)
                acc += (int64_t)a[k] * (int64_t)b[k];
            if (acc > INT32_MAX || acc < INT32_MIN)
                ++bad;
            C[ri * N + n] = (int32_t)acc;
        }
    }
    return bad;
}

/* ---------------------------------------------------------------------------
 * LLM.int8() mixed-precision linear, step by step.
 *   1. O = outlier columns of X (all M rows)            [AIInfra-Q01 detection]
 *   2. per selected row: s_x = absmax over j not in O / 127, codes with the
 *      outlier columns set to 0                         ["a. 向量级量化"]
 *   3. C = sum_k Xq * Wq over all K (int32)             ["b. INT8 矩阵乘法"]
 *   4. normal part C * s_x * s_w (the outer product of the scales)
 *   5. outlier part sum_{h in O, ascending} X[m,h] * w~[n,h] with fp16
 *      operands; w~ = W16 if given, else fp16(fl32(s_w[n] * Wq[n,h]))
 *   6. out = outlier part + normal part                  [merge step]
 * Output is fp64 [nrows x N]; round with orc_round_output.
 * ------------------------------------------------------------------------- */
static void orc_mixed_with_set(const uint16_t* X, int64_t M, int64_t K,
                               const int8_t* Wq, const float* s_w, const uint16_t* W16,
                               int64_t N, const uint8_t* mask, const int32_t* idx, int32_t count,
                               const int64_t* rows, int64_t nrows, double* out);

void orc_qlinear_int8_mixed(const uint16_t* X, int64_t M, int64_t K,
                            const int8_t* Wq, const float* s_w, const uint16_t* W16,
                            int64_t N, float tau, const int64_t* rows, int64_t nrows,
                            double* out)
{
    uint8_t* mask = (uint8_t*)calloc((size_t)(K > 0 ? K : 1), 1);
    int32_t* idx = (int32_t*)calloc((size_t)(K > 0 ? K : 1), sizeof(int32_t));
    int32_t count = 0;
    orc_outlier_cols(X, M, K, tau, mask, idx, &count, NULL);
    orc_mixed_with_set(X, M, K, Wq, s_w, W16, N, mask, idx, count, rows, nrows, out);
    free(idx);
    free(mask);
}

/* The same linear with the outlier set O chosen as the top-k columns. */
void orc_qlinear_int8_topk(const uint16_t* X, int64_t M, int64_t K,
                           const int8_t* Wq, const float* s_w, const uint16_t* W16,
                           int64_t N, int64_t k, const int64_t* rows, int64_t nrows,
                           double* out)
{
    uint8_t* mask = (uint8_t*)calloc((size_t)(K > 0 ? K : 1), 1);
    int32_t* idx = (int32_t*)calloc((size_t)(K > 0 ? K : 1), sizeof(int32_t));
    int32_t count = 0;
    orc_outlier_topk(X, M, K, k, mask, idx, &count, NULL);
    orc_mixed_with_set(X, M, K, Wq, s_w, W16, N, mask, idx, count, rows, nrows, out);
    free(idx);
    free(mask);
}

/* Steps 2-6 for a given outlier set (mask, ascending idx, count). */
static void orc_mixed_with_set(const uint16_t* X, int64_t M, int64_t K,
                               const int8_t* Wq, const float* s_w, const uint16_t* W16,
                               int64_t N, const uint8_t* mask, const int32_t* idx, int32_t count,
                               const int64_t* rows, int64_t nrows, double* out)
{
    if (!rows)
        nrows = M;

    /* fp16 outlier weights w~, gathered as doubles [N x count] */
    double* wt = (double*)malloc(sizeof(double) * (size_t)(N * count > 0 ? N * count : 1));
    for (int64_t n = 0; n < N; ++n) {
        for (int32_t h = 0; h < count; ++h) {
            int64_t k = idx[h];
            if (W16) {
                wt[n * count + h] = orc_f16_to_f64(W16[n * K + k]);
            } else {
                float p = s_w[n] * (float)Wq[n * K + k];
                wt[n * count + h] = orc_f16_to_f64(orc_f64_to_f16((double)p));
            }
        }
    }

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t ri = 0; ri < nrows; ++ri) {
        int64_t m = rows ? rows[ri] : ri;
        int8_t* xq = (int8_t*)malloc((size_t)K);
        float s_x = 0.0f;
        orc_quant_rows_f16(X + m * K, 1, K, K, mask, -127, 127, NULL, NULL, xq, &s_x);
        for (int64_t n = 0; n < N; ++n) {
            const int8_t* w = Wq + n * K;
            int64_t c = 0;
            for (int64_t k = 0; k < K; ++k)
                c += (int64_t)xq[k] * (int64_t)w[k];
            double normal = (double)c * (double)s_x * (double)s_w[n];
            double outl = 0.0;
            for (int32_t h = 0; h < count; ++h)
                outl += orc_f16_to_f64(X[m * K + idx[h]]) * wt[n * count + h];
            out[ri * N + n] = outl + normal;
        }
        free(xq);
    }
    free(wt);
}

/* ---------------------------------------------------------------------------
 * Kronecker affine transform  [FlatQuant]
 * ------------------------------------------------------------------------- */

void orc_pack_int4(const int8_t* q, int64_t rows, int64_t K, uint32_t* packed);
void orc_unpack_int4(const uint32_t* packed, int64_t rows, int64_t K, int8_t* q);

/* (n1, n2) minimizing n1 + n2 over n1 n2 = n, n1 <= n2. */
void orc_kron_sizes(int64_t n, int64_t* n1, int64_t* n2)
{
    int64_t b1 = 1, b2 = n;
    for (int64_t a = 1; a * a <= n; ++a) {
        if (n % a != 0)
            continue;
        if (a + n / a < b1 + b2) {
            b1 = a;
            b2 = n / a;
        }
    }
    *n1 = b1;
    *n2 = b2;
}

/* out[r] = reshape( P1^T X~_r P2 ), X~_r = x[r] as [n1 x n2] row-major.
 * P1 [n1 x n1], P2 [n2 x n2] row-major.  Mode 1 first:
 *   Y[a][j]  = sum_i P1[i][a] X~[i][j]     (fmaf chain, i ascending)
 *   X'[a][b] = sum_j Y[a][j] P2[j][b]      (fmaf chain, j ascending) */
void orc_kron_transform_f32(const float* x, int64_t rows, int64_t n1, int64_t n2, const float* P1,
                            const float* P2, float* out)
{
    int64_t n = n1 * n2;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const float* xt = x + r * n;
        float* y = (float*)malloc(sizeof(float) * (size_t)(n > 0 ? n : 1));
        for (int64_t a = 0; a < n1; ++a)
            for (int64_t j = 0; j < n2; ++j) {
                float acc = 0.0f;
                for (int64_t i = 0; i < n1; ++i)
                    acc = fmaf(P1[i * n1 + a], xt[i * n2 + j], acc);
                y[a * n2 + j] = acc;
            }
        for (int64_t a = 0; a < n1; ++a)
            for (int64_t b = 0; b < n2; ++b) {
                float acc = 0.0f;
                for (int64_t j = 0; j < n2; ++j)
                    acc = fmaf(y[a * n2 + j], P2[j * n2 + b], acc);
                out[r * n + a * n2 + b] = acc;
            }
        free(y);
    }
}

/* Transform + int4 codes (one scale per gsize columns; gsize = K: per row)
 * + packing, as the Hadamard path does after its rotation. */
void orc_kron_quant_int4(const uint16_t* X, int64_t rows, int64_t K, int64_t n1, int64_t n2,
                         const float* P1, const float* P2, int64_t gsize, int32_t qmin, int32_t qmax,
                         uint32_t* packed, float* s)
{
    size_t n = (size_t)(rows * K > 0 ? rows * K : 1);
    float* xf = (float*)malloc(sizeof(float) * n);
    float* xt = (float*)malloc(sizeof(float) * n);
    int8_t* q = (int8_t*)malloc(n);
    orc_f16_to_f32_array(X, rows * K, xf);
    orc_kron_transform_f32(xf, rows, n1, n2, P1, P2, xt);
    orc_quant_rows_f32(xt, rows, K, gsize, NULL, qmin, qmax, NULL, NULL, q, s);
    orc_pack_int4(q, rows, K, packed);
    free(q);
    free(xt);
    free(xf);
}

/* W4A4 linear with the Kronecker transform of X (per-token int4 scale) and
 * the offline-transformed weight (Wp, s_w per (row, G-group)):
 * out[m][n] = s_x[m] sum_g s_w[n][g] sum_{k in g} qx[m][k] qw[n][k]. */
void orc_qlinear_kron_w4a4(const uint16_t* X, int64_t M, int64_t K, int64_t n1, int64_t n2, const float* P1,
                           const float* P2, const uint32_t* Wp, const float* s_w, int64_t N, int32_t G,
                           const int64_t* rows, int64_t nrows, double* out)
{
    if (!rows)
        nrows = M;
    int64_t ng = K / G;
    int8_t* wq = (int8_t*)malloc((size_t)(N * K > 0 ? N * K : 1));
    orc_unpack_int4(Wp, N, K, wq);
    for (int64_t ri = 0; ri < nrows; ++ri) {
        int64_t m = rows ? rows[ri] : ri;
        uint32_t* xp = (uint32_t*)malloc(sizeof(uint32_t) * (size_t)(K / 8 > 0 ? K / 8 : 1));
        int8_t* xq = (int8_t*)malloc((size_t)K);
        float s_x = 0.0f;
        orc_kron_quant_int4(X + m * K, 1, K, n1, n2, P1, P2, K, -7, 7, xp, &s_x);
        orc_unpack_int4(xp, 1, K, xq);
#pragma omp parallel for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            double sum = 0.0;
            for (int64_t g = 0; g < ng; ++g) {
                int64_t a = 0;
                for (int64_t k = g * G; k < (g + 1) * G; ++k)
                    a += (int64_t)xq[k] * (int64_t)wq[n * K + k];
                sum += (double)s_w[n * ng + g] * (double)a;
            }
            out[ri * N + n] = (double)s_x * sum;
        }
        free(xq);
        free(xp);
    }
    free(wq);
}

/* ---------------------------------------------------------------------------
 * Asymmetric (affine) quantization  [Scholia-IQ §6: q = round(x/s) + z,
 * x^ = s (q - z), z is the integer standing for real 0; §6.2: the integer
 * grid shifted onto a range such as [-0.2, 1.7], q clipped to [qmin, qmax]]
 * The pages leave the choice of s and z open; the min-max rule is taken:
 * the grid spans [lo, hi] = [min(min x, 0), max(max x, 0)], lo -> qmin.
 * ------------------------------------------------------------------------- */
void orc_minmax_params(const float* x, int64_t n, int32_t qmin, int32_t qmax, float* s_out, int32_t* z_out)
{
    float lo = 0.0f, hi = 0.0f;
    for (int64_t j = 0; j < n; ++j) {
        if (x[j] < lo) lo = x[j];
        if (x[j] > hi) hi = x[j];
    }
    float s = 1.0f;
    if (hi != lo) {
        float d = hi - lo;                                  /* fp32, correctly rounded */
        s = d / (float)(qmax - qmin);
    }
    double z = (double)qmin - (double)rintf(lo / s);
    if (z < qmin) z = qmin;
    if (z > qmax) z = qmax;
    *s_out = s;
    *z_out = (int32_t)z;
}

/* Per-row asymmetric codes of fp32 rows: (s, z) from orc_minmax_params, then
 * q = clip(rint(x/s) + z), and the row sums of the codes. */
void orc_quant_rows_asym_f32(const float* x, int64_t rows, int64_t K, int32_t qmin, int32_t qmax,
                             int8_t* q, float* s_out, int32_t* z_out, int32_t* rowsum)
{
    for (int64_t r = 0; r < rows; ++r) {
        orc_minmax_params(x + r * K, K, qmin, qmax, &s_out[r], &z_out[r]);
        orc_quant_rows_f32(x + r * K, 1, K, K, NULL, qmin, qmax, &s_out[r], &z_out[r], q + r * K, NULL);
        int64_t sum = 0;
        for (int64_t j = 0; j < K; ++j)
            sum += q[r * K + j];
        if (rowsum)
            rowsum[r] = (int32_t)sum;
    }
}

/* W8A8 linear with asymmetric per-token activations: out[m][n] =
 * sum_k s_x[m] (xq[m][k] - z_x[m]) * s_w[n] (wq[n][k] - z_w[n]), the
 * integer sum exact in int64.  z_w may be NULL (symmetric weight).
 * Activation codes in [-128, 127].  Output fp64 [nrows x N]. */
void orc_qlinear_int8_asym(const uint16_t* X, int64_t M, int64_t K, const int8_t* Wq, const float* s_w,
                           const int32_t* z_w, int64_t N, const int64_t* rows, int64_t nrows, double* out)
{
    if (!rows)
        nrows = M;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t ri = 0; ri < nrows; ++ri) {
        int64_t m = rows ? rows[ri] : ri;
        float* xf = (float*)malloc(sizeof(float) * (size_t)(K > 0 ? K : 1));
        int8_t* xq = (int8_t*)malloc((size_t)(K > 0 ? K : 1));
        float s_x;
        int32_t z_x;
        orc_f16_to_f32_array(X + m * K, K, xf);
        orc_quant_rows_asym_f32(xf, 1, K, -128, 127, xq, &s_x, &z_x, NULL);
        for (int64_t n = 0; n < N; ++n) {
            int64_t zw = z_w ? z_w[n] : 0;
            int64_t acc = 0;
            for (int64_t k = 0; k < K; ++k)
                acc += ((int64_t)xq[k] - z_x) * ((int64_t)Wq[n * K + k] - zw);
            out[ri * N + n] = (double)acc * (double)s_x * (double)s_w[n];
        }
        free(xq);
        free(xf);
    }
}

/* ---------------------------------------------------------------------------
 * SmoothQuant  [QE2 §4.2]
 * Equivalent per-input-channel scaling: column j of X is divided by s_j and
 * column j of the weight (row j of the page's W, column j of our [N x K]
 * layout) is multiplied by s_j, so X W^T is unchanged in exact arithmetic.
 * ------------------------------------------------------------------------- */

/* colmax[j] = max_r |a[r][j]| (0 when rows == 0). */
void orc_col_absmax_f32(const float* a, int64_t rows, int64_t K, float* colmax)
{
    for (int64_t j = 0; j < K; ++j)
        colmax[j] = 0.0f;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t j = 0; j < K; ++j) {
            float v = fabsf(a[r * K + j]);
            if (v > colmax[j])
                colmax[j] = v;
        }
}

/* s_j = cx_j^alpha / cw_j^(1-alpha); 1 when either maximum is 0. */
void orc_smooth_factors(const float* cx, const float* cw, int64_t K, double alpha, float* s)
{
    for (int64_t j = 0; j < K; ++j) {
        if (cx[j] == 0.0f || cw[j] == 0.0f) {
            s[j] = 1.0f;
            continue;
        }
        double num = pow((double)cx[j], alpha);
        double den = pow((double)cw[j], 1.0 - alpha);
        s[j] = (float)(num / den);
    }
}

/* out = a / s (op 0, activations) or a * s (op 1, weights), per column. */
void orc_smooth_apply_f32(const float* a, int64_t rows, int64_t K, const float* s, int op, float* out)
{
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t j = 0; j < K; ++j) {
            float v = a[r * K + j];
            out[r * K + j] = op == 0 ? v / s[j] : v * s[j];
        }
}

/* Smoothing followed by symmetric [-127, 127] absmax quantization with one
 * scale per row (per_tensor == 0) or one scale for the whole matrix, written
 * to every s_out[r] (per_tensor != 0). */
void orc_smooth_quant_f32(const float* a, int64_t rows, int64_t K, const float* s, int op, int per_tensor,
                          int8_t* q, float* s_out)
{
    size_t n = (size_t)(rows * K > 0 ? rows * K : 1);
    float* h = (float*)malloc(sizeof(float) * n);
    orc_smooth_apply_f32(a, rows, K, s, op, h);
    if (!per_tensor) {
        orc_quant_rows_f32(h, rows, K, K, NULL, -127, 127, NULL, NULL, q, s_out);
    } else {
        float m = 0.0f;
        for (int64_t i = 0; i < rows * K; ++i)
            if (fabsf(h[i]) > m)
                m = fabsf(h[i]);
        float st = (m == 0.0f) ? 1.0f : m / 127.0f;
        for (int64_t r = 0; r < rows; ++r)
            s_out[r] = st;
        orc_quant_rows_f32(h, rows, K, K, NULL, -127, 127, s_out, NULL, q, NULL);
    }
    free(h);
}

/* SmoothQuant W8A8 linear: Xs = X / s, activation codes and scales from
 * orc_smooth_quant_f32, C = Xq Wq^T (int32), out = C * s_x[m] * s_w[n].
 * Wq, s_w come from the smoothed weight (op 1).  Output fp64 [nrows x N]. */
void orc_qlinear_int8_smooth(const uint16_t* X, int64_t M, int64_t K, const float* s, int per_tensor,
                             const int8_t* Wq, const float* s_w, int64_t N, const int64_t* rows, int64_t nrows,
                             double* out)
{
    if (!rows)
        nrows = M;
    size_t n = (size_t)(M * K > 0 ? M * K : 1);
    float* xf = (float*)malloc(sizeof(float) * n);
    int8_t* xq = (int8_t*)malloc(n);
    float* s_x = (float*)malloc(sizeof(float) * (size_t)(M > 0 ? M : 1));
    orc_f16_to_f32_array(X, M * K, xf);
    orc_smooth_quant_f32(xf, M, K, s, 0, per_tensor, xq, s_x);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t ri = 0; ri < nrows; ++ri) {
        int64_t m = rows ? rows[ri] : ri;
        for (int64_t nn = 0; nn < N; ++nn) {
            int64_t c = 0;
            for (int64_t k = 0; k < K; ++k)
                c += (int64_t)xq[m * K + k] * (int64_t)Wq[nn * K + k];
            out[ri * N + nn] = (double)c * (double)s_x[m] * (double)s_w[nn];
        }
    }
    free(s_x);
    free(xq);
    free(xf);
}

/* ---------------------------------------------------------------------------
 * Normalized block Hadamard  [GroupRot §二, §5.1, §5.2]
 * out[r, b*G + j] = fl32( fl64(1/sqrt(G)) * sum_i x[r, b*G + i] * H_G[i][j] )
 * with H_G[i][j] = (-1)^popcount(i & j).  The sum is exact in fp64: fp16
 * values are multiples of 2^-24 below 2^16, so |sum| < G * 2^16 needs at most
 * 40 + log2(G) bits.
 * ------------------------------------------------------------------------- */
static int orc_parity(uint32_t v)
{
    int p = 0;
    while (v) {
        p ^= (int)(v & 1u);
        v >>= 1;
    }
    return p;
}

int orc_hadamard_entry(int32_t i, int32_t j) { return orc_parity((uint32_t)(i & j)) ? -1 : 1; }

void orc_hadamard_rows(const uint16_t* X, int64_t rows, int64_t K, int32_t G, float* out)
{
    const double c = 1.0 / sqrt((double)G);
    int64_t nb = K / G;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double* xb = (double*)malloc(sizeof(double) * (size_t)G);
        for (int64_t b = 0; b < nb; ++b) {
            for (int32_t i = 0; i < G; ++i)
                xb[i] = orc_f16_to_f64(X[r * K + b * G + i]);
            for (int32_t j = 0; j < G; ++j) {
                double y = 0.0;
                for (int32_t i = 0; i < G; ++i)
                    y += orc_hadamard_entry(i, j) > 0 ? xb[i] : -xb[i];
                out[r * K + b * G + j] = (float)(y * c);
            }
        }
        free(xb);
    }
}

/* ---------------------------------------------------------------------------
 * int4 packing  [GroupRot §5.4: eight 4-bit integers per 32-bit word]
 * ------------------------------------------------------------------------- */
void orc_pack_int4(const int8_t* q, int64_t rows, int64_t K, uint32_t* packed)
{
    int64_t words = K / 8;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t w = 0; w < words; ++w) {
            uint32_t v = 0;
            for (int i = 0; i < 8; ++i)
                v |= ((uint32_t)(uint8_t)q[r * K + 8 * w + i] & 0xFu) << (4 * i);
            packed[r * words + w] = v;
        }
}

void orc_unpack_int4(const uint32_t* packed, int64_t rows, int64_t K, int8_t* q)
{
    int64_t words = K / 8;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t w = 0; w < words; ++w) {
            uint32_t v = packed[r * words + w];
            for (int i = 0; i < 8; ++i) {
                int nib = (int)((v >> (4 * i)) & 0xFu);
                q[r * K + 8 * w + i] = (int8_t)(nib >= 8 ? nib - 16 : nib);
            }
        }
}

/* Rotate, quantize (per row: mode 0, per G-block: mode 1) and pack.
 * [GroupRot §5.1 (weights, offline), §5.2 (activations, dynamic)] */
void orc_hadamard_quant_int4(const uint16_t* X, int64_t rows, int64_t K, int32_t G, int mode,
                             int32_t qmin, int32_t qmax, uint32_t* packed, float* s)
{
    size_t n = (size_t)(rows * K > 0 ? rows * K : 1);
    float* xr = (float*)malloc(sizeof(float) * n);
    int8_t* q = (int8_t*)malloc(n);
    orc_hadamard_rows(X, rows, K, G, xr);
    orc_quant_rows_f32(xr, rows, K, mode ? G : K, NULL, qmin, qmax, NULL, NULL, q, s);
    orc_pack_int4(q, rows, K, packed);
    free(q);
    free(xr);
}

/* ---------------------------------------------------------------------------
 * W4A4 per-group int32 accumulators  [GroupRot §5.4]
 * acc[ri][n][g] = sum_{k in group g} qx[m][k] * qw[n][k], m = rows[ri].
 * Returns the count of results outside int32.
 * ------------------------------------------------------------------------- */
int64_t orc_w4a4_group_acc(const uint32_t* Xp, const uint32_t* Wp, int64_t M, int64_t K,
                           int64_t N, int32_t G, const int64_t* rows, int64_t nrows,
                           int32_t* acc)
{
    if (!rows)
        nrows = M;
    int64_t ng = K / G, bad = 0;
    int8_t* wq = (int8_t*)malloc((size_t)(N * K > 0 ? N * K : 1));
    orc_unpack_int4(Wp, N, K, wq);
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : bad)
    for (int64_t ri = 0; ri < nrows; ++ri) {
        int64_t m = rows ? rows[ri] : ri;
        int8_t* xq = (int8_t*)malloc((size_t)K);
        orc_unpack_int4(Xp + m * (K / 8), 1, K, xq);
        for (int64_t n = 0; n < N; ++n)
            for (int64_t g = 0; g < ng; ++g) {
                int64_t a = 0;
                for (int64_t k = g * G; k < (g + 1) * G; ++k)
                    a += (int64_t)xq[k] * (int64_t)wq[n * K + k];
                if (a > INT32_MAX || a < INT32_MIN)
                    ++bad;
                acc[(ri * N + n) * ng + g] = (int32_t)a;
            }
        free(xq);
    }
    free(wq);
    return bad;
}

/* ---------------------------------------------------------------------------
 * W4A4 group-Hadamard linear  [GroupRot §5.2, §5.4]
 *   X' = X * blockdiag(H_G); s_x = absmax(row of X')/7; codes in [-7, 7];
 *   out[m][n] = s_x[m] * sum_g s_w[n][g] * acc_g   (fp64), acc_g as above.
 * Wp / s_w are the offline weights (orc_hadamard_quant_int4, mode 1).
 * ------------------------------------------------------------------------- */
void orc_qlinear_w4a4(const uint16_t* X, int64_t M, int64_t K, const uint32_t* Wp,
                      const float* s_w, int64_t N, int32_t G, const int64_t* rows,
                      int64_t nrows, double* out)
{
    if (!rows)
        nrows = M;
    int64_t ng = K / G;
    int8_t* wq = (int8_t*)malloc((size_t)(N * K > 0 ? N * K : 1));
    orc_unpack_int4(Wp, N, K, wq);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t ri = 0; ri < nrows; ++ri) {
        int64_t m = rows ? rows[ri] : ri;
        uint32_t* xp = (uint32_t*)malloc(sizeof(uint32_t) * (size_t)(K / 8 > 0 ? K / 8 : 1));
        int8_t* xq = (int8_t*)malloc((size_t)K);
        float s_x = 0.0f;
        orc_hadamard_quant_int4(X + m * K, 1, K, G, 0, -7, 7, xp, &s_x);
        orc_unpack_int4(xp, 1, K, xq);
        for (int64_t n = 0; n < N; ++n) {
            double sum = 0.0;
            for (int64_t g = 0; g < ng; ++g) {
                int64_t a = 0;
                for (int64_t k = g * G; k < (g + 1) * G; ++k)
                    a += (int64_t)xq[k] * (int64_t)wq[n * K + k];
                sum += (double)s_w[n * ng + g] * (double)a;
            }
            out[ri * N + n] = (double)s_x * sum;
        }
        free(xq);
        free(xp);
    }
    free(wq);
}

/* ---------------------------------------------------------------------------
 * W4A8: 4-bit weights, 8-bit activations  [Scholia-IQ §2.1-§2.2; FlatQuant
 * §4 (the W4A4 transform reused for W4A8); GroupRot §5.2 (online rotation
 * fused with dynamic per-token quantization), §5.4 (int32 accumulation)]
 *   X' = X * blockdiag(H_G) (as for W4A4); s_x = fl32(absmax(row of X')/127);
 *   int8 codes in [-127, 127]; the weight is the offline W4A4 weight (per-group
 *   int4 of W * blockdiag(H_G));
 *   out[m][n] = s_x[m] * sum_g s_w[n][g] * acc_g   (fp64), acc_g the exact
 *   integer sum of the group's products.
 * ------------------------------------------------------------------------- */
void orc_hadamard_quant_int8(const uint16_t* X, int64_t rows, int64_t K, int32_t G,
                             int32_t qmin, int32_t qmax, int8_t* q, float* s)
{
    size_t n = (size_t)(rows * K > 0 ? rows * K : 1);
    float* xr = (float*)malloc(sizeof(float) * n);
    orc_hadamard_rows(X, rows, K, G, xr);
    orc_quant_rows_f32(xr, rows, K, K, NULL, qmin, qmax, NULL, NULL, q, s);
    free(xr);
}

/* acc[ri][n][g] = sum_{k in group g} Xq[m][k] * qw[n][k], m = rows[ri].
 * Returns the count of results outside int32. */
int64_t orc_w4a8_group_acc(const int8_t* Xq, const uint32_t* Wp, int64_t M, int64_t K,
                           int64_t N, int32_t G, const int64_t* rows, int64_t nrows,
                           int32_t* acc)
{
    if (!rows)
        nrows = M;
    int64_t ng = K / G, bad = 0;
    int8_t* wq = (int8_t*)malloc((size_t)(N * K > 0 ? N * K : 1));
    orc_unpack_int4(Wp, N, K, wq);
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : bad)
    for (int64_t ri = 0; ri < nrows; ++ri) {
        int64_t m = rows ? rows[ri] : ri;
        const int8_t* xq = Xq + m * K;
        for (int64_t n = 0; n < N; ++n)
            for (int64_t g = 0; g < ng; ++g) {
                int64_t a = 0;
                for (int64_t k = g * G; k < (g + 1) * G; ++k)
                    a += (int64_t)xq[k] * (int64_t)wq[n * K + k];
                if (a > INT32_MAX || a < INT32_MIN)
                    ++bad;
                acc[(ri * N + n) * ng + g] = (int32_t)a;
            }
    }
    free(wq);
    return bad;
}

void orc_qlinear_w4a8(const uint16_t* X, int64_t M, int64_t K, const uint32_t* Wp,
                      const float* s_w, int64_t N, int32_t G, const int64_t* rows,
                      int64_t nrows, double* out)
{
    if (!rows)
        nrows = M;
    int64_t ng = K / G;
    int8_t* wq = (int8_t*)malloc((size_t)(N * K > 0 ? N * K : 1));
    orc_unpack_int4(Wp, N, K, wq);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t ri = 0; ri < nrows; ++ri) {
        int64_t m = rows ? rows[ri] : ri;
        int8_t* xq = (int8_t*)malloc((size_t)(K > 0 ? K : 1));
        float s_x = 0.0f;
        orc_hadamard_quant_int8(X + m * K, 1, K, G, -127, 127, xq, &s_x);
        for (int64_t n = 0; n < N; ++n) {
            double sum = 0.0;
            for (int64_t g = 0; g < ng; ++g) {
                int64_t a = 0;
                for (int64_t k = g * G; k < (g + 1) * G; ++k)
                    a += (int64_t)xq[k] * (int64_t)wq[n * K + k];
                sum += (double)s_w[n * ng + g] * (double)a;
            }
            out[ri * N + n] = (double)s_x * sum;
        }
        free(xq);
    }
    free(wq);
}

/* ---------------------------------------------------------------------------
 * W4A4 with zero-point activations  [Scholia-IQ §6 (q = round(x/s) + z,
 * x^ = s (q - z)), §6.2 (the grid shifted onto the data's range, clip to
 * [q_min, q_max]), §7.3; GroupRot §5.2, §5.4]
 *   X' = X * blockdiag(H_G) (as for W4A4); per row (s, z) by the min-max rule
 *   over [0, 15]; q = clip(rint(fl32(x'/s)) + z, 0, 15);
 *   the weight is the W4A4 weight (symmetric int4 per G-group);
 *   out[m][n] = s_x[m] * sum_g s_w[n][g] * sum_{k in g} (q[m][k] - z[m]) qw[n][k]
 *   (integer sums exact, fp64).
 * Packed activation codes: nibble = (q - 8) mod 16, i.e. the two's complement
 * nibble of q - 8 (the packing of the symmetric codes); z is returned in
 * [0, 15].
 * ------------------------------------------------------------------------- */
void orc_hadamard_quant_int4_asym(const uint16_t* X, int64_t rows, int64_t K, int32_t G,
                                  uint32_t* packed, float* s, int32_t* z)
{
    size_t n = (size_t)(rows * K > 0 ? rows * K : 1);
    float* xr = (float*)malloc(sizeof(float) * n);
    int8_t* q = (int8_t*)malloc(n);
    orc_hadamard_rows(X, rows, K, G, xr);
    orc_quant_rows_asym_f32(xr, rows, K, 0, 15, q, s, z, NULL);
    for (size_t i = 0; i < (size_t)(rows * K); ++i)
        q[i] = (int8_t)(q[i] - 8);
    orc_pack_int4(q, rows, K, packed);
    free(q);
    free(xr);
}

/* Column term of the zero-point linear  [Scholia-IQ §6: dequantization
 * s (q - z), so sum_k (q - z) w splits into sum_k q w - z sum_k w;
 * GroupRot §5.4: per-group weight scales]
 *   c[n] = fl32( sum_g s_w[n][g] * sum_{k in g} qw[n][k] )
 * the group sums exact (int64), the sum over the groups in fp64 with g
 * ascending, rounded once to fp32.
 * ------------------------------------------------------------------------- */
void orc_w4_column_terms(const uint32_t* Wp, const float* s_w, int64_t N, int64_t K, int32_t G, float* c)
{
    int64_t ng = K / G;
    int8_t* wq = (int8_t*)malloc((size_t)(N * K > 0 ? N * K : 1));
    orc_unpack_int4(Wp, N, K, wq);
    for (int64_t n = 0; n < N; ++n) {
        double sum = 0.0;
        for (int64_t g = 0; g < ng; ++g) {
            int64_t a = 0;
            for (int64_t k = g * G; k < (g + 1) * G; ++k)
                a += (int64_t)wq[n * K + k];
            sum += (double)s_w[n * ng + g] * (double)a;
        }
        c[n] = (float)sum;
    }
    free(wq);
}

void orc_qlinear_w4a4_asym(const uint16_t* X, int64_t M, int64_t K, const uint32_t* Wp,
                           const float* s_w, int64_t N, int32_t G, const int64_t* rows,
                           int64_t nrows, double* out)
{
    if (!rows)
        nrows = M;
    int64_t ng = K / G;
    int8_t* wq = (int8_t*)malloc((size_t)(N * K > 0 ? N * K : 1));
    orc_unpack_int4(Wp, N, K, wq);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t ri = 0; ri < nrows; ++ri) {
        int64_t m = rows ? rows[ri] : ri;
        uint32_t* xp = (uint32_t*)malloc(sizeof(uint32_t) * (size_t)(K / 8 > 0 ? K / 8 : 1));
        int8_t* xq = (int8_t*)malloc((size_t)K);
        float s_x = 0.0f;
        int32_t z_x = 0;
        orc_hadamard_quant_int4_asym(X + m * K, 1, K, G, xp, &s_x, &z_x);
        orc_unpack_int4(xp, 1, K, xq);           /* q - 8 */
        for (int64_t n = 0; n < N; ++n) {
            double sum = 0.0;
            for (int64_t g = 0; g < ng; ++g) {
                int64_t a = 0;
                for (int64_t k = g * G; k < (g + 1) * G; ++k)
                    a += ((int64_t)xq[k] + 8 - z_x) * (int64_t)wq[n * K + k];
                sum += (double)s_w[n * ng + g] * (double)a;
            }
            out[ri * N + n] = (double)s_x * sum;
        }
        free(xq);
        free(xp);
    }
    free(wq);
}
