// qa_launch.hpp -- host-side launchers of the gfx950 kernels (internal).
// Arguments are validated by the C ABI layer (qa_api.cpp) before any call.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "qa.h"

namespace qa {

// Shared by the C entry points (qa_api.cpp): record an error message for
// qa_last_error() and return s; check every argument of an LLM.int8() call
// (no HIP call; *empty is set for M == 0 or N == 0, a valid no-op); enqueue
// the call's kernels on a workspace of at least qa_qlinear_int8_mixed_workspace
// bytes.
qa_status record_error(qa_status s, const char* fmt, ...);
qa_status mixed_validate(const char* fn, const void* X_f16, int64_t M, int64_t K, const int8_t* Wq,
                         const float* s_w, const void* W_f16_or_null, int64_t N, float threshold, const void* out,
                         qa_dtype out_dtype, bool with_workspace, const void* workspace, size_t workspace_bytes,
                         bool* empty);
qa_status mixed_run(const char* fn, const void* X_f16, int64_t M, int64_t K, const int8_t* Wq, const float* s_w,
                    const void* W_f16_or_null, int64_t N, float threshold, void* out, qa_dtype out_dtype,
                    void* workspace, void* stream);

// Scratch of the outlier-column scan: up to 32 row segments' partial flag
// words (one 64-bit word per 64 columns) and partial column maxima [K], all
// overwritten by every scan (no clearing).
size_t outlier_scratch_bytes(int64_t K);

// Public outlier detection: scan + one-block finalize (mask, list, count, max).
hipError_t launch_outlier_cols(const uint16_t* X, int64_t M, int64_t K, float tau, uint8_t* mask,
                               int32_t* idx, int32_t* count, float* colmax, void* scratch, hipStream_t st);

// Outlier flag words only (for the mixed linear, which consumes them in the
// row quantizer); *segs receives the number of partial flag sets written.
hipError_t launch_outlier_flags(const uint16_t* X, int64_t M, int64_t K, float tau, void* scratch, int* segs,
                                hipStream_t st);

hipError_t launch_rowquant_i8(const uint16_t* X, int64_t rows, int64_t K, const uint8_t* mask,
                              int qmin, int qmax, const float* s_in, const int32_t* z_in,
                              int8_t* q, float* s_out, hipStream_t st);

// Width of the compact outlier rows: xo[m][r] holds X[m][idx[r]] (fp16) for
// the first XO_CAP outlier columns, written by the flag-masked row
// quantizer and read by the GEMM epilogue with contiguous loads.
constexpr int XO_CAP = 256;
// Up to this many outlier columns the GEMM configurations with registers to
// spare gather X and w~ themselves (issued behind their first pipeline
// stages); the compact rows (written for every nonzero count) serve larger
// counts and the register-bound wide configuration.
constexpr int OUTLIER_PREFETCH = 8;

// Dynamic [-127, 127] row quantization with the outlier flags of `scratch`
// (launch_outlier_flags, nseg partial sets) as the mask; also writes the
// ascending outlier list and its count, and the compact outlier rows xo
// [rows x XO_CAP] when rowquant_writes_xo(K) (entries past the count are
// left as they were).
bool rowquant_writes_xo(int64_t K);
hipError_t launch_rowquant_i8_flags(const uint16_t* X, int64_t rows, int64_t K, const void* scratch, int nseg,
                                    int8_t* q, float* s_out, int32_t* idx, int32_t* count, uint16_t* xo,
                                    hipStream_t st);

// Dynamic [-127, 127] row quantization with no outlier columns; *count = 0.
hipError_t launch_rowquant_i8_no_outliers(const uint16_t* X, int64_t rows, int64_t K, int8_t* q, float* s_out,
                                          int32_t* count, hipStream_t st);

// Top-k decomposition: the k columns with the largest column maximum (ties
// to the lower column) as the outlier set.  K <= topk_max_columns().
int64_t topk_max_columns();
hipError_t launch_outlier_topk(const uint16_t* X, int64_t M, int64_t K, int64_t k, uint8_t* mask, int32_t* idx,
                               int32_t* count, float* colmax, void* scratch, hipStream_t st);
// Flag words only (consumed by launch_rowquant_i8_flags with *segs sets).
hipError_t launch_outlier_topk_flags(const uint16_t* X, int64_t M, int64_t K, int64_t k, void* scratch, int* segs,
                                     hipStream_t st);

// Column absolute maxima of A [rows x K] (maxed into colmax when accumulating);
// scratch as for the outlier scan.
hipError_t launch_col_absmax(const uint16_t* A, int64_t rows, int64_t K, float* colmax, bool accumulate,
                             void* scratch, hipStream_t st);

// SmoothQuant migration factors and the smoothing fused with [-127, 127]
// absmax quantization (per row, or per tensor broadcast into s_out[rows]);
// a non-null count is set to 0 for the GEMM epilogue.
hipError_t launch_smooth_factors(const float* cx, const float* cw, int64_t K, float alpha, float* s, hipStream_t st);
hipError_t launch_smoothquant_i8(const uint16_t* X, int64_t rows, int64_t K, const float* sm, bool multiply,
                                 bool per_tensor, int8_t* q, float* s_out, int32_t* count, hipStream_t st);

// Kronecker transform X' = P1^T X~ P2 of each row (n1 n2 = K) fused with int4
// codes: per row (G == 0) or per G-wide group; kron_supported(n1, n2, G)
// tells which sizes have a kernel.
bool kron_supported(int64_t n1, int64_t n2, int G);
hipError_t launch_kron_quant_i4(const uint16_t* X, int64_t rows, int64_t n1, int64_t n2, const float* P1,
                                const float* P2, int G, int qmin, int qmax, uint32_t* packed, float* s,
                                hipStream_t st);

hipError_t launch_hadamard_quant_i4(const uint16_t* X, int64_t rows, int64_t K, int G,
                                    bool per_group, int qmin, int qmax, uint32_t* packed, float* s,
                                    hipStream_t st);
hipError_t launch_hadamard_quant_i8(const uint16_t* X, int64_t rows, int64_t K, int G, int qmin, int qmax,
                                    int8_t* q, float* s, hipStream_t st);
hipError_t launch_hadamard_quant_i4_asym(const uint16_t* X, int64_t rows, int64_t K, int G, uint32_t* packed,
                                         float* s, int32_t* z, hipStream_t st);
// Per output channel of a per-group int4 weight: c[n] = fl32(sum_g s_w[n][g] *
// sum_{k in g} qw[n][k]), the sum in fp64 over g ascending.
hipError_t launch_w4_column_terms(const uint32_t* Wp, const float* s_w, int64_t N, int64_t K, int G, float* c,
                                  hipStream_t st);

// int8 GEMM C = A * B^T (A [M x K], B [N x K]) with either an int32 store
// (out_dtype < 0) or the LLM.int8() epilogue.
struct MixedEpilogue {
    const float* s_x;          // [M]
    const float* s_w;          // [N]
    const uint16_t* X;         // fp16 [M x K] (outlier gather)
    const uint16_t* W16;       // fp16 [N x K] or nullptr
    const int8_t* Wq;          // for w~ when W16 is null
    const int32_t* idx;        // outlier list
    const int32_t* count;      // device count
    const uint16_t* Xo;        // compact outlier rows [M x XO_CAP] or nullptr (then X is gathered)
    void* out;
    int64_t ldo;               // row stride of out, in elements
    int out_dtype;             // 0 f32, 1 f16, 2 bf16
};

hipError_t launch_gemm_i8_i32(const int8_t* A, const int8_t* B, int64_t M, int64_t K, int64_t N,
                              int32_t* C, hipStream_t st);

// Zero-point dequantization of the int8 GEMM (see k_gemm_i8_asym).
struct AsymEpilogue {
    const float* s_x;          // [M]
    const int32_t* z_x;        // [M]
    const int32_t* r_x;        // [M] row sums of Xq (read only with z_w)
    const float* s_w;          // [N]
    const int32_t* z_w;        // [N] or nullptr (symmetric weight)
    const int32_t* r_w;        // [N] row sums of Wq
    void* out;
    int64_t ldo;
    int out_dtype;
};
hipError_t launch_gemm_i8_asym(const int8_t* Xq, const int8_t* Wq, int64_t M, int64_t K, int64_t N,
                               const AsymEpilogue& ep, hipStream_t st);

// Per-row asymmetric (min-max) int8 quantization with the row sums of the
// codes; and plain row sums of int8 rows.
hipError_t launch_rowquant_i8_asym(const uint16_t* X, int64_t rows, int64_t K, int qmin, int qmax, int8_t* q,
                                   float* s_out, int32_t* z_out, int32_t* rowsum, hipStream_t st);
hipError_t launch_row_sums_i8(const int8_t* A, int64_t rows, int64_t K, int32_t* sums, hipStream_t st);

hipError_t launch_gemm_i8_mixed(const int8_t* Xq, const int8_t* Wq, int64_t M, int64_t K, int64_t N,
                                const MixedEpilogue& ep, hipStream_t st);

// Fused single-kernel LLM.int8() linear for decode shapes.  Its first
// workgroup also stores the integer stages it computed (outlier list and
// count, per-token scales, codes [M x K]) at these workspace addresses.
struct DecodeStages {
    int32_t* idx;
    int32_t* count;
    float* s_x;
    int8_t* xq;
};
bool decode_supported(int64_t M, int64_t K);
// Measurement helper: `bytes` of src read by `wgs` workgroups of 512 threads,
// lane_bytes (4, 8, 16) per lane and load, `unroll` (1, 2, 4, 8) loads in flight.
hipError_t launch_stream_read(const uint8_t* src, uint64_t bytes, int wgs, int lane_bytes, int unroll, uint32_t* sink,
                              hipStream_t st);

hipError_t launch_decode_mixed(const uint16_t* X, int64_t M, int64_t K, const int8_t* Wq, const float* s_w,
                               const uint16_t* W16, int64_t N, float tau, void* out, int out_dtype,
                               const DecodeStages& stages, hipStream_t st);
// The same with the outlier set = the k columns of largest column maximum
// (ties: lower column first); needs decode_supported(M, K) and
// 0 <= k <= min(K, decode_topk_max()).
int64_t decode_topk_max();
hipError_t launch_decode_topk(const uint16_t* X, int64_t M, int64_t K, int64_t k, const int8_t* Wq, const float* s_w,
                              const uint16_t* W16, int64_t N, void* out, int out_dtype, const DecodeStages& stages,
                              hipStream_t st);
// The SmoothQuant linear for decode shapes in the same single kernel: X / sm by
// column (IEEE fp32 division), per-token or (per_tensor) one scale, int8 codes,
// the product with the offline-smoothed weight; no outlier columns.  Needs
// decode_smooth_supported(M, K) (M <= 8 at K <= 4096, M <= 4 at K <= 8192,
// K % 256 == 0).
bool decode_smooth_supported(int64_t M, int64_t K);
hipError_t launch_decode_smooth(const uint16_t* X, int64_t M, int64_t K, const float* sm, bool per_tensor,
                                const int8_t* Wq, const float* s_w, int64_t N, void* out, int out_dtype,
                                const DecodeStages& stages, hipStream_t st);

hipError_t launch_gemm_w4a4(const uint32_t* Xp, const float* s_x, const uint32_t* Wp,
                            const float* s_w, int64_t M, int64_t K, int64_t N, int G, void* out,
                            int out_dtype, hipStream_t st);

hipError_t launch_gemm_w4a4_group_acc(const uint32_t* Xp, const uint32_t* Wp, int64_t M, int64_t K,
                                      int64_t N, int G, int32_t* acc, hipStream_t st);

hipError_t launch_gemm_w4a8(const int8_t* Xq, const float* s_x, const uint32_t* Wp, const float* s_w, int64_t M,
                            int64_t K, int64_t N, int G, void* out, int out_dtype, hipStream_t st);
// W4A4 with zero-point activations: Xp holds q - 8 and z_x (in [0, 15]) the
// zero-points; out = s_x[m] (sum_g s_w[n][g] acc_g - (z_x[m] - 8) c_w[n]).
hipError_t launch_gemm_w4a4_asym(const uint32_t* Xp, const float* s_x, const int32_t* z_x, const uint32_t* Wp,
                                 const float* s_w, const float* c_w, int64_t M, int64_t K, int64_t N, int G,
                                 void* out, int out_dtype, hipStream_t st);
hipError_t launch_gemm_w4a8_group_acc(const int8_t* Xq, const uint32_t* Wp, int64_t M, int64_t K, int64_t N, int G,
                                      int32_t* acc, hipStream_t st);

}  // namespace qa
