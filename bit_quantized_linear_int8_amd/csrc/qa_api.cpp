// qa_api.cpp -- the C ABI of libqa (declared in include/qa.h).
//
// Every entry point validates all of its arguments before it touches the HIP
// runtime; on error it launches nothing and records a message readable with
// qa_last_error().  Then it carves the caller's workspace and enqueues the
// kernels on the caller's stream.  Nothing here allocates or synchronizes.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>

#include "qa.h"
#include "qa_launch.hpp"

namespace {

thread_local char g_last_error[512] = "";

qa_status fail(qa_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return s;
}

qa_status ok() {
    g_last_error[0] = '\0';
    return QA_OK;
}

qa_status device_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(QA_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr size_t kAlign = 256;
size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Largest K for which |sum_k q_x q_w| < 2^31 with codes in [-127, 127].
constexpr int64_t kMaxK_i8 = 131072;

// Row quantizers address a row with 32-bit byte offsets (16 bytes of fp16
// and 32 bytes of factors per 8 columns).
constexpr int64_t kMaxK_quant = (int64_t)1 << 26;

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

struct MixedLayout {
    size_t cmax, idx, count, s_x, xq, xo, total;
};

MixedLayout mixed_layout(int64_t M, int64_t K) {
    MixedLayout L;
    size_t off = 0;
    L.cmax = off; off += up(qa::outlier_scratch_bytes(K));
    L.idx = off; off += up((size_t)K * 4);
    L.count = off; off += up(4);
    L.s_x = off; off += up((size_t)M * 4);
    L.xq = off; off += up((size_t)M * (size_t)K);
    L.xo = off; off += up((size_t)M * qa::XO_CAP * 2);
    L.total = off;
    return L;
}

struct SmoothLayout {
    size_t count, s_x, xq, total;
};

SmoothLayout smooth_layout(int64_t M, int64_t K) {
    SmoothLayout L;
    size_t off = 0;
    L.count = off; off += up(4);
    L.s_x = off; off += up((size_t)M * 4);
    L.xq = off; off += up((size_t)M * (size_t)K);
    L.total = off;
    return L;
}

struct AsymLayout {
    size_t s_x, z_x, r_x, xq, total;
};

AsymLayout asym_layout(int64_t M, int64_t K) {
    AsymLayout L;
    size_t off = 0;
    L.s_x = off; off += up((size_t)M * 4);
    L.z_x = off; off += up((size_t)M * 4);
    L.r_x = off; off += up((size_t)M * 4);
    L.xq = off; off += up((size_t)M * (size_t)K);
    L.total = off;
    return L;
}

// K bound of the zero-point linear: sum_k (xq - z_x)(wq - z_w) has |.| <= 255^2 K
// and is evaluated in int32.
constexpr int64_t kMaxK_asym = 32768;

struct W4Layout {
    size_t xp, s_x, total;
};

W4Layout w4_layout(int64_t M, int64_t K) {
    W4Layout L;
    size_t off = 0;
    L.xp = off; off += up((size_t)M * (size_t)(K / 2));
    L.s_x = off; off += up((size_t)M * 4);
    L.total = off;
    return L;
}

W4Layout w4a8_layout(int64_t M, int64_t K) {
    W4Layout L;
    size_t off = 0;
    L.xp = off; off += up((size_t)M * (size_t)K);
    L.s_x = off; off += up((size_t)M * 4);
    L.total = off;
    return L;
}

struct W4zLayout {
    size_t xp, s_x, z_x, total;
};

W4zLayout w4z_layout(int64_t M, int64_t K) {
    W4zLayout L;
    size_t off = 0;
    L.xp = off; off += up((size_t)M * (size_t)(K / 2));
    L.s_x = off; off += up((size_t)M * 4);
    L.z_x = off; off += up((size_t)M * 4);
    L.total = off;
    return L;
}

bool valid_dtype(qa_dtype d) { return d == QA_F32 || d == QA_F16 || d == QA_BF16; }

}  // namespace

namespace qa {

qa_status record_error(qa_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return s;
}

qa_status mixed_validate(const char* fn, const void* X_f16, int64_t M, int64_t K, const int8_t* Wq,
                         const float* s_w, const void* W_f16_or_null, int64_t N, float threshold, const void* out,
                         qa_dtype out_dtype, bool with_workspace, const void* workspace, size_t workspace_bytes,
                         bool* empty) {
    *empty = false;
    if (M < 0 || N < 0 || K <= 0 || K % 16 != 0 || K > kMaxK_i8)
        return fail(QA_ERR_SHAPE, "%s: need M, N >= 0, 0 < K <= %lld, K %% 16 == 0", fn, (long long)kMaxK_i8);
    if (std::isnan(threshold)) return fail(QA_ERR_VALUE, "%s: threshold is NaN", fn);
    if (!valid_dtype(out_dtype)) return fail(QA_ERR_VALUE, "%s: bad out_dtype %d", fn, (int)out_dtype);
    if (M == 0 || N == 0) {
        *empty = true;
        return ok();
    }
    if (!X_f16 || !Wq || !s_w || !out || (with_workspace && !workspace))
        return fail(QA_ERR_NULL, "%s: NULL pointer", fn);
    if (!aligned(X_f16, 16) || !aligned(Wq, 16) || !aligned(s_w, 4) || (with_workspace && !aligned(workspace, kAlign)) ||
        (W_f16_or_null && !aligned(W_f16_or_null, 2)) || !aligned(out, 4))
        return fail(QA_ERR_ALIGN, "%s: X, Wq 16-byte, workspace 256-byte, out/s_w 4-byte aligned", fn);
    if (with_workspace && workspace_bytes < mixed_layout(M, K).total)
        return fail(QA_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, workspace_bytes, mixed_layout(M, K).total);
    return ok();
}

qa_status mixed_run(const char* fn, const void* X_f16, int64_t M, int64_t K, const int8_t* Wq, const float* s_w,
                    const void* W_f16_or_null, int64_t N, float threshold, void* out, qa_dtype out_dtype,
                    void* workspace, void* stream) {
    const MixedLayout L = mixed_layout(M, K);
    const uint16_t* X = static_cast<const uint16_t*>(X_f16);
    hipStream_t st = as_stream(stream);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    int32_t* idx = reinterpret_cast<int32_t*>(ws + L.idx);
    int32_t* count = reinterpret_cast<int32_t*>(ws + L.count);
    float* s_x = reinterpret_cast<float*>(ws + L.s_x);
    int8_t* xq = reinterpret_cast<int8_t*>(ws + L.xq);
    uint16_t* xo = reinterpret_cast<uint16_t*>(ws + L.xo);
    if (decode_supported(M, K)) {
        const hipError_t e = launch_decode_mixed(X, M, K, Wq, s_w, static_cast<const uint16_t*>(W_f16_or_null), N,
                                                 threshold, out, (int)out_dtype, DecodeStages{idx, count, s_x, xq}, st);
        return e == hipSuccess ? ok() : fail(QA_ERR_DEVICE, "%s (decode kernel): %s", fn, hipGetErrorString(e));
    }
    hipError_t e;
    if (!(threshold < 65504.0f)) {
        // no finite fp16 magnitude exceeds the threshold: no outlier columns
        e = launch_rowquant_i8_no_outliers(X, M, K, xq, s_x, count, st);
        if (e != hipSuccess) return fail(QA_ERR_DEVICE, "%s (row quantization): %s", fn, hipGetErrorString(e));
    } else {
        int segs = 1;
        e = launch_outlier_flags(X, M, K, threshold, ws + L.cmax, &segs, st);
        if (e != hipSuccess) return fail(QA_ERR_DEVICE, "%s (outlier columns): %s", fn, hipGetErrorString(e));
        e = launch_rowquant_i8_flags(X, M, K, ws + L.cmax, segs, xq, s_x, idx, count, xo, st);
        if (e != hipSuccess) return fail(QA_ERR_DEVICE, "%s (row quantization): %s", fn, hipGetErrorString(e));
    }
    MixedEpilogue ep;
    ep.s_x = s_x;
    ep.s_w = s_w;
    ep.X = X;
    ep.W16 = static_cast<const uint16_t*>(W_f16_or_null);
    ep.Wq = Wq;
    ep.idx = idx;
    ep.count = count;
    ep.Xo = rowquant_writes_xo(K) ? xo : nullptr;
    ep.out = out;
    ep.ldo = N;
    ep.out_dtype = (int)out_dtype;
    e = launch_gemm_i8_mixed(xq, Wq, M, K, N, ep, st);
    return e == hipSuccess ? ok() : fail(QA_ERR_DEVICE, "%s (gemm): %s", fn, hipGetErrorString(e));
}

}  // namespace qa

extern "C" {

const char* qa_status_string(qa_status s) {
    switch (s) {
        case QA_OK: return "QA_OK";
        case QA_ERR_NULL: return "QA_ERR_NULL";
        case QA_ERR_SHAPE: return "QA_ERR_SHAPE";
        case QA_ERR_ALIGN: return "QA_ERR_ALIGN";
        case QA_ERR_VALUE: return "QA_ERR_VALUE";
        case QA_ERR_WORKSPACE: return "QA_ERR_WORKSPACE";
        case QA_ERR_UNSUPPORTED: return "QA_ERR_UNSUPPORTED";
        case QA_ERR_DEVICE: return "QA_ERR_DEVICE";
    }
    return "QA_ERR_UNKNOWN";
}

const char* qa_last_error(void) { return g_last_error; }

// ----------------------------------------------------------------- outliers
size_t qa_outlier_cols_workspace(int64_t K) { return K > 0 ? up(qa::outlier_scratch_bytes(K)) : 0; }

qa_status qa_outlier_cols(const void* X_f16, int64_t M, int64_t K, float threshold, uint8_t* mask, int32_t* idx,
                          int32_t* count, float* colmax_or_null, void* scratch, size_t scratch_bytes,
                          void* stream) {
    if (M < 0 || K <= 0 || K % 8 != 0 || K > ((int64_t)1 << 22))
        return fail(QA_ERR_SHAPE, "qa_outlier_cols: need M >= 0, 0 < K <= 2^22, K %% 8 == 0 (M=%lld K=%lld)",
                    (long long)M, (long long)K);
    if ((M > 0 && !X_f16) || !mask || !idx || !count || !scratch)
        return fail(QA_ERR_NULL, "qa_outlier_cols: NULL pointer");
    if (!aligned(X_f16, 16) || !aligned(idx, 4) || !aligned(count, 4) || !aligned(scratch, 4) ||
        (colmax_or_null && !aligned(colmax_or_null, 4)))
        return fail(QA_ERR_ALIGN, "qa_outlier_cols: X must be 16-byte aligned, idx/count/colmax/scratch 4-byte");
    if (std::isnan(threshold)) return fail(QA_ERR_VALUE, "qa_outlier_cols: threshold is NaN");
    if (scratch_bytes < qa_outlier_cols_workspace(K))
        return fail(QA_ERR_WORKSPACE, "qa_outlier_cols: scratch %zu < %zu bytes", scratch_bytes,
                    qa_outlier_cols_workspace(K));
    return device_status(qa::launch_outlier_cols(static_cast<const uint16_t*>(X_f16), M, K, threshold, mask, idx,
                                                 count, colmax_or_null, scratch, as_stream(stream)),
                         "qa_outlier_cols");
}

qa_status qa_outlier_topk(const void* X_f16, int64_t M, int64_t K, int64_t k, uint8_t* mask, int32_t* idx,
                          int32_t* count, float* colmax_or_null, void* scratch, size_t scratch_bytes, void* stream) {
    if (M < 0 || K <= 0 || K % 8 != 0 || K > qa::topk_max_columns())
        return fail(QA_ERR_SHAPE, "qa_outlier_topk: need M >= 0, 0 < K <= %lld, K %% 8 == 0 (M=%lld K=%lld)",
                    (long long)qa::topk_max_columns(), (long long)M, (long long)K);
    if (k < 0 || k > K) return fail(QA_ERR_VALUE, "qa_outlier_topk: need 0 <= k <= K (k=%lld)", (long long)k);
    if ((M > 0 && !X_f16) || !mask || !idx || !count || !scratch)
        return fail(QA_ERR_NULL, "qa_outlier_topk: NULL pointer");
    if (!aligned(X_f16, 16) || !aligned(idx, 4) || !aligned(count, 4) || !aligned(scratch, 8) ||
        (colmax_or_null && !aligned(colmax_or_null, 4)))
        return fail(QA_ERR_ALIGN, "qa_outlier_topk: X must be 16-byte aligned, scratch 8-byte, idx/count/colmax 4-byte");
    if (scratch_bytes < qa_outlier_cols_workspace(K))
        return fail(QA_ERR_WORKSPACE, "qa_outlier_topk: scratch %zu < %zu bytes", scratch_bytes,
                    qa_outlier_cols_workspace(K));
    return device_status(qa::launch_outlier_topk(static_cast<const uint16_t*>(X_f16), M, K, k, mask, idx, count,
                                                 colmax_or_null, scratch, as_stream(stream)),
                         "qa_outlier_topk");
}

// ----------------------------------------------------------------- row quant
qa_status qa_quantize_rowwise_int8(const void* X_f16, int64_t rows, int64_t K, const uint8_t* mask_or_null,
                                   int32_t q_min, int32_t q_max, const float* s_in_or_null,
                                   const int32_t* z_in_or_null, int8_t* Xq, float* s_out_or_null, void* stream) {
    const bool dynamic = s_in_or_null == nullptr;
    if (rows < 0 || K <= 0 || K % 8 != 0 || K > kMaxK_quant)
        return fail(QA_ERR_SHAPE, "qa_quantize_rowwise_int8: need rows >= 0, 0 < K <= 2^26, K %% 8 == 0");
    if (q_min > q_max || q_min < -128 || q_max > 127)
        return fail(QA_ERR_VALUE, "qa_quantize_rowwise_int8: need -128 <= q_min <= q_max <= 127");
    if (dynamic && (q_max <= 0 || z_in_or_null))
        return fail(QA_ERR_VALUE, "qa_quantize_rowwise_int8: dynamic mode needs q_max > 0 and no zero-point");
    if (rows == 0) return ok();
    if (!X_f16 || !Xq || (dynamic && !s_out_or_null))
        return fail(QA_ERR_NULL, "qa_quantize_rowwise_int8: NULL X, Xq, or s_out in dynamic mode");
    if (!aligned(X_f16, 16) || !aligned(Xq, 16) || (mask_or_null && !aligned(mask_or_null, 8)) ||
        (s_out_or_null && !aligned(s_out_or_null, 4)) || (s_in_or_null && !aligned(s_in_or_null, 4)) ||
        (z_in_or_null && !aligned(z_in_or_null, 4)))
        return fail(QA_ERR_ALIGN, "qa_quantize_rowwise_int8: X, Xq 16-byte, mask 8-byte, scales 4-byte aligned");
    return device_status(qa::launch_rowquant_i8(static_cast<const uint16_t*>(X_f16), rows, K, mask_or_null, q_min,
                                                q_max, s_in_or_null, z_in_or_null, Xq, s_out_or_null,
                                                as_stream(stream)),
                         "qa_quantize_rowwise_int8");
}

// ----------------------------------------------------------------- int8 mixed linear
size_t qa_qlinear_int8_mixed_workspace(int64_t M, int64_t K) {
    if (M < 0 || K <= 0) return 0;
    return mixed_layout(M, K).total;
}

qa_status qa_qlinear_int8_mixed_offsets(int64_t M, int64_t K, size_t* offsets) {
    if (M <= 0 || K <= 0)
        return fail(QA_ERR_SHAPE, "qa_qlinear_int8_mixed_offsets: need M, K > 0 (M=%lld K=%lld)", (long long)M,
                    (long long)K);
    if (!offsets) return fail(QA_ERR_NULL, "qa_qlinear_int8_mixed_offsets: NULL offsets");
    const MixedLayout L = mixed_layout(M, K);
    offsets[0] = L.idx;
    offsets[1] = L.count;
    offsets[2] = L.s_x;
    offsets[3] = L.xq;
    return ok();
}

qa_status qa_qlinear_int8_mixed(const void* X_f16, int64_t M, int64_t K, const int8_t* Wq, const float* s_w,
                                const void* W_f16_or_null, int64_t N, float threshold, void* out,
                                qa_dtype out_dtype, void* workspace, size_t workspace_bytes, void* stream) {
    bool empty = false;
    const qa_status v = qa::mixed_validate("qa_qlinear_int8_mixed", X_f16, M, K, Wq, s_w, W_f16_or_null, N,
                                           threshold, out, out_dtype, true, workspace, workspace_bytes, &empty);
    if (v != QA_OK || empty) return v;
    return qa::mixed_run("qa_qlinear_int8_mixed", X_f16, M, K, Wq, s_w, W_f16_or_null, N, threshold, out,
                         out_dtype, workspace, stream);
}

// ----------------------------------------------------------------- top-k mixed linear
size_t qa_qlinear_int8_topk_workspace(int64_t M, int64_t K) { return qa_qlinear_int8_mixed_workspace(M, K); }

qa_status qa_qlinear_int8_topk(const void* X_f16, int64_t M, int64_t K, int64_t k, const int8_t* Wq, const float* s_w,
                               const void* W_f16_or_null, int64_t N, void* out, qa_dtype out_dtype, void* workspace,
                               size_t workspace_bytes, void* stream) {
    if (M < 0 || N < 0 || K <= 0 || K % 16 != 0 || K > qa::topk_max_columns())
        return fail(QA_ERR_SHAPE, "qa_qlinear_int8_topk: need M, N >= 0, 0 < K <= %lld, K %% 16 == 0",
                    (long long)qa::topk_max_columns());
    if (k < 0 || k > K) return fail(QA_ERR_VALUE, "qa_qlinear_int8_topk: need 0 <= k <= K (k=%lld)", (long long)k);
    if (!valid_dtype(out_dtype)) return fail(QA_ERR_VALUE, "qa_qlinear_int8_topk: bad out_dtype %d", (int)out_dtype);
    if (M == 0 || N == 0) return ok();
    if (!X_f16 || !Wq || !s_w || !out || !workspace) return fail(QA_ERR_NULL, "qa_qlinear_int8_topk: NULL pointer");
    if (!aligned(X_f16, 16) || !aligned(Wq, 16) || !aligned(s_w, 4) || !aligned(workspace, kAlign) ||
        (W_f16_or_null && !aligned(W_f16_or_null, 2)) || !aligned(out, 4))
        return fail(QA_ERR_ALIGN, "qa_qlinear_int8_topk: X, Wq 16-byte, workspace 256-byte, out/s_w 4-byte aligned");
    const MixedLayout L = mixed_layout(M, K);
    if (workspace_bytes < L.total)
        return fail(QA_ERR_WORKSPACE, "qa_qlinear_int8_topk: workspace %zu < %zu bytes", workspace_bytes, L.total);
    const uint16_t* X = static_cast<const uint16_t*>(X_f16);
    hipStream_t st = as_stream(stream);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    int32_t* idx = reinterpret_cast<int32_t*>(ws + L.idx);
    int32_t* count = reinterpret_cast<int32_t*>(ws + L.count);
    float* s_x = reinterpret_cast<float*>(ws + L.s_x);
    int8_t* xq = reinterpret_cast<int8_t*>(ws + L.xq);
    uint16_t* xo = reinterpret_cast<uint16_t*>(ws + L.xo);
    if (qa::decode_supported(M, K) && k <= qa::decode_topk_max())
        return device_status(qa::launch_decode_topk(X, M, K, k, Wq, s_w, static_cast<const uint16_t*>(W_f16_or_null),
                                                    N, out, (int)out_dtype, qa::DecodeStages{idx, count, s_x, xq}, st),
                             "qa_qlinear_int8_topk (decode kernel)");
    int segs = 1;
    hipError_t e = qa::launch_outlier_topk_flags(X, M, K, k, ws + L.cmax, &segs, st);
    if (e != hipSuccess) return device_status(e, "qa_qlinear_int8_topk (top-k columns)");
    e = qa::launch_rowquant_i8_flags(X, M, K, ws + L.cmax, segs, xq, s_x, idx, count, xo, st);
    if (e != hipSuccess) return device_status(e, "qa_qlinear_int8_topk (row quantization)");
    qa::MixedEpilogue ep;
    ep.s_x = s_x;
    ep.s_w = s_w;
    ep.X = X;
    ep.W16 = static_cast<const uint16_t*>(W_f16_or_null);
    ep.Wq = Wq;
    ep.idx = idx;
    ep.count = count;
    ep.Xo = qa::rowquant_writes_xo(K) ? xo : nullptr;
    ep.out = out;
    ep.ldo = N;
    ep.out_dtype = (int)out_dtype;
    return device_status(qa::launch_gemm_i8_mixed(xq, Wq, M, K, N, ep, st), "qa_qlinear_int8_topk (gemm)");
}

// ----------------------------------------------------------------- zero-point (asymmetric)
qa_status qa_quantize_rowwise_int8_asym(const void* X_f16, int64_t rows, int64_t K, int32_t q_min, int32_t q_max,
                                        int8_t* q, float* s_out, int32_t* z_out, int32_t* rowsum_or_null,
                                        void* stream) {
    if (rows < 0 || K <= 0 || K % 8 != 0 || K > kMaxK_quant)
        return fail(QA_ERR_SHAPE, "qa_quantize_rowwise_int8_asym: need rows >= 0, 0 < K <= 2^26, K %% 8 == 0");
    if (q_min >= q_max || q_min < -128 || q_max > 127)
        return fail(QA_ERR_VALUE, "qa_quantize_rowwise_int8_asym: need -128 <= q_min < q_max <= 127");
    if (rows == 0) return ok();
    if (!X_f16 || !q || !s_out || !z_out) return fail(QA_ERR_NULL, "qa_quantize_rowwise_int8_asym: NULL pointer");
    if (!aligned(X_f16, 16) || !aligned(q, 16) || !aligned(s_out, 4) || !aligned(z_out, 4) ||
        (rowsum_or_null && !aligned(rowsum_or_null, 4)))
        return fail(QA_ERR_ALIGN, "qa_quantize_rowwise_int8_asym: X, q 16-byte, s/z/rowsum 4-byte aligned");
    return device_status(qa::launch_rowquant_i8_asym(static_cast<const uint16_t*>(X_f16), rows, K, q_min, q_max, q,
                                                     s_out, z_out, rowsum_or_null, as_stream(stream)),
                         "qa_quantize_rowwise_int8_asym");
}

qa_status qa_int8_row_sums(const int8_t* A, int64_t rows, int64_t K, int32_t* sums, void* stream) {
    if (rows < 0 || K <= 0 || K % 16 != 0 || K > kMaxK_quant)
        return fail(QA_ERR_SHAPE, "qa_int8_row_sums: need rows >= 0, 0 < K <= 2^26, K %% 16 == 0");
    if (rows == 0) return ok();
    if (!A || !sums) return fail(QA_ERR_NULL, "qa_int8_row_sums: NULL pointer");
    if (!aligned(A, 16) || !aligned(sums, 4))
        return fail(QA_ERR_ALIGN, "qa_int8_row_sums: A 16-byte, sums 4-byte aligned");
    return device_status(qa::launch_row_sums_i8(A, rows, K, sums, as_stream(stream)), "qa_int8_row_sums");
}

size_t qa_qlinear_int8_asym_workspace(int64_t M, int64_t K) {
    if (M < 0 || K <= 0) return 0;
    return asym_layout(M, K).total;
}

qa_status qa_qlinear_int8_asym(const void* X_f16, int64_t M, int64_t K, const int8_t* Wq, const float* s_w,
                               const int32_t* z_w_or_null, const int32_t* w_rowsum, int64_t N, void* out,
                               qa_dtype out_dtype, void* workspace, size_t workspace_bytes, void* stream) {
    if (M < 0 || N < 0 || K <= 0 || K % 16 != 0 || K > kMaxK_asym)
        return fail(QA_ERR_SHAPE, "qa_qlinear_int8_asym: need M, N >= 0, 0 < K <= %lld, K %% 16 == 0",
                    (long long)kMaxK_asym);
    if (!valid_dtype(out_dtype)) return fail(QA_ERR_VALUE, "qa_qlinear_int8_asym: bad out_dtype %d", (int)out_dtype);
    if (M == 0 || N == 0) return ok();
    if (!X_f16 || !Wq || !s_w || !w_rowsum || !out || !workspace)
        return fail(QA_ERR_NULL, "qa_qlinear_int8_asym: NULL pointer");
    if (!aligned(X_f16, 16) || !aligned(Wq, 16) || !aligned(s_w, 4) || !aligned(w_rowsum, 4) || !aligned(out, 4) ||
        (z_w_or_null && !aligned(z_w_or_null, 4)) || !aligned(workspace, kAlign))
        return fail(QA_ERR_ALIGN, "qa_qlinear_int8_asym: X, Wq 16-byte, workspace 256-byte, other arrays 4-byte");
    const AsymLayout L = asym_layout(M, K);
    if (workspace_bytes < L.total)
        return fail(QA_ERR_WORKSPACE, "qa_qlinear_int8_asym: workspace %zu < %zu bytes", workspace_bytes, L.total);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    float* s_x = reinterpret_cast<float*>(ws + L.s_x);
    int32_t* z_x = reinterpret_cast<int32_t*>(ws + L.z_x);
    int32_t* r_x = reinterpret_cast<int32_t*>(ws + L.r_x);
    int8_t* xq = reinterpret_cast<int8_t*>(ws + L.xq);
    hipStream_t st = as_stream(stream);
    hipError_t e = qa::launch_rowquant_i8_asym(static_cast<const uint16_t*>(X_f16), M, K, -128, 127, xq, s_x, z_x,
                                               r_x, st);
    if (e != hipSuccess) return device_status(e, "qa_qlinear_int8_asym (row quantization)");
    qa::AsymEpilogue ep;
    ep.s_x = s_x;
    ep.z_x = z_x;
    ep.r_x = r_x;
    ep.s_w = s_w;
    ep.z_w = z_w_or_null;
    ep.r_w = w_rowsum;
    ep.out = out;
    ep.ldo = N;
    ep.out_dtype = (int)out_dtype;
    return device_status(qa::launch_gemm_i8_asym(xq, Wq, M, K, N, ep, st), "qa_qlinear_int8_asym (gemm)");
}

// ----------------------------------------------------------------- SmoothQuant
size_t qa_col_absmax_workspace(int64_t K) { return qa_outlier_cols_workspace(K); }

qa_status qa_col_absmax(const void* A_f16, int64_t rows, int64_t K, float* colmax, int accumulate, void* scratch,
                        size_t scratch_bytes, void* stream) {
    if (rows < 0 || K <= 0 || K % 8 != 0 || K > ((int64_t)1 << 22))
        return fail(QA_ERR_SHAPE, "qa_col_absmax: need rows >= 0, 0 < K <= 2^22, K %% 8 == 0 (rows=%lld K=%lld)",
                    (long long)rows, (long long)K);
    if (rows == 0) return ok();
    if (!A_f16 || !colmax || !scratch) return fail(QA_ERR_NULL, "qa_col_absmax: NULL pointer");
    if (!aligned(A_f16, 16) || !aligned(colmax, 4) || !aligned(scratch, 4))
        return fail(QA_ERR_ALIGN, "qa_col_absmax: A must be 16-byte aligned, colmax/scratch 4-byte");
    if (scratch_bytes < qa_col_absmax_workspace(K))
        return fail(QA_ERR_WORKSPACE, "qa_col_absmax: scratch %zu < %zu bytes", scratch_bytes,
                    qa_col_absmax_workspace(K));
    return device_status(qa::launch_col_absmax(static_cast<const uint16_t*>(A_f16), rows, K, colmax, accumulate != 0,
                                               scratch, as_stream(stream)),
                         "qa_col_absmax");
}

qa_status qa_smooth_factors(const float* act_absmax, const float* w_absmax, int64_t K, float alpha, float* s,
                            void* stream) {
    if (K < 0) return fail(QA_ERR_SHAPE, "qa_smooth_factors: K < 0");
    if (!(alpha >= 0.0f && alpha <= 1.0f)) return fail(QA_ERR_VALUE, "qa_smooth_factors: alpha must be in [0, 1]");
    if (K == 0) return ok();
    if (!act_absmax || !w_absmax || !s) return fail(QA_ERR_NULL, "qa_smooth_factors: NULL pointer");
    if (!aligned(act_absmax, 4) || !aligned(w_absmax, 4) || !aligned(s, 4))
        return fail(QA_ERR_ALIGN, "qa_smooth_factors: arrays must be 4-byte aligned");
    return device_status(qa::launch_smooth_factors(act_absmax, w_absmax, K, alpha, s, as_stream(stream)),
                         "qa_smooth_factors");
}

qa_status qa_quantize_smooth_int8(const void* A_f16, int64_t rows, int64_t K, const float* s, qa_smooth_op op,
                                  qa_scale_mode mode, int8_t* q, float* s_out, void* stream) {
    if (rows < 0 || K <= 0 || K % 8 != 0 || K > kMaxK_quant)
        return fail(QA_ERR_SHAPE, "qa_quantize_smooth_int8: need rows >= 0, 0 < K <= 2^26, K %% 8 == 0");
    if (op != QA_SMOOTH_DIVIDE && op != QA_SMOOTH_MULTIPLY)
        return fail(QA_ERR_VALUE, "qa_quantize_smooth_int8: bad op %d", (int)op);
    if (mode != QA_SCALE_PER_ROW && mode != QA_SCALE_PER_TENSOR)
        return fail(QA_ERR_VALUE, "qa_quantize_smooth_int8: mode must be PER_ROW or PER_TENSOR (%d)", (int)mode);
    if (rows == 0) return ok();
    if (!A_f16 || !s || !q || !s_out) return fail(QA_ERR_NULL, "qa_quantize_smooth_int8: NULL pointer");
    if (!aligned(A_f16, 16) || !aligned(q, 16) || !aligned(s, 4) || !aligned(s_out, 4))
        return fail(QA_ERR_ALIGN, "qa_quantize_smooth_int8: A, q 16-byte, s, s_out 4-byte aligned");
    return device_status(qa::launch_smoothquant_i8(static_cast<const uint16_t*>(A_f16), rows, K, s,
                                                   op == QA_SMOOTH_MULTIPLY, mode == QA_SCALE_PER_TENSOR, q, s_out,
                                                   nullptr, as_stream(stream)),
                         "qa_quantize_smooth_int8");
}

size_t qa_qlinear_int8_smooth_workspace(int64_t M, int64_t K) {
    if (M < 0 || K <= 0) return 0;
    return smooth_layout(M, K).total;
}

qa_status qa_qlinear_int8_smooth(const void* X_f16, int64_t M, int64_t K, const float* s, qa_scale_mode mode,
                                 const int8_t* Wq, const float* s_w, int64_t N, void* out, qa_dtype out_dtype,
                                 void* workspace, size_t workspace_bytes, void* stream) {
    if (M < 0 || N < 0 || K <= 0 || K % 16 != 0 || K > kMaxK_i8)
        return fail(QA_ERR_SHAPE, "qa_qlinear_int8_smooth: need M, N >= 0, 0 < K <= %lld, K %% 16 == 0",
                    (long long)kMaxK_i8);
    if (mode != QA_SCALE_PER_ROW && mode != QA_SCALE_PER_TENSOR)
        return fail(QA_ERR_VALUE, "qa_qlinear_int8_smooth: mode must be PER_ROW or PER_TENSOR (%d)", (int)mode);
    if (!valid_dtype(out_dtype)) return fail(QA_ERR_VALUE, "qa_qlinear_int8_smooth: bad out_dtype %d", (int)out_dtype);
    if (M == 0 || N == 0) return ok();
    if (!X_f16 || !s || !Wq || !s_w || !out || !workspace)
        return fail(QA_ERR_NULL, "qa_qlinear_int8_smooth: NULL pointer");
    if (!aligned(X_f16, 16) || !aligned(Wq, 16) || !aligned(s, 4) || !aligned(s_w, 4) || !aligned(out, 4) ||
        !aligned(workspace, kAlign))
        return fail(QA_ERR_ALIGN, "qa_qlinear_int8_smooth: X, Wq 16-byte, workspace 256-byte, s/s_w/out 4-byte");
    const SmoothLayout L = smooth_layout(M, K);
    if (workspace_bytes < L.total)
        return fail(QA_ERR_WORKSPACE, "qa_qlinear_int8_smooth: workspace %zu < %zu bytes", workspace_bytes, L.total);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    int32_t* count = reinterpret_cast<int32_t*>(ws + L.count);
    float* s_x = reinterpret_cast<float*>(ws + L.s_x);
    int8_t* xq = reinterpret_cast<int8_t*>(ws + L.xq);
    hipStream_t st = as_stream(stream);
    const uint16_t* X = static_cast<const uint16_t*>(X_f16);
    if (qa::decode_smooth_supported(M, K)) {
        // decode shapes: one launch of the fused decode kernel (the count is
        // 0, so the outlier list slot is never written)
        return device_status(qa::launch_decode_smooth(X, M, K, s, mode == QA_SCALE_PER_TENSOR, Wq, s_w, N, out,
                                                      (int)out_dtype, qa::DecodeStages{count, count, s_x, xq}, st),
                             "qa_qlinear_int8_smooth (decode kernel)");
    }
    hipError_t e = qa::launch_smoothquant_i8(X, M, K, s, false, mode == QA_SCALE_PER_TENSOR, xq, s_x, count, st);
    if (e != hipSuccess) return device_status(e, "qa_qlinear_int8_smooth (smoothing quantization)");
    qa::MixedEpilogue ep;
    ep.s_x = s_x;
    ep.s_w = s_w;
    ep.X = X;
    ep.W16 = nullptr;
    ep.Wq = Wq;
    ep.idx = count;            // never read: the count is 0
    ep.count = count;
    ep.Xo = nullptr;
    ep.out = out;
    ep.ldo = N;
    ep.out_dtype = (int)out_dtype;
    return device_status(qa::launch_gemm_i8_mixed(xq, Wq, M, K, N, ep, st), "qa_qlinear_int8_smooth (gemm)");
}

// ----------------------------------------------------------------- Hadamard + int4
qa_status qa_hadamard_quant_int4(const void* X_f16, int64_t rows, int64_t K, int32_t G, qa_scale_mode mode,
                                 int32_t q_min, int32_t q_max, uint32_t* packed, float* s, void* stream) {
    if (mode != QA_SCALE_PER_ROW && mode != QA_SCALE_PER_GROUP)
        return fail(QA_ERR_VALUE, "qa_hadamard_quant_int4: bad scale mode %d", (int)mode);
    if (G < 1 || G > 256 || (G & (G - 1)) != 0)
        return fail(QA_ERR_SHAPE, "qa_hadamard_quant_int4: G must be a power of two in [1, 256] (G=%d)", G);
    if (rows < 0 || K <= 0 || K % 8 != 0 || K % G != 0 || (mode == QA_SCALE_PER_GROUP && G < 8))
        return fail(QA_ERR_SHAPE,
                    "qa_hadamard_quant_int4: need rows >= 0, K > 0, K %% 8 == 0, K %% G == 0, G >= 8 per group");
    if (q_min > q_max || q_min < -8 || q_max > 7 || q_max <= 0)
        return fail(QA_ERR_VALUE, "qa_hadamard_quant_int4: need -8 <= q_min <= q_max <= 7, q_max > 0");
    if (rows == 0) return ok();
    if (!X_f16 || !packed || !s) return fail(QA_ERR_NULL, "qa_hadamard_quant_int4: NULL pointer");
    if (!aligned(X_f16, 16) || !aligned(packed, 4) || !aligned(s, 4))
        return fail(QA_ERR_ALIGN, "qa_hadamard_quant_int4: X 16-byte, packed/s 4-byte aligned");
    return device_status(qa::launch_hadamard_quant_i4(static_cast<const uint16_t*>(X_f16), rows, K, G,
                                                      mode == QA_SCALE_PER_GROUP, q_min, q_max, packed, s,
                                                      as_stream(stream)),
                         "qa_hadamard_quant_int4");
}

// ----------------------------------------------------------------- W4A4 linear
size_t qa_qlinear_w4a4_workspace(int64_t M, int64_t K) {
    if (M < 0 || K <= 0) return 0;
    return w4_layout(M, K).total;
}

// Every power of two from 8 to 256: G >= 64 on the MFMA GEMMs, 8 <= G <= 32
// on the VALU dot-product kernels (a 64-deep MFMA step would span groups).
static bool w4_group_ok(int32_t G) { return G >= 8 && G <= 256 && (G & (G - 1)) == 0; }

qa_status qa_qlinear_w4a4(const void* X_f16, int64_t M, int64_t K, const uint32_t* Wp, const float* s_w, int64_t N,
                          int32_t G, void* out, qa_dtype out_dtype, void* workspace, size_t workspace_bytes,
                          void* stream) {
    if (!w4_group_ok(G) || M < 0 || N < 0 || K <= 0 || K % G != 0)
        return fail(QA_ERR_SHAPE, "qa_qlinear_w4a4: need G a power of two in [8, 256], M, N >= 0, K > 0, K %% G == 0");
    if (!valid_dtype(out_dtype)) return fail(QA_ERR_VALUE, "qa_qlinear_w4a4: bad out_dtype %d", (int)out_dtype);
    if (M == 0 || N == 0) return ok();
    if (!X_f16 || !Wp || !s_w || !out || !workspace) return fail(QA_ERR_NULL, "qa_qlinear_w4a4: NULL pointer");
    if (!aligned(X_f16, 16) || !aligned(Wp, 16) || !aligned(s_w, 4) || !aligned(out, 4) ||
        !aligned(workspace, kAlign))
        return fail(QA_ERR_ALIGN, "qa_qlinear_w4a4: X, Wp 16-byte, workspace 256-byte, out/s_w 4-byte aligned");
    const W4Layout L = w4_layout(M, K);
    if (workspace_bytes < L.total)
        return fail(QA_ERR_WORKSPACE, "qa_qlinear_w4a4: workspace %zu < %zu bytes", workspace_bytes, L.total);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    uint32_t* xp = reinterpret_cast<uint32_t*>(ws + L.xp);
    float* s_x = reinterpret_cast<float*>(ws + L.s_x);
    hipStream_t st = as_stream(stream);
    hipError_t e = qa::launch_hadamard_quant_i4(static_cast<const uint16_t*>(X_f16), M, K, G, false, -7, 7, xp, s_x, st);
    if (e != hipSuccess) return device_status(e, "qa_qlinear_w4a4 (hadamard quant)");
    return device_status(qa::launch_gemm_w4a4(xp, s_x, Wp, s_w, M, K, N, G, out, (int)out_dtype, st),
                         "qa_qlinear_w4a4 (gemm)");
}

// ----------------------------------------------------------------- W4A8
qa_status qa_hadamard_quant_int8(const void* X_f16, int64_t rows, int64_t K, int32_t G, int32_t q_min, int32_t q_max,
                                 int8_t* q, float* s, void* stream) {
    if (G < 1 || G > 256 || (G & (G - 1)) != 0)
        return fail(QA_ERR_SHAPE, "qa_hadamard_quant_int8: G must be a power of two in [1, 256] (G=%d)", G);
    if (rows < 0 || K <= 0 || K % 8 != 0 || K % G != 0)
        return fail(QA_ERR_SHAPE, "qa_hadamard_quant_int8: need rows >= 0, K > 0, K %% 8 == 0, K %% G == 0");
    if (q_min > q_max || q_min < -128 || q_max > 127 || q_max <= 0)
        return fail(QA_ERR_VALUE, "qa_hadamard_quant_int8: need -128 <= q_min <= q_max <= 127, q_max > 0");
    if (rows == 0) return ok();
    if (!X_f16 || !q || !s) return fail(QA_ERR_NULL, "qa_hadamard_quant_int8: NULL pointer");
    if (!aligned(X_f16, 16) || !aligned(q, 8) || !aligned(s, 4))
        return fail(QA_ERR_ALIGN, "qa_hadamard_quant_int8: X 16-byte, q 8-byte, s 4-byte aligned");
    return device_status(qa::launch_hadamard_quant_i8(static_cast<const uint16_t*>(X_f16), rows, K, G, q_min, q_max,
                                                      q, s, as_stream(stream)),
                         "qa_hadamard_quant_int8");
}

size_t qa_qlinear_w4a8_workspace(int64_t M, int64_t K) {
    if (M < 0 || K <= 0) return 0;
    return w4a8_layout(M, K).total;
}

qa_status qa_qlinear_w4a8(const void* X_f16, int64_t M, int64_t K, const uint32_t* Wp, const float* s_w, int64_t N,
                          int32_t G, void* out, qa_dtype out_dtype, void* workspace, size_t workspace_bytes,
                          void* stream) {
    if (!w4_group_ok(G) || M < 0 || N < 0 || K <= 0 || K % G != 0)
        return fail(QA_ERR_SHAPE, "qa_qlinear_w4a8: need G a power of two in [8, 256], M, N >= 0, K > 0, K %% G == 0");
    if (!valid_dtype(out_dtype)) return fail(QA_ERR_VALUE, "qa_qlinear_w4a8: bad out_dtype %d", (int)out_dtype);
    if (M == 0 || N == 0) return ok();
    if (!X_f16 || !Wp || !s_w || !out || !workspace) return fail(QA_ERR_NULL, "qa_qlinear_w4a8: NULL pointer");
    if (!aligned(X_f16, 16) || !aligned(Wp, 16) || !aligned(s_w, 4) || !aligned(out, 4) ||
        !aligned(workspace, kAlign))
        return fail(QA_ERR_ALIGN, "qa_qlinear_w4a8: X, Wp 16-byte, workspace 256-byte, out/s_w 4-byte aligned");
    const W4Layout L = w4a8_layout(M, K);
    if (workspace_bytes < L.total)
        return fail(QA_ERR_WORKSPACE, "qa_qlinear_w4a8: workspace %zu < %zu bytes", workspace_bytes, L.total);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    int8_t* xq = reinterpret_cast<int8_t*>(ws + L.xp);
    float* s_x = reinterpret_cast<float*>(ws + L.s_x);
    hipStream_t st = as_stream(stream);
    hipError_t e =
        qa::launch_hadamard_quant_i8(static_cast<const uint16_t*>(X_f16), M, K, G, -127, 127, xq, s_x, st);
    if (e != hipSuccess) return device_status(e, "qa_qlinear_w4a8 (hadamard quant)");
    return device_status(qa::launch_gemm_w4a8(xq, s_x, Wp, s_w, M, K, N, G, out, (int)out_dtype, st),
                         "qa_qlinear_w4a8 (gemm)");
}

// ----------------------------------------------------------------- W4A4, zero-point activations
qa_status qa_hadamard_quant_int4_asym(const void* X_f16, int64_t rows, int64_t K, int32_t G, uint32_t* packed,
                                      float* s, int32_t* z, void* stream) {
    if (G < 1 || G > 256 || (G & (G - 1)) != 0)
        return fail(QA_ERR_SHAPE, "qa_hadamard_quant_int4_asym: G must be a power of two in [1, 256] (G=%d)", G);
    if (rows < 0 || K <= 0 || K % 8 != 0 || K % G != 0)
        return fail(QA_ERR_SHAPE, "qa_hadamard_quant_int4_asym: need rows >= 0, K > 0, K %% 8 == 0, K %% G == 0");
    if (rows == 0) return ok();
    if (!X_f16 || !packed || !s || !z) return fail(QA_ERR_NULL, "qa_hadamard_quant_int4_asym: NULL pointer");
    if (!aligned(X_f16, 16) || !aligned(packed, 4) || !aligned(s, 4) || !aligned(z, 4))
        return fail(QA_ERR_ALIGN, "qa_hadamard_quant_int4_asym: X 16-byte, packed/s/z 4-byte aligned");
    return device_status(qa::launch_hadamard_quant_i4_asym(static_cast<const uint16_t*>(X_f16), rows, K, G, packed, s,
                                                           z, as_stream(stream)),
                         "qa_hadamard_quant_int4_asym");
}

qa_status qa_w4_column_terms(const uint32_t* Wp, const float* s_w, int64_t N, int64_t K, int32_t G, float* c,
                             void* stream) {
    if (G < 8 || G > 256 || (G & (G - 1)) != 0 || N < 0 || K <= 0 || K % G != 0)
        return fail(QA_ERR_SHAPE, "qa_w4_column_terms: need N >= 0, K > 0, G a power of two in [8, 256], K %% G == 0");
    if (N == 0) return ok();
    if (!Wp || !s_w || !c) return fail(QA_ERR_NULL, "qa_w4_column_terms: NULL pointer");
    if (!aligned(Wp, 4) || !aligned(s_w, 4) || !aligned(c, 4))
        return fail(QA_ERR_ALIGN, "qa_w4_column_terms: Wp, s_w, c 4-byte aligned");
    return device_status(qa::launch_w4_column_terms(Wp, s_w, N, K, G, c, as_stream(stream)), "qa_w4_column_terms");
}

size_t qa_qlinear_w4a4_asym_workspace(int64_t M, int64_t K) {
    if (M < 0 || K <= 0) return 0;
    return w4z_layout(M, K).total;
}

qa_status qa_qlinear_w4a4_asym(const void* X_f16, int64_t M, int64_t K, const uint32_t* Wp, const float* s_w,
                               const float* c_w, int64_t N, int32_t G, void* out, qa_dtype out_dtype, void* workspace,
                               size_t workspace_bytes, void* stream) {
    if (!w4_group_ok(G) || M < 0 || N < 0 || K <= 0 || K % G != 0)
        return fail(QA_ERR_SHAPE, "qa_qlinear_w4a4_asym: need G a power of two in [8, 256], M, N >= 0, K > 0, K %% G == 0");
    if (!valid_dtype(out_dtype)) return fail(QA_ERR_VALUE, "qa_qlinear_w4a4_asym: bad out_dtype %d", (int)out_dtype);
    if (M == 0 || N == 0) return ok();
    if (!X_f16 || !Wp || !s_w || !c_w || !out || !workspace)
        return fail(QA_ERR_NULL, "qa_qlinear_w4a4_asym: NULL pointer");
    if (!aligned(X_f16, 16) || !aligned(Wp, 16) || !aligned(s_w, 4) || !aligned(c_w, 4) || !aligned(out, 4) ||
        !aligned(workspace, kAlign))
        return fail(QA_ERR_ALIGN,
                    "qa_qlinear_w4a4_asym: X, Wp 16-byte, workspace 256-byte, out/s_w/c_w 4-byte aligned");
    const W4zLayout L = w4z_layout(M, K);
    if (workspace_bytes < L.total)
        return fail(QA_ERR_WORKSPACE, "qa_qlinear_w4a4_asym: workspace %zu < %zu bytes", workspace_bytes, L.total);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    uint32_t* xp = reinterpret_cast<uint32_t*>(ws + L.xp);
    float* s_x = reinterpret_cast<float*>(ws + L.s_x);
    int32_t* z_x = reinterpret_cast<int32_t*>(ws + L.z_x);
    hipStream_t st = as_stream(stream);
    hipError_t e = qa::launch_hadamard_quant_i4_asym(static_cast<const uint16_t*>(X_f16), M, K, G, xp, s_x, z_x, st);
    if (e != hipSuccess) return device_status(e, "qa_qlinear_w4a4_asym (hadamard quant)");
    return device_status(qa::launch_gemm_w4a4_asym(xp, s_x, z_x, Wp, s_w, c_w, M, K, N, G, out, (int)out_dtype, st),
                         "qa_qlinear_w4a4_asym (gemm)");
}

// ----------------------------------------------------------------- Kronecker transform (FlatQuant)
qa_status qa_kron_quant_int4(const void* X_f16, int64_t rows, int64_t K, int64_t n1, int64_t n2, const float* P1,
                             const float* P2, qa_scale_mode mode, int32_t G, int32_t q_min, int32_t q_max,
                             uint32_t* packed, float* s, void* stream) {
    if (mode != QA_SCALE_PER_ROW && mode != QA_SCALE_PER_GROUP)
        return fail(QA_ERR_VALUE, "qa_kron_quant_int4: bad scale mode %d", (int)mode);
    if (rows < 0 || K <= 0 || n1 <= 0 || n2 <= 0 || n1 * n2 != K)
        return fail(QA_ERR_SHAPE, "qa_kron_quant_int4: need rows >= 0, n1 n2 == K > 0 (K=%lld n1=%lld n2=%lld)",
                    (long long)K, (long long)n1, (long long)n2);
    if (q_min > q_max || q_min < -8 || q_max > 7 || q_max <= 0)
        return fail(QA_ERR_VALUE, "qa_kron_quant_int4: need -8 <= q_min <= q_max <= 7, q_max > 0");
    const int g = mode == QA_SCALE_PER_GROUP ? G : 0;
    if (mode == QA_SCALE_PER_GROUP && (G <= 0 || K % G != 0))
        return fail(QA_ERR_SHAPE, "qa_kron_quant_int4: per-group needs 0 < G, K %% G == 0 (G=%d)", G);
    if (!qa::kron_supported(n1, n2, g))
        return fail(QA_ERR_UNSUPPORTED,
                    "qa_kron_quant_int4: no kernel for n1=%lld n2=%lld G=%d (sizes 8x8, 8x16, 16x16, 16x32, 32x32, "
                    "32x64, 64x64, 64x128; per group 8 <= G <= 512, G <= 8 n1 n2 / R^2)",
                    (long long)n1, (long long)n2, g);
    if (rows == 0) return ok();
    if (!X_f16 || !P1 || !P2 || !packed || !s) return fail(QA_ERR_NULL, "qa_kron_quant_int4: NULL pointer");
    if (!aligned(X_f16, 16) || !aligned(P1, 16) || !aligned(P2, 16) || !aligned(packed, 4) || !aligned(s, 4))
        return fail(QA_ERR_ALIGN, "qa_kron_quant_int4: X, P1, P2 16-byte, packed/s 4-byte aligned");
    return device_status(qa::launch_kron_quant_i4(static_cast<const uint16_t*>(X_f16), rows, n1, n2, P1, P2, g, q_min,
                                                  q_max, packed, s, as_stream(stream)),
                         "qa_kron_quant_int4");
}

qa_status qa_kron_sizes(int64_t n, int64_t* n1, int64_t* n2, int32_t* has_kernel) {
    if (!n1 || !n2) return fail(QA_ERR_NULL, "qa_kron_sizes: NULL n1 or n2");
    if (n <= 0) return fail(QA_ERR_SHAPE, "qa_kron_sizes: need n > 0 (n=%lld)", (long long)n);
    // for a fixed product the sum is smallest for the closest pair: walk down
    // from floor(sqrt(n)) to the first divisor
    int64_t d = (int64_t)std::sqrt((double)n);
    while (d * d > n) --d;
    while ((d + 1) * (d + 1) <= n) ++d;
    while (n % d != 0) --d;
    *n1 = d;
    *n2 = n / d;
    if (has_kernel) *has_kernel = qa::kron_supported(d, n / d, 0) ? 1 : 0;
    return ok();
}

size_t qa_qlinear_kron_w4a4_workspace(int64_t M, int64_t K) { return qa_qlinear_w4a4_workspace(M, K); }

qa_status qa_qlinear_kron_w4a4(const void* X_f16, int64_t M, int64_t K, int64_t n1, int64_t n2, const float* P1,
                               const float* P2, const uint32_t* Wp, const float* s_w, int64_t N, int32_t G, void* out,
                               qa_dtype out_dtype, void* workspace, size_t workspace_bytes, void* stream) {
    if (!w4_group_ok(G) || M < 0 || N < 0 || K <= 0 || K % G != 0 || n1 <= 0 || n2 <= 0 || n1 * n2 != K)
        return fail(QA_ERR_SHAPE, "qa_qlinear_kron_w4a4: need G a power of two in [8, 256], M, N >= 0, K %% G == 0, n1 n2 == K");
    if (!qa::kron_supported(n1, n2, 0))
        return fail(QA_ERR_UNSUPPORTED, "qa_qlinear_kron_w4a4: no kernel for n1=%lld n2=%lld", (long long)n1,
                    (long long)n2);
    if (!valid_dtype(out_dtype)) return fail(QA_ERR_VALUE, "qa_qlinear_kron_w4a4: bad out_dtype %d", (int)out_dtype);
    if (M == 0 || N == 0) return ok();
    if (!X_f16 || !P1 || !P2 || !Wp || !s_w || !out || !workspace)
        return fail(QA_ERR_NULL, "qa_qlinear_kron_w4a4: NULL pointer");
    if (!aligned(X_f16, 16) || !aligned(P1, 16) || !aligned(P2, 16) || !aligned(Wp, 16) || !aligned(s_w, 4) ||
        !aligned(out, 4) || !aligned(workspace, kAlign))
        return fail(QA_ERR_ALIGN, "qa_qlinear_kron_w4a4: X, P1, P2, Wp 16-byte, workspace 256-byte, out/s_w 4-byte");
    const W4Layout L = w4_layout(M, K);
    if (workspace_bytes < L.total)
        return fail(QA_ERR_WORKSPACE, "qa_qlinear_kron_w4a4: workspace %zu < %zu bytes", workspace_bytes, L.total);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    uint32_t* xp = reinterpret_cast<uint32_t*>(ws + L.xp);
    float* s_x = reinterpret_cast<float*>(ws + L.s_x);
    hipStream_t st = as_stream(stream);
    hipError_t e = qa::launch_kron_quant_i4(static_cast<const uint16_t*>(X_f16), M, n1, n2, P1, P2, 0, -7, 7, xp, s_x,
                                            st);
    if (e != hipSuccess) return device_status(e, "qa_qlinear_kron_w4a4 (transform + quant)");
    return device_status(qa::launch_gemm_w4a4(xp, s_x, Wp, s_w, M, K, N, G, out, (int)out_dtype, st),
                         "qa_qlinear_kron_w4a4 (gemm)");
}

// ----------------------------------------------------------------- parity entry points
qa_status qa_gemm_i8_i32(const int8_t* A, const int8_t* B, int64_t M, int64_t K, int64_t N, int32_t* C,
                         void* stream) {
    if (M < 0 || N < 0 || K <= 0 || K % 16 != 0)
        return fail(QA_ERR_SHAPE, "qa_gemm_i8_i32: need M, N >= 0, K > 0, K %% 16 == 0");
    if (M == 0 || N == 0) return ok();
    if (!A || !B || !C) return fail(QA_ERR_NULL, "qa_gemm_i8_i32: NULL pointer");
    if (!aligned(A, 16) || !aligned(B, 16) || !aligned(C, 4))
        return fail(QA_ERR_ALIGN, "qa_gemm_i8_i32: A, B 16-byte, C 4-byte aligned");
    return device_status(qa::launch_gemm_i8_i32(A, B, M, K, N, C, as_stream(stream)), "qa_gemm_i8_i32");
}

qa_status qa_gemm_w4a4_group_acc(const uint32_t* Xp, const uint32_t* Wp, int64_t M, int64_t K, int64_t N, int32_t G,
                                 int32_t* acc, void* stream) {
    if (!w4_group_ok(G) || M < 0 || N < 0 || K <= 0 || K % G != 0)
        return fail(QA_ERR_SHAPE, "qa_gemm_w4a4_group_acc: need G a power of two in [8, 256], M, N >= 0, K > 0, K %% G == 0");
    if (M == 0 || N == 0) return ok();
    if (!Xp || !Wp || !acc) return fail(QA_ERR_NULL, "qa_gemm_w4a4_group_acc: NULL pointer");
    if (!aligned(Xp, 16) || !aligned(Wp, 16) || !aligned(acc, 4))
        return fail(QA_ERR_ALIGN, "qa_gemm_w4a4_group_acc: Xp, Wp 16-byte, acc 4-byte aligned");
    return device_status(qa::launch_gemm_w4a4_group_acc(Xp, Wp, M, K, N, G, acc, as_stream(stream)),
                         "qa_gemm_w4a4_group_acc");
}

qa_status qa_gemm_w4a8_group_acc(const int8_t* Xq, const uint32_t* Wp, int64_t M, int64_t K, int64_t N, int32_t G,
                                 int32_t* acc, void* stream) {
    if (!w4_group_ok(G) || M < 0 || N < 0 || K <= 0 || K % G != 0)
        return fail(QA_ERR_SHAPE, "qa_gemm_w4a8_group_acc: need G a power of two in [8, 256], M, N >= 0, K > 0, K %% G == 0");
    if (M == 0 || N == 0) return ok();
    if (!Xq || !Wp || !acc) return fail(QA_ERR_NULL, "qa_gemm_w4a8_group_acc: NULL pointer");
    if (!aligned(Xq, 16) || !aligned(Wp, 16) || !aligned(acc, 4))
        return fail(QA_ERR_ALIGN, "qa_gemm_w4a8_group_acc: Xq, Wp 16-byte, acc 4-byte aligned");
    return device_status(qa::launch_gemm_w4a8_group_acc(Xq, Wp, M, K, N, G, acc, as_stream(stream)),
                         "qa_gemm_w4a8_group_acc");
}

qa_status qa_probe_stream_read(const void* src, size_t bytes, int32_t wgs, int32_t lane_bytes, int32_t unroll,
                               uint32_t* sink, void* stream) {
    if (wgs < 1 || wgs > 65536) return fail(QA_ERR_SHAPE, "qa_probe_stream_read: need wgs in [1, 65536]");
    if (lane_bytes != 4 && lane_bytes != 8 && lane_bytes != 16)
        return fail(QA_ERR_VALUE, "qa_probe_stream_read: lane_bytes must be 4, 8 or 16");
    if (unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8)
        return fail(QA_ERR_VALUE, "qa_probe_stream_read: unroll must be 1, 2, 4 or 8");
    if (!src || !sink) return fail(QA_ERR_NULL, "qa_probe_stream_read: NULL pointer");
    if (!aligned(src, 16) || !aligned(sink, 4))
        return fail(QA_ERR_ALIGN, "qa_probe_stream_read: src 16-byte, sink 4-byte aligned");
    return device_status(qa::launch_stream_read(static_cast<const uint8_t*>(src), (uint64_t)bytes, wgs, lane_bytes,
                                                unroll, sink, as_stream(stream)),
                         "qa_probe_stream_read");
}

}  // extern "C"
