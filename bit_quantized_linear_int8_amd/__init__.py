"""Python binding of libqa -- quantized linear layers on AMD MI355X (gfx950).

A thin ctypes layer over the C ABI of ``include/qa.h``: every function has the
name of the C entry point it calls, takes torch tensors that live on the GPU,
allocates the outputs it returns, passes raw device pointers and the current
HIP stream, and raises ``QAError`` on a non-zero status.  All arithmetic runs
in the HIP kernels of ``libqa.so``; there is no fallback path.  If the library
is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqa.so")

QA_F32, QA_F16, QA_BF16 = 0, 1, 2
QA_SCALE_PER_ROW, QA_SCALE_PER_GROUP, QA_SCALE_PER_TENSOR = 0, 1, 2
QA_SMOOTH_DIVIDE, QA_SMOOTH_MULTIPLY = 0, 1

EXPORTS = (
    "qa_status_string", "qa_last_error",
    "qa_outlier_cols_workspace", "qa_outlier_cols", "qa_outlier_topk",
    "qa_quantize_rowwise_int8",
    "qa_qlinear_int8_mixed_workspace", "qa_qlinear_int8_mixed", "qa_qlinear_int8_mixed_offsets",
    "qa_qlinear_int8_mixed_noalloc",
    "qa_qlinear_int8_topk_workspace", "qa_qlinear_int8_topk",
    "qa_quantize_rowwise_int8_asym", "qa_int8_row_sums", "qa_qlinear_int8_asym_workspace", "qa_qlinear_int8_asym",
    "qa_col_absmax_workspace", "qa_col_absmax", "qa_smooth_factors", "qa_quantize_smooth_int8",
    "qa_qlinear_int8_smooth_workspace", "qa_qlinear_int8_smooth",
    "qa_hadamard_quant_int4", "qa_kron_sizes", "qa_kron_quant_int4", "qa_qlinear_kron_w4a4_workspace",
    "qa_qlinear_kron_w4a4",
    "qa_qlinear_w4a4_workspace", "qa_qlinear_w4a4",
    "qa_hadamard_quant_int8", "qa_qlinear_w4a8_workspace", "qa_qlinear_w4a8",
    "qa_hadamard_quant_int4_asym", "qa_w4_column_terms", "qa_qlinear_w4a4_asym_workspace", "qa_qlinear_w4a4_asym",
    "qa_gemm_i8_i32", "qa_gemm_w4a4_group_acc", "qa_gemm_w4a8_group_acc",
    "qa_probe_stream_read",
)

_DTYPE_CODE = {torch.float32: QA_F32, torch.float16: QA_F16, torch.bfloat16: QA_BF16}


class QAError(RuntimeError):
    def __init__(self, fn, status, detail):
        super().__init__("%s failed: %s (%s)" % (fn, status, detail))
        self.status = status
        self.detail = detail


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libqa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libqa.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I32, F, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
        S = ctypes.c_int
        sig = {
            "qa_status_string": (ctypes.c_char_p, [S]),
            "qa_last_error": (ctypes.c_char_p, []),
            "qa_outlier_cols_workspace": (SZ, [I64]),
            "qa_outlier_cols": (S, [P, I64, I64, F, P, P, P, P, P, SZ, P]),
            "qa_outlier_topk": (S, [P, I64, I64, I64, P, P, P, P, P, SZ, P]),
            "qa_qlinear_int8_topk_workspace": (SZ, [I64, I64]),
            "qa_qlinear_int8_topk": (S, [P, I64, I64, I64, P, P, P, I64, P, S, P, SZ, P]),
            "qa_quantize_rowwise_int8": (S, [P, I64, I64, P, I32, I32, P, P, P, P, P]),
            "qa_qlinear_int8_mixed_workspace": (SZ, [I64, I64]),
            "qa_qlinear_int8_mixed": (S, [P, I64, I64, P, P, P, I64, F, P, S, P, SZ, P]),
            "qa_qlinear_int8_mixed_offsets": (S, [I64, I64, P]),
            "qa_qlinear_int8_mixed_noalloc": (S, [P, I64, I64, P, P, P, I64, F, P, S, P]),
            "qa_quantize_rowwise_int8_asym": (S, [P, I64, I64, I32, I32, P, P, P, P, P]),
            "qa_int8_row_sums": (S, [P, I64, I64, P, P]),
            "qa_qlinear_int8_asym_workspace": (SZ, [I64, I64]),
            "qa_qlinear_int8_asym": (S, [P, I64, I64, P, P, P, P, I64, P, S, P, SZ, P]),
            "qa_col_absmax_workspace": (SZ, [I64]),
            "qa_col_absmax": (S, [P, I64, I64, P, S, P, SZ, P]),
            "qa_smooth_factors": (S, [P, P, I64, F, P, P]),
            "qa_quantize_smooth_int8": (S, [P, I64, I64, P, S, S, P, P, P]),
            "qa_qlinear_int8_smooth_workspace": (SZ, [I64, I64]),
            "qa_qlinear_int8_smooth": (S, [P, I64, I64, P, S, P, P, I64, P, S, P, SZ, P]),
            "qa_hadamard_quant_int4": (S, [P, I64, I64, I32, S, I32, I32, P, P, P]),
            "qa_kron_sizes": (S, [I64, P, P, P]),
            "qa_kron_quant_int4": (S, [P, I64, I64, I64, I64, P, P, S, I32, I32, I32, P, P, P]),
            "qa_qlinear_kron_w4a4_workspace": (SZ, [I64, I64]),
            "qa_qlinear_kron_w4a4": (S, [P, I64, I64, I64, I64, P, P, P, P, I64, I32, P, S, P, SZ, P]),
            "qa_qlinear_w4a4_workspace": (SZ, [I64, I64]),
            "qa_qlinear_w4a4": (S, [P, I64, I64, P, P, I64, I32, P, S, P, SZ, P]),
            "qa_gemm_i8_i32": (S, [P, P, I64, I64, I64, P, P]),
            "qa_gemm_w4a4_group_acc": (S, [P, P, I64, I64, I64, I32, P, P]),
            "qa_hadamard_quant_int8": (S, [P, I64, I64, I32, I32, I32, P, P, P]),
            "qa_qlinear_w4a8_workspace": (SZ, [I64, I64]),
            "qa_qlinear_w4a8": (S, [P, I64, I64, P, P, I64, I32, P, S, P, SZ, P]),
            "qa_gemm_w4a8_group_acc": (S, [P, P, I64, I64, I64, I32, P, P]),
            "qa_hadamard_quant_int4_asym": (S, [P, I64, I64, I32, P, P, P, P]),
            "qa_w4_column_terms": (S, [P, P, I64, I64, I32, P, P]),
            "qa_qlinear_w4a4_asym_workspace": (SZ, [I64, I64]),
            "qa_qlinear_w4a4_asym": (S, [P, I64, I64, P, P, P, I64, I32, P, S, P, SZ, P]),
            "qa_probe_stream_read": (S, [P, SZ, I32, I32, I32, P, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_string(s: int) -> str:
    return lib().qa_status_string(int(s)).decode()


def last_error() -> str:
    return lib().qa_last_error().decode()


def _check(fn: str, s: int):
    if s != 0:
        raise QAError(fn, status_string(s), last_error())


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t, name, dtype=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a CUDA (HIP) tensor" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _empty(stream, *args, **kw):
    """torch.empty on the stream the library call runs on: the caching
    allocator then keeps the block for that stream, so memory a call still
    uses is not handed to work on another stream after it is released."""
    if stream is None:
        return torch.empty(*args, **kw)
    with torch.cuda.stream(stream):
        return torch.empty(*args, **kw)


def _workspace(stream, nbytes, device, ws):
    if ws is not None:
        return ws
    return _empty(stream, max(int(nbytes), 1), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------- entry points
def qa_outlier_cols_workspace(K: int) -> int:
    return int(lib().qa_outlier_cols_workspace(K))


def qa_outlier_cols(X, threshold=6.0, scratch=None, stream=None):
    """-> (mask u8 [K], idx i32 [K] (first `count` valid), count i32 [1], colmax f32 [K])."""
    _dev(X, "X", torch.float16)
    M, K = X.shape
    dev = X.device
    mask = _empty(stream, K, dtype=torch.uint8, device=dev)
    idx = _empty(stream, K, dtype=torch.int32, device=dev)
    count = _empty(stream, 1, dtype=torch.int32, device=dev)
    colmax = _empty(stream, K, dtype=torch.float32, device=dev)
    nb = qa_outlier_cols_workspace(K)
    scratch = _workspace(stream, nb, dev, scratch)
    _check("qa_outlier_cols", lib().qa_outlier_cols(_p(X), M, K, float(threshold), _p(mask), _p(idx), _p(count),
                                                     _p(colmax), _p(scratch), scratch.numel(), _stream(stream)))
    return mask, idx, count, colmax


def qa_outlier_topk(X, k: int, scratch=None, stream=None):
    """The k columns of largest max |x| (ties: lower column first)
    -> (mask u8 [K], idx i32 [K] (first `count` valid), count i32 [1], colmax f32 [K])."""
    _dev(X, "X", torch.float16)
    M, K = X.shape
    dev = X.device
    mask = _empty(stream, K, dtype=torch.uint8, device=dev)
    idx = _empty(stream, K, dtype=torch.int32, device=dev)
    count = _empty(stream, 1, dtype=torch.int32, device=dev)
    colmax = _empty(stream, K, dtype=torch.float32, device=dev)
    scratch = _workspace(stream, qa_outlier_cols_workspace(K), dev, scratch)
    _check("qa_outlier_topk", lib().qa_outlier_topk(_p(X), M, K, int(k), _p(mask), _p(idx), _p(count), _p(colmax),
                                                     _p(scratch), scratch.numel(), _stream(stream)))
    return mask, idx, count, colmax


def topk_count(share: float, K: int) -> int:
    """Number of decomposed columns for a share of the K dimensions: ceil(share * K)."""
    import math
    return min(K, max(0, math.ceil(share * K)))


def qa_quantize_rowwise_int8(X, mask=None, q_min=-127, q_max=127, s_in=None, z_in=None, stream=None):
    """-> (Xq i8 [rows x K], s f32 [rows] or None in static mode)."""
    _dev(X, "X", torch.float16)
    rows, K = X.shape
    Xq = _empty(stream, (rows, K), dtype=torch.int8, device=X.device)
    s_out = None if s_in is not None else _empty(stream, rows, dtype=torch.float32, device=X.device)
    _check("qa_quantize_rowwise_int8",
           lib().qa_quantize_rowwise_int8(_p(X), rows, K, _p(mask), int(q_min), int(q_max), _p(s_in), _p(z_in),
                                          _p(Xq), _p(s_out), _stream(stream)))
    return Xq, s_out


def qa_qlinear_int8_mixed_workspace(M: int, K: int) -> int:
    return int(lib().qa_qlinear_int8_mixed_workspace(M, K))


def qa_qlinear_int8_mixed(X, Wq, s_w, W16=None, threshold=6.0, out_dtype=torch.float16, out=None,
                          workspace=None, stream=None):
    """LLM.int8() mixed-precision linear -> out [M x N] of out_dtype."""
    _dev(X, "X", torch.float16)
    _dev(Wq, "Wq", torch.int8)
    _dev(s_w, "s_w", torch.float32)
    if W16 is not None:
        _dev(W16, "W16", torch.float16)
    M, K = X.shape
    N = Wq.shape[0]
    if out is None:
        out = _empty(stream, (M, N), dtype=out_dtype, device=X.device)
    workspace = _workspace(stream, qa_qlinear_int8_mixed_workspace(M, K), X.device, workspace)
    _check("qa_qlinear_int8_mixed",
           lib().qa_qlinear_int8_mixed(_p(X), M, K, _p(Wq), _p(s_w), _p(W16), N, float(threshold), _p(out),
                                       _DTYPE_CODE[out.dtype], _p(workspace), workspace.numel(), _stream(stream)))
    return out


NOALLOC_SCRATCH_BYTES = 40 << 20


def qa_qlinear_int8_mixed_noalloc(X, Wq, s_w, out, W16=None, threshold=6.0, stream=None):
    """LLM.int8() mixed-precision linear into the caller's `out` [M x N] (fp32,
    fp16 or bf16) with the library's static per-GPU scratch: nothing is
    allocated, here or in the library.  Calls that overlap on one GPU race."""
    _dev(X, "X", torch.float16)
    _dev(Wq, "Wq", torch.int8)
    _dev(s_w, "s_w", torch.float32)
    _dev(out, "out")
    if W16 is not None:
        _dev(W16, "W16", torch.float16)
    M, K = X.shape
    N = Wq.shape[0]
    if tuple(out.shape) != (M, N):
        raise ValueError("out must be [%d x %d]" % (M, N))
    _check("qa_qlinear_int8_mixed_noalloc",
           lib().qa_qlinear_int8_mixed_noalloc(_p(X), M, K, _p(Wq), _p(s_w), _p(W16), N, float(threshold), _p(out),
                                               _DTYPE_CODE[out.dtype], _stream(stream)))
    return out


def qa_qlinear_int8_mixed_offsets(M: int, K: int):
    """Byte offsets of (idx, count, s_x, Xq) in the workspace of an LLM.int8()
    call with M tokens and K in-features."""
    off = (ctypes.c_size_t * 4)()
    _check("qa_qlinear_int8_mixed_offsets", lib().qa_qlinear_int8_mixed_offsets(int(M), int(K), off))
    return tuple(int(v) for v in off)


def qa_quantize_rowwise_int8_asym(X, q_min=-128, q_max=127, stream=None):
    """Per-row min-max zero-point codes -> (q i8 [rows x K], s f32 [rows], z i32 [rows], rowsum i32 [rows])."""
    _dev(X, "X", torch.float16)
    rows, K = X.shape
    d = X.device
    q = _empty(stream, (rows, K), dtype=torch.int8, device=d)
    s = _empty(stream, rows, dtype=torch.float32, device=d)
    z = _empty(stream, rows, dtype=torch.int32, device=d)
    rs = _empty(stream, rows, dtype=torch.int32, device=d)
    _check("qa_quantize_rowwise_int8_asym",
           lib().qa_quantize_rowwise_int8_asym(_p(X), rows, K, int(q_min), int(q_max), _p(q), _p(s), _p(z), _p(rs),
                                               _stream(stream)))
    return q, s, z, rs


def qa_int8_row_sums(A, stream=None):
    """Row sums of an int8 matrix -> i32 [rows]."""
    _dev(A, "A", torch.int8)
    rows, K = A.shape
    sums = _empty(stream, rows, dtype=torch.int32, device=A.device)
    _check("qa_int8_row_sums", lib().qa_int8_row_sums(_p(A), rows, K, _p(sums), _stream(stream)))
    return sums


def qa_qlinear_int8_asym_workspace(M: int, K: int) -> int:
    return int(lib().qa_qlinear_int8_asym_workspace(M, K))


def qa_qlinear_int8_asym(X, Wq, s_w, w_rowsum, z_w=None, out_dtype=torch.float16, out=None, workspace=None,
                         stream=None):
    """W8A8 linear with per-token zero-point activations -> out [M x N] of out_dtype."""
    _dev(X, "X", torch.float16)
    _dev(Wq, "Wq", torch.int8)
    _dev(s_w, "s_w", torch.float32)
    _dev(w_rowsum, "w_rowsum", torch.int32)
    if z_w is not None:
        _dev(z_w, "z_w", torch.int32)
    M, K = X.shape
    N = Wq.shape[0]
    if out is None:
        out = _empty(stream, (M, N), dtype=out_dtype, device=X.device)
    workspace = _workspace(stream, qa_qlinear_int8_asym_workspace(M, K), X.device, workspace)
    _check("qa_qlinear_int8_asym",
           lib().qa_qlinear_int8_asym(_p(X), M, K, _p(Wq), _p(s_w), _p(z_w), _p(w_rowsum), N, _p(out),
                                      _DTYPE_CODE[out.dtype], _p(workspace), workspace.numel(), _stream(stream)))
    return out


def qa_col_absmax_workspace(K: int) -> int:
    return int(lib().qa_col_absmax_workspace(K))


def qa_col_absmax(A, colmax=None, accumulate=False, scratch=None, stream=None):
    """Column absolute maxima of A fp16 [rows x K] -> colmax f32 [K] (maxed into
    the given colmax when accumulate)."""
    _dev(A, "A", torch.float16)
    rows, K = A.shape
    if colmax is None:
        if accumulate:
            raise ValueError("accumulate needs the running colmax")
        colmax = _empty(stream, K, dtype=torch.float32, device=A.device)
    _dev(colmax, "colmax", torch.float32)
    scratch = _workspace(stream, qa_col_absmax_workspace(K), A.device, scratch)
    _check("qa_col_absmax", lib().qa_col_absmax(_p(A), rows, K, _p(colmax), int(bool(accumulate)), _p(scratch),
                                                 scratch.numel(), _stream(stream)))
    return colmax


def qa_smooth_factors(act_absmax, w_absmax, alpha=0.5, stream=None):
    """SmoothQuant migration factors -> s f32 [K]."""
    _dev(act_absmax, "act_absmax", torch.float32)
    _dev(w_absmax, "w_absmax", torch.float32)
    K = act_absmax.numel()
    if w_absmax.numel() != K:
        raise ValueError("act_absmax and w_absmax differ in length")
    s = _empty(stream, K, dtype=torch.float32, device=act_absmax.device)
    _check("qa_smooth_factors", lib().qa_smooth_factors(_p(act_absmax), _p(w_absmax), K, float(alpha), _p(s),
                                                         _stream(stream)))
    return s


def qa_quantize_smooth_int8(A, s, multiply=False, per_tensor=False, stream=None):
    """Smoothing (A / s, or A * s for a weight) + int8 absmax codes -> (q i8 [rows x K], s_out f32 [rows])."""
    _dev(A, "A", torch.float16)
    _dev(s, "s", torch.float32)
    rows, K = A.shape
    q = _empty(stream, (rows, K), dtype=torch.int8, device=A.device)
    s_out = _empty(stream, rows, dtype=torch.float32, device=A.device)
    _check("qa_quantize_smooth_int8",
           lib().qa_quantize_smooth_int8(_p(A), rows, K, _p(s), QA_SMOOTH_MULTIPLY if multiply else QA_SMOOTH_DIVIDE,
                                         QA_SCALE_PER_TENSOR if per_tensor else QA_SCALE_PER_ROW, _p(q), _p(s_out),
                                         _stream(stream)))
    return q, s_out


def qa_qlinear_int8_smooth_workspace(M: int, K: int) -> int:
    return int(lib().qa_qlinear_int8_smooth_workspace(M, K))


def qa_qlinear_int8_smooth(X, s, Wq, s_w, per_tensor=False, out_dtype=torch.float16, out=None, workspace=None,
                           stream=None):
    """SmoothQuant W8A8 linear -> out [M x N] of out_dtype."""
    _dev(X, "X", torch.float16)
    _dev(s, "s", torch.float32)
    _dev(Wq, "Wq", torch.int8)
    _dev(s_w, "s_w", torch.float32)
    M, K = X.shape
    N = Wq.shape[0]
    if out is None:
        out = _empty(stream, (M, N), dtype=out_dtype, device=X.device)
    workspace = _workspace(stream, qa_qlinear_int8_smooth_workspace(M, K), X.device, workspace)
    _check("qa_qlinear_int8_smooth",
           lib().qa_qlinear_int8_smooth(_p(X), M, K, _p(s), QA_SCALE_PER_TENSOR if per_tensor else QA_SCALE_PER_ROW,
                                        _p(Wq), _p(s_w), N, _p(out), _DTYPE_CODE[out.dtype], _p(workspace),
                                        workspace.numel(), _stream(stream)))
    return out


def qa_qlinear_int8_topk_workspace(M: int, K: int) -> int:
    return int(lib().qa_qlinear_int8_topk_workspace(M, K))


def qa_qlinear_int8_topk(X, Wq, s_w, k: int, W16=None, out_dtype=torch.float16, out=None, workspace=None,
                         stream=None):
    """LLM.int8() linear with the top-k columns decomposed -> out [M x N] of out_dtype."""
    _dev(X, "X", torch.float16)
    _dev(Wq, "Wq", torch.int8)
    _dev(s_w, "s_w", torch.float32)
    if W16 is not None:
        _dev(W16, "W16", torch.float16)
    M, K = X.shape
    N = Wq.shape[0]
    if out is None:
        out = _empty(stream, (M, N), dtype=out_dtype, device=X.device)
    workspace = _workspace(stream, qa_qlinear_int8_topk_workspace(M, K), X.device, workspace)
    _check("qa_qlinear_int8_topk",
           lib().qa_qlinear_int8_topk(_p(X), M, K, int(k), _p(Wq), _p(s_w), _p(W16), N, _p(out),
                                      _DTYPE_CODE[out.dtype], _p(workspace), workspace.numel(), _stream(stream)))
    return out


def qa_hadamard_quant_int4(X, G: int, per_group: bool, q_min=-7, q_max=7, stream=None):
    """-> (packed u32 as int32 [rows x K/8], s f32 [rows x (K/G if per_group else 1)])."""
    _dev(X, "X", torch.float16)
    rows, K = X.shape
    packed = _empty(stream, (rows, K // 8), dtype=torch.int32, device=X.device)
    s = _empty(stream, (rows, K // G if per_group else 1), dtype=torch.float32, device=X.device)
    _check("qa_hadamard_quant_int4",
           lib().qa_hadamard_quant_int4(_p(X), rows, K, int(G), QA_SCALE_PER_GROUP if per_group else QA_SCALE_PER_ROW,
                                        int(q_min), int(q_max), _p(packed), _p(s), _stream(stream)))
    return packed, s


def qa_kron_sizes(n: int):
    """-> (n1, n2, has_kernel): n1 n2 = n, n1 <= n2, n1 + n2 smallest; has_kernel
    tells whether the Kronecker entry points take that pair."""
    n1, n2, hk = ctypes.c_int64(0), ctypes.c_int64(0), ctypes.c_int32(0)
    _check("qa_kron_sizes", lib().qa_kron_sizes(int(n), ctypes.byref(n1), ctypes.byref(n2), ctypes.byref(hk)))
    return n1.value, n2.value, bool(hk.value)


def qa_kron_quant_int4(X, P1, P2, G=None, q_min=-7, q_max=7, stream=None):
    """Kronecker transform P1^T X~ P2 of each row + int4 codes -> (packed u32 as int32 [rows x K/8],
    s f32 [rows x (K/G if G else 1)])."""
    _dev(X, "X", torch.float16)
    _dev(P1, "P1", torch.float32)
    _dev(P2, "P2", torch.float32)
    rows, K = X.shape
    n1, n2 = P1.shape[0], P2.shape[0]
    packed = _empty(stream, (rows, K // 8), dtype=torch.int32, device=X.device)
    s = _empty(stream, (rows, K // G if G else 1), dtype=torch.float32, device=X.device)
    _check("qa_kron_quant_int4",
           lib().qa_kron_quant_int4(_p(X), rows, K, n1, n2, _p(P1), _p(P2),
                                    QA_SCALE_PER_GROUP if G else QA_SCALE_PER_ROW, int(G or 0), int(q_min), int(q_max),
                                    _p(packed), _p(s), _stream(stream)))
    return packed, s


def qa_qlinear_kron_w4a4_workspace(M: int, K: int) -> int:
    return int(lib().qa_qlinear_kron_w4a4_workspace(M, K))


def qa_qlinear_kron_w4a4(X, P1, P2, Wp, s_w, G=128, out_dtype=torch.float32, out=None, workspace=None, stream=None):
    """W4A4 linear with the Kronecker transform of X -> out [M x N]."""
    _dev(X, "X", torch.float16)
    _dev(P1, "P1", torch.float32)
    _dev(P2, "P2", torch.float32)
    _dev(Wp, "Wp", torch.int32)
    _dev(s_w, "s_w", torch.float32)
    M, K = X.shape
    N = Wp.shape[0]
    if out is None:
        out = _empty(stream, (M, N), dtype=out_dtype, device=X.device)
    workspace = _workspace(stream, qa_qlinear_kron_w4a4_workspace(M, K), X.device, workspace)
    _check("qa_qlinear_kron_w4a4",
           lib().qa_qlinear_kron_w4a4(_p(X), M, K, P1.shape[0], P2.shape[0], _p(P1), _p(P2), _p(Wp), _p(s_w), N,
                                      int(G), _p(out), _DTYPE_CODE[out.dtype], _p(workspace), workspace.numel(),
                                      _stream(stream)))
    return out


def qa_qlinear_w4a4_workspace(M: int, K: int) -> int:
    return int(lib().qa_qlinear_w4a4_workspace(M, K))


def qa_qlinear_w4a4(X, Wp, s_w, G=128, out_dtype=torch.float32, out=None, workspace=None, stream=None):
    """W4A4 group-Hadamard linear -> out [M x N]."""
    _dev(X, "X", torch.float16)
    _dev(Wp, "Wp", torch.int32)
    _dev(s_w, "s_w", torch.float32)
    M, K = X.shape
    N = Wp.shape[0]
    if out is None:
        out = _empty(stream, (M, N), dtype=out_dtype, device=X.device)
    workspace = _workspace(stream, qa_qlinear_w4a4_workspace(M, K), X.device, workspace)
    _check("qa_qlinear_w4a4",
           lib().qa_qlinear_w4a4(_p(X), M, K, _p(Wp), _p(s_w), N, int(G), _p(out), _DTYPE_CODE[out.dtype],
                                 _p(workspace), workspace.numel(), _stream(stream)))
    return out


def qa_hadamard_quant_int8(X, G: int, q_min=-127, q_max=127, stream=None):
    """Hadamard rotation + per-row int8 codes -> (q i8 [rows x K], s f32 [rows])."""
    _dev(X, "X", torch.float16)
    rows, K = X.shape
    q = _empty(stream, (rows, K), dtype=torch.int8, device=X.device)
    s = _empty(stream, rows, dtype=torch.float32, device=X.device)
    _check("qa_hadamard_quant_int8",
           lib().qa_hadamard_quant_int8(_p(X), rows, K, int(G), int(q_min), int(q_max), _p(q), _p(s),
                                        _stream(stream)))
    return q, s


def qa_qlinear_w4a8_workspace(M: int, K: int) -> int:
    return int(lib().qa_qlinear_w4a8_workspace(M, K))


def qa_qlinear_w4a8(X, Wp, s_w, G=128, out_dtype=torch.float32, out=None, workspace=None, stream=None):
    """W4A8 group-Hadamard linear (int8 activations, offline int4 weight) -> out [M x N]."""
    _dev(X, "X", torch.float16)
    _dev(Wp, "Wp", torch.int32)
    _dev(s_w, "s_w", torch.float32)
    M, K = X.shape
    N = Wp.shape[0]
    if out is None:
        out = _empty(stream, (M, N), dtype=out_dtype, device=X.device)
    workspace = _workspace(stream, qa_qlinear_w4a8_workspace(M, K), X.device, workspace)
    _check("qa_qlinear_w4a8",
           lib().qa_qlinear_w4a8(_p(X), M, K, _p(Wp), _p(s_w), N, int(G), _p(out), _DTYPE_CODE[out.dtype],
                                 _p(workspace), workspace.numel(), _stream(stream)))
    return out


def qa_hadamard_quant_int4_asym(X, G: int, stream=None):
    """Hadamard rotation + zero-point int4 codes per row -> (packed u32 as int32 [rows x K/8] holding q - 8,
    s f32 [rows], z i32 [rows])."""
    _dev(X, "X", torch.float16)
    rows, K = X.shape
    packed = _empty(stream, (rows, K // 8), dtype=torch.int32, device=X.device)
    s = _empty(stream, rows, dtype=torch.float32, device=X.device)
    z = _empty(stream, rows, dtype=torch.int32, device=X.device)
    _check("qa_hadamard_quant_int4_asym",
           lib().qa_hadamard_quant_int4_asym(_p(X), rows, K, int(G), _p(packed), _p(s), _p(z), _stream(stream)))
    return packed, s, z


def qa_w4_column_terms(Wp, s_w, K: int, G: int, stream=None):
    """c[n] = sum_g s_w[n][g] * sum_{k in g} qw[n][k] of a per-group int4 weight -> f32 [N]."""
    _dev(Wp, "Wp", torch.int32)
    _dev(s_w, "s_w", torch.float32)
    N = Wp.shape[0]
    c = _empty(stream, N, dtype=torch.float32, device=Wp.device)
    _check("qa_w4_column_terms", lib().qa_w4_column_terms(_p(Wp), _p(s_w), N, int(K), int(G), _p(c), _stream(stream)))
    return c


def qa_qlinear_w4a4_asym_workspace(M: int, K: int) -> int:
    return int(lib().qa_qlinear_w4a4_asym_workspace(M, K))


def qa_qlinear_w4a4_asym(X, Wp, s_w, c_w, G=128, out_dtype=torch.float32, out=None, workspace=None, stream=None):
    """W4A4 group-Hadamard linear with zero-point int4 activations -> out [M x N]."""
    _dev(X, "X", torch.float16)
    _dev(Wp, "Wp", torch.int32)
    _dev(s_w, "s_w", torch.float32)
    _dev(c_w, "c_w", torch.float32)
    M, K = X.shape
    N = Wp.shape[0]
    if out is None:
        out = _empty(stream, (M, N), dtype=out_dtype, device=X.device)
    workspace = _workspace(stream, qa_qlinear_w4a4_asym_workspace(M, K), X.device, workspace)
    _check("qa_qlinear_w4a4_asym",
           lib().qa_qlinear_w4a4_asym(_p(X), M, K, _p(Wp), _p(s_w), _p(c_w), N, int(G), _p(out),
                                      _DTYPE_CODE[out.dtype], _p(workspace), workspace.numel(), _stream(stream)))
    return out


def qa_gemm_i8_i32(A, B, stream=None):
    _dev(A, "A", torch.int8)
    _dev(B, "B", torch.int8)
    M, K = A.shape
    N = B.shape[0]
    C = _empty(stream, (M, N), dtype=torch.int32, device=A.device)
    _check("qa_gemm_i8_i32", lib().qa_gemm_i8_i32(_p(A), _p(B), M, K, N, _p(C), _stream(stream)))
    return C


def qa_gemm_w4a4_group_acc(Xp, Wp, K: int, G: int, stream=None):
    _dev(Xp, "Xp", torch.int32)
    _dev(Wp, "Wp", torch.int32)
    M, N = Xp.shape[0], Wp.shape[0]
    acc = _empty(stream, (M, N, K // G), dtype=torch.int32, device=Xp.device)
    _check("qa_gemm_w4a4_group_acc",
           lib().qa_gemm_w4a4_group_acc(_p(Xp), _p(Wp), M, K, N, int(G), _p(acc), _stream(stream)))
    return acc


def qa_gemm_w4a8_group_acc(Xq, Wp, G: int, stream=None):
    _dev(Xq, "Xq", torch.int8)
    _dev(Wp, "Wp", torch.int32)
    M, K = Xq.shape
    N = Wp.shape[0]
    acc = _empty(stream, (M, N, K // G), dtype=torch.int32, device=Xq.device)
    _check("qa_gemm_w4a8_group_acc",
           lib().qa_gemm_w4a8_group_acc(_p(Xq), _p(Wp), M, K, N, int(G), _p(acc), _stream(stream)))
    return acc


def qa_probe_stream_read(src, nbytes: int, wgs: int, lane_bytes: int = 16, unroll: int = 4, sink=None, stream=None):
    """Measurement helper: read src[0 .. nbytes) once (the single-launch HBM read floor)."""
    _dev(src, "src", None)
    if sink is None:
        sink = _empty(stream, (int(wgs) * 512,), dtype=torch.int32, device=src.device)
    _check("qa_probe_stream_read",
           lib().qa_probe_stream_read(_p(src), int(nbytes), int(wgs), int(lane_bytes), int(unroll), _p(sink),
                                      _stream(stream)))
    return sink

