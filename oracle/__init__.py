"""CPU oracle for the quantized linear layer -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may import this package.  It wraps ``liboracle.so`` (plain C, built from
``oracle.c`` with gcc, no fast-math, no FP contraction) with numpy marshalling.
It shares no code with the GPU library ``bit_quantized_linear_int8_amd``.

Every function follows the page passages cited in ``oracle.c``:
LLM.int8() (AIInfra 05Quantization01; Quantization explained part 2, §1.2),
scale / zero-point / group granularity (模型推理量化 §4-§7), the group
Hadamard W4A4 scheme (分组旋转方法从W8A8到W4A4, §二, §5.1-§5.4) and the
SmoothQuant migration (Quantization explained part 2, §4.2), zero-point
quantization (模型推理量化 §6) and the FlatQuant Kronecker transform (AIInfra
05Quantization01, FlatQuant section).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, F16, BF16 = 0, 1, 2

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
          "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (always when ``force``)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        P, I64, I32, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
        sig = {
            "orc_f16_to_f64": (ctypes.c_double, [ctypes.c_uint16]),
            "orc_f64_to_f16": (ctypes.c_uint16, [ctypes.c_double]),
            "orc_f64_to_bf16": (ctypes.c_uint16, [ctypes.c_double]),
            "orc_round_output": (None, [P, I64, ctypes.c_int, P]),
            "orc_f16_to_f32_array": (None, [P, I64, P]),
            "orc_outlier_cols": (None, [P, I64, I64, F, P, P, P, P]),
            "orc_quant_rows_f32": (None, [P, I64, I64, I64, P, I32, I32, P, P, P, P]),
            "orc_quant_rows_f16": (None, [P, I64, I64, I64, P, I32, I32, P, P, P, P]),
            "orc_gemm_i8_i32": (I64, [P, P, I64, I64, I64, P, I64, P]),
            "orc_qlinear_int8_mixed": (None, [P, I64, I64, P, P, P, I64, F, P, I64, P]),
            "orc_outlier_topk": (None, [P, I64, I64, I64, P, P, P, P]),
            "orc_qlinear_int8_topk": (None, [P, I64, I64, P, P, P, I64, I64, P, I64, P]),
            "orc_kron_sizes": (None, [I64, P, P]),
            "orc_kron_transform_f32": (None, [P, I64, I64, I64, P, P, P]),
            "orc_kron_quant_int4": (None, [P, I64, I64, I64, I64, P, P, I64, I32, I32, P, P]),
            "orc_qlinear_kron_w4a4": (None, [P, I64, I64, I64, I64, P, P, P, P, I64, I32, P, I64, P]),
            "orc_minmax_params": (None, [P, I64, I32, I32, P, P]),
            "orc_quant_rows_asym_f32": (None, [P, I64, I64, I32, I32, P, P, P, P]),
            "orc_qlinear_int8_asym": (None, [P, I64, I64, P, P, P, I64, P, I64, P]),
            "orc_col_absmax_f32": (None, [P, I64, I64, P]),
            "orc_smooth_factors": (None, [P, P, I64, ctypes.c_double, P]),
            "orc_smooth_apply_f32": (None, [P, I64, I64, P, ctypes.c_int, P]),
            "orc_smooth_quant_f32": (None, [P, I64, I64, P, ctypes.c_int, ctypes.c_int, P, P]),
            "orc_qlinear_int8_smooth": (None, [P, I64, I64, P, ctypes.c_int, P, P, I64, P, I64, P]),
            "orc_hadamard_entry": (ctypes.c_int, [I32, I32]),
            "orc_hadamard_rows": (None, [P, I64, I64, I32, P]),
            "orc_pack_int4": (None, [P, I64, I64, P]),
            "orc_unpack_int4": (None, [P, I64, I64, P]),
            "orc_hadamard_quant_int4": (None, [P, I64, I64, I32, ctypes.c_int, I32, I32, P, P]),
            "orc_w4a4_group_acc": (I64, [P, P, I64, I64, I64, I32, P, I64, P]),
            "orc_qlinear_w4a4": (None, [P, I64, I64, P, P, I64, I32, P, I64, P]),
            "orc_hadamard_quant_int8": (None, [P, I64, I64, I32, I32, I32, P, P]),
            "orc_w4a8_group_acc": (I64, [P, P, I64, I64, I64, I32, P, I64, P]),
            "orc_qlinear_w4a8": (None, [P, I64, I64, P, P, I64, I32, P, I64, P]),
            "orc_hadamard_quant_int4_asym": (None, [P, I64, I64, I32, P, P, P]),
            "orc_qlinear_w4a4_asym": (None, [P, I64, I64, P, P, I64, I32, P, I64, P]),
            "orc_w4_column_terms": (None, [P, P, I64, I64, I32, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _h16(x):
    """fp16 array -> its uint16 bit patterns."""
    return np.ascontiguousarray(x, dtype=np.float16).view(np.uint16)


def _rows(rows):
    if rows is None:
        return None, 0
    r = np.ascontiguousarray(rows, dtype=np.int64)
    return r, int(r.size)


# ---------------------------------------------------------------- formats
def f16_to_f64(bits: int) -> float:
    return lib().orc_f16_to_f64(int(bits))


def f64_to_f16_bits(v: float) -> int:
    return int(lib().orc_f64_to_f16(float(v)))


def f64_to_bf16_bits(v: float) -> int:
    return int(lib().orc_f64_to_bf16(float(v)))


def round_output(x64: np.ndarray, dtype: int) -> np.ndarray:
    """fp64 results -> fp32 array, or uint16 bit patterns for fp16 / bf16."""
    x = _c(x64, np.float64)
    out = np.empty(x.shape, np.float32 if dtype == F32 else np.uint16)
    lib().orc_round_output(_ptr(x), x.size, dtype, _ptr(out))
    return out


def f16_to_f32(x16) -> np.ndarray:
    h = _h16(x16)
    out = np.empty(h.shape, np.float32)
    lib().orc_f16_to_f32_array(_ptr(h), h.size, _ptr(out))
    return out


# ---------------------------------------------------------------- int8 path
def outlier_cols(X16, tau: float):
    """-> (mask u8 [K], idx i32 [count] ascending, colmax f32 [K])."""
    h = _h16(X16)
    M, K = h.shape
    mask = np.zeros(K, np.uint8)
    idx = np.zeros(max(K, 1), np.int32)
    count = np.zeros(1, np.int32)
    colmax = np.zeros(K, np.float32)
    lib().orc_outlier_cols(_ptr(h), M, K, float(tau), _ptr(mask), _ptr(idx), _ptr(count), _ptr(colmax))
    return mask, idx[: int(count[0])].copy(), colmax


def outlier_topk(X16, k: int):
    """The k columns of largest max |x| (ties: lower column first)
    -> (mask u8 [K], idx i32 [count] ascending, colmax f32 [K])."""
    h = _h16(X16)
    M, K = h.shape
    mask = np.zeros(K, np.uint8)
    idx = np.zeros(max(K, 1), np.int32)
    count = np.zeros(1, np.int32)
    colmax = np.zeros(K, np.float32)
    lib().orc_outlier_topk(_ptr(h), M, K, int(k), _ptr(mask), _ptr(idx), _ptr(count), _ptr(colmax))
    return mask, idx[: int(count[0])].copy(), colmax


def qlinear_int8_topk(X16, Wq, s_w, W16=None, k=0, rows=None):
    """LLM.int8() linear with the top-k columns decomposed, fp64 [nrows x N]."""
    h = _h16(X16)
    M, K = h.shape
    Wq = _c(Wq, np.int8)
    N = Wq.shape[0]
    sw = _c(s_w, np.float32)
    w16 = None if W16 is None else _h16(W16)
    r, nr = _rows(rows)
    out = np.zeros((nr if r is not None else M, N), np.float64)
    lib().orc_qlinear_int8_topk(_ptr(h), M, K, _ptr(Wq), _ptr(sw), _ptr(w16), N, int(k), _ptr(r), nr, _ptr(out))
    return out


def quant_rows(x, gsize=None, mask=None, qmin=-127, qmax=127, s_in=None, z_in=None):
    """Quantize rows of x (fp16 or fp32 array [rows x K]).  Returns (codes i8, scales f32|None)."""
    x = np.asarray(x)
    if x.ndim == 1:
        x = x[None, :]
    rows, K = x.shape
    g = K if gsize is None else int(gsize)
    q = np.zeros((rows, K), np.int8)
    s_out = None if s_in is not None else np.zeros((rows, K // g), np.float32)
    m = None if mask is None else _c(mask, np.uint8)
    si = None if s_in is None else _c(s_in, np.float32)
    zi = None if z_in is None else _c(z_in, np.int32)
    if x.dtype == np.float16:
        h = _h16(x)
        lib().orc_quant_rows_f16(_ptr(h), rows, K, g, _ptr(m), qmin, qmax, _ptr(si), _ptr(zi), _ptr(q), _ptr(s_out))
    else:
        xf = _c(x, np.float32)
        lib().orc_quant_rows_f32(_ptr(xf), rows, K, g, _ptr(m), qmin, qmax, _ptr(si), _ptr(zi), _ptr(q), _ptr(s_out))
    return q, s_out


def gemm_i8_i32(A, B, rows=None):
    """C = A @ B.T with int64 sums stored as int32 ([nrows x N])."""
    A = _c(A, np.int8)
    B = _c(B, np.int8)
    M, K = A.shape
    N = B.shape[0]
    r, nr = _rows(rows)
    C = np.zeros((nr if r is not None else M, N), np.int32)
    bad = lib().orc_gemm_i8_i32(_ptr(A), _ptr(B), M, K, N, _ptr(r), nr, _ptr(C))
    if bad:
        raise OverflowError("int32 accumulator overflow in %d results" % bad)
    return C


def qlinear_int8_mixed(X16, Wq, s_w, W16=None, tau=6.0, rows=None):
    """LLM.int8() mixed linear in fp64: [nrows x N] (all rows if rows is None)."""
    h = _h16(X16)
    M, K = h.shape
    Wq = _c(Wq, np.int8)
    N = Wq.shape[0]
    sw = _c(s_w, np.float32)
    w16 = None if W16 is None else _h16(W16)
    r, nr = _rows(rows)
    out = np.zeros((nr if r is not None else M, N), np.float64)
    lib().orc_qlinear_int8_mixed(_ptr(h), M, K, _ptr(Wq), _ptr(sw), _ptr(w16), N, float(tau),
                                 _ptr(r), nr, _ptr(out))
    return out


# ---------------------------------------------------------------- Kronecker transform (FlatQuant apply side)
def kron_sizes(n: int):
    """(n1, n2) with n1 n2 = n, n1 <= n2, n1 + n2 smallest."""
    a = np.zeros(1, np.int64)
    b = np.zeros(1, np.int64)
    lib().orc_kron_sizes(int(n), _ptr(a), _ptr(b))
    return int(a[0]), int(b[0])


def kron_transform(x, P1, P2):
    """Rows of x (fp16 or fp32, [rows x n1 n2]) -> fp32 rows of P1^T X~ P2."""
    a = _f32_matrix(x)
    rows, n = a.shape
    p1 = _c(P1, np.float32)
    p2 = _c(P2, np.float32)
    n1, n2 = p1.shape[0], p2.shape[0]
    assert n1 * n2 == n
    out = np.zeros((rows, n), np.float32)
    lib().orc_kron_transform_f32(_ptr(a), rows, n1, n2, _ptr(p1), _ptr(p2), _ptr(out))
    return out


def kron_quant_int4(X16, P1, P2, per_group_G=None, qmin=-7, qmax=7):
    """Transform + int4 codes + packing -> (packed u32 [rows x K/8], s f32 [rows x groups])."""
    h = _h16(X16)
    if h.ndim == 1:
        h = h[None, :]
    rows, K = h.shape
    p1 = _c(P1, np.float32)
    p2 = _c(P2, np.float32)
    g = K if per_group_G is None else int(per_group_G)
    packed = np.zeros((rows, K // 8), np.uint32)
    s = np.zeros((rows, K // g), np.float32)
    lib().orc_kron_quant_int4(_ptr(h), rows, K, p1.shape[0], p2.shape[0], _ptr(p1), _ptr(p2), g, int(qmin),
                              int(qmax), _ptr(packed), _ptr(s))
    return packed, s


def qlinear_kron_w4a4(X16, P1, P2, Wp, s_w, G=128, rows=None):
    """W4A4 linear with the Kronecker transform of X, fp64 [nrows x N]."""
    h = _h16(X16)
    M, K = h.shape
    p1 = _c(P1, np.float32)
    p2 = _c(P2, np.float32)
    wp = _c(Wp, np.uint32)
    sw = _c(s_w, np.float32)
    N = wp.shape[0]
    r, nr = _rows(rows)
    out = np.zeros((nr if r is not None else M, N), np.float64)
    lib().orc_qlinear_kron_w4a4(_ptr(h), M, K, p1.shape[0], p2.shape[0], _ptr(p1), _ptr(p2), _ptr(wp), _ptr(sw), N,
                                int(G), _ptr(r), nr, _ptr(out))
    return out


# ---------------------------------------------------------------- asymmetric (zero-point)
def minmax_params(x, qmin, qmax):
    """Min-max affine parameters of one vector -> (s f32, z int)."""
    xf = _c(np.asarray(x, np.float32).ravel(), np.float32)
    s = np.zeros(1, np.float32)
    z = np.zeros(1, np.int32)
    lib().orc_minmax_params(_ptr(xf), xf.size, int(qmin), int(qmax), _ptr(s), _ptr(z))
    return s[0], int(z[0])


def quant_rows_asym(x, qmin=-128, qmax=127):
    """Per-row asymmetric codes of an fp16 or fp32 matrix -> (codes i8, s f32 [rows], z i32 [rows],
    row sums of the codes i32 [rows])."""
    a = _f32_matrix(x)
    rows, K = a.shape
    q = np.zeros((rows, K), np.int8)
    s = np.zeros(rows, np.float32)
    z = np.zeros(rows, np.int32)
    rs = np.zeros(rows, np.int32)
    lib().orc_quant_rows_asym_f32(_ptr(a), rows, K, int(qmin), int(qmax), _ptr(q), _ptr(s), _ptr(z), _ptr(rs))
    return q, s, z, rs


def qlinear_int8_asym(X16, Wq, s_w, z_w=None, rows=None):
    """W8A8 linear with asymmetric per-token activations, fp64 [nrows x N]."""
    h = _h16(X16)
    M, K = h.shape
    Wq = _c(Wq, np.int8)
    N = Wq.shape[0]
    sw = _c(s_w, np.float32)
    zw = None if z_w is None else _c(z_w, np.int32)
    r, nr = _rows(rows)
    out = np.zeros((nr if r is not None else M, N), np.float64)
    lib().orc_qlinear_int8_asym(_ptr(h), M, K, _ptr(Wq), _ptr(sw), _ptr(zw), N, _ptr(r), nr, _ptr(out))
    return out


# ---------------------------------------------------------------- SmoothQuant
SMOOTH_DIVIDE, SMOOTH_MULTIPLY = 0, 1


def _f32_matrix(a):
    """fp16 (widened exactly) or fp32 matrix as contiguous fp32 [rows x K]."""
    a = np.asarray(a)
    if a.ndim == 1:
        a = a[None, :]
    return f16_to_f32(a) if a.dtype == np.float16 else _c(a, np.float32)


def col_absmax(A):
    """max_r |A[r, j]| per column of an fp16 or fp32 matrix -> f32 [K]."""
    a = _f32_matrix(A)
    rows, K = a.shape
    out = np.zeros(K, np.float32)
    lib().orc_col_absmax_f32(_ptr(a), rows, K, _ptr(out))
    return out


def smooth_factors(cx, cw, alpha=0.5):
    """Migration factors s_j = cx_j^alpha / cw_j^(1-alpha) (1 where a max is 0) -> f32 [K]."""
    cx = _c(cx, np.float32)
    cw = _c(cw, np.float32)
    s = np.zeros(cx.size, np.float32)
    lib().orc_smooth_factors(_ptr(cx), _ptr(cw), cx.size, float(alpha), _ptr(s))
    return s


def smooth_apply(A, s, op):
    """A / s (SMOOTH_DIVIDE, activations) or A * s (SMOOTH_MULTIPLY, weights) per column, fp32."""
    a = _f32_matrix(A)
    rows, K = a.shape
    sv = _c(s, np.float32)
    out = np.zeros((rows, K), np.float32)
    lib().orc_smooth_apply_f32(_ptr(a), rows, K, _ptr(sv), int(op), _ptr(out))
    return out


def smooth_quantize(A, s, op, per_tensor=False):
    """Smoothing + [-127, 127] absmax codes -> (codes i8 [rows x K], scales f32 [rows])."""
    a = _f32_matrix(A)
    rows, K = a.shape
    sv = _c(s, np.float32)
    q = np.zeros((rows, K), np.int8)
    s_out = np.zeros(rows, np.float32)
    lib().orc_smooth_quant_f32(_ptr(a), rows, K, _ptr(sv), int(op), int(bool(per_tensor)), _ptr(q), _ptr(s_out))
    return q, s_out


def qlinear_int8_smooth(X16, s, Wq, s_w, per_tensor=False, rows=None):
    """SmoothQuant W8A8 linear in fp64: [nrows x N] (all rows if rows is None)."""
    h = _h16(X16)
    M, K = h.shape
    sv = _c(s, np.float32)
    Wq = _c(Wq, np.int8)
    N = Wq.shape[0]
    sw = _c(s_w, np.float32)
    r, nr = _rows(rows)
    out = np.zeros((nr if r is not None else M, N), np.float64)
    lib().orc_qlinear_int8_smooth(_ptr(h), M, K, _ptr(sv), int(bool(per_tensor)), _ptr(Wq), _ptr(sw), N,
                                  _ptr(r), nr, _ptr(out))
    return out


# ---------------------------------------------------------------- W4A4 path
def hadamard_entry(i: int, j: int) -> int:
    return int(lib().orc_hadamard_entry(i, j))


def hadamard_rows(X16, G: int) -> np.ndarray:
    h = _h16(X16)
    if h.ndim == 1:
        h = h[None, :]
    rows, K = h.shape
    out = np.zeros((rows, K), np.float32)
    lib().orc_hadamard_rows(_ptr(h), rows, K, int(G), _ptr(out))
    return out


def pack_int4(q) -> np.ndarray:
    q = _c(q, np.int8)
    if q.ndim == 1:
        q = q[None, :]
    rows, K = q.shape
    out = np.zeros((rows, K // 8), np.uint32)
    lib().orc_pack_int4(_ptr(q), rows, K, _ptr(out))
    return out


def unpack_int4(p, K: int) -> np.ndarray:
    p = _c(p, np.uint32)
    if p.ndim == 1:
        p = p[None, :]
    rows = p.shape[0]
    out = np.zeros((rows, K), np.int8)
    lib().orc_unpack_int4(_ptr(p), rows, K, _ptr(out))
    return out


def hadamard_quant_int4(X16, G: int, per_group: bool, qmin=-7, qmax=7):
    """-> (packed u32 [rows x K/8], scales f32 [rows x (K/G if per_group else 1)])."""
    h = _h16(X16)
    if h.ndim == 1:
        h = h[None, :]
    rows, K = h.shape
    packed = np.zeros((rows, K // 8), np.uint32)
    s = np.zeros((rows, K // G if per_group else 1), np.float32)
    lib().orc_hadamard_quant_int4(_ptr(h), rows, K, int(G), 1 if per_group else 0, qmin, qmax,
                                  _ptr(packed), _ptr(s))
    return packed, s


def w4a4_group_acc(Xp, Wp, K: int, G: int, rows=None):
    Xp = _c(Xp, np.uint32)
    Wp = _c(Wp, np.uint32)
    M, N = Xp.shape[0], Wp.shape[0]
    r, nr = _rows(rows)
    acc = np.zeros((nr if r is not None else M, N, K // G), np.int32)
    bad = lib().orc_w4a4_group_acc(_ptr(Xp), _ptr(Wp), M, K, N, int(G), _ptr(r), nr, _ptr(acc))
    if bad:
        raise OverflowError("int32 accumulator overflow in %d results" % bad)
    return acc


def qlinear_w4a4(X16, Wp, s_w, G: int, rows=None):
    h = _h16(X16)
    M, K = h.shape
    Wp = _c(Wp, np.uint32)
    N = Wp.shape[0]
    sw = _c(s_w, np.float32)
    r, nr = _rows(rows)
    out = np.zeros((nr if r is not None else M, N), np.float64)
    lib().orc_qlinear_w4a4(_ptr(h), M, K, _ptr(Wp), _ptr(sw), N, int(G), _ptr(r), nr, _ptr(out))
    return out


# ---------------------------------------------------------------- W4A8 path
def hadamard_quant_int8(X16, G: int, qmin=-127, qmax=127):
    """-> (codes i8 [rows x K], per-row scales f32 [rows])."""
    h = _h16(X16)
    if h.ndim == 1:
        h = h[None, :]
    rows, K = h.shape
    q = np.zeros((rows, K), np.int8)
    s = np.zeros(rows, np.float32)
    lib().orc_hadamard_quant_int8(_ptr(h), rows, K, int(G), qmin, qmax, _ptr(q), _ptr(s))
    return q, s


def w4a8_group_acc(Xq, Wp, G: int, rows=None):
    Xq = _c(Xq, np.int8)
    Wp = _c(Wp, np.uint32)
    M, K = Xq.shape
    N = Wp.shape[0]
    r, nr = _rows(rows)
    acc = np.zeros((nr if r is not None else M, N, K // G), np.int32)
    bad = lib().orc_w4a8_group_acc(_ptr(Xq), _ptr(Wp), M, K, N, int(G), _ptr(r), nr, _ptr(acc))
    if bad:
        raise OverflowError("int32 accumulator overflow in %d results" % bad)
    return acc


def qlinear_w4a8(X16, Wp, s_w, G: int, rows=None):
    h = _h16(X16)
    M, K = h.shape
    Wp = _c(Wp, np.uint32)
    N = Wp.shape[0]
    sw = _c(s_w, np.float32)
    r, nr = _rows(rows)
    out = np.zeros((nr if r is not None else M, N), np.float64)
    lib().orc_qlinear_w4a8(_ptr(h), M, K, _ptr(Wp), _ptr(sw), N, int(G), _ptr(r), nr, _ptr(out))
    return out


# ---------------------------------------------------------------- W4A4, zero-point activations
def hadamard_quant_int4_asym(X16, G: int):
    """-> (packed u32 [rows x K/8] holding q - 8, s f32 [rows], z i32 [rows] in [0, 15])."""
    h = _h16(X16)
    if h.ndim == 1:
        h = h[None, :]
    rows, K = h.shape
    packed = np.zeros((rows, K // 8), np.uint32)
    s = np.zeros(rows, np.float32)
    z = np.zeros(rows, np.int32)
    lib().orc_hadamard_quant_int4_asym(_ptr(h), rows, K, int(G), _ptr(packed), _ptr(s), _ptr(z))
    return packed, s, z


def w4_column_terms(Wp, s_w, K: int, G: int):
    """c[n] = fl32(sum_g s_w[n][g] * sum_{k in g} qw[n][k]) (zero-point term, per output column)."""
    Wp = _c(Wp, np.uint32)
    N = Wp.shape[0]
    sw = _c(s_w, np.float32)
    c = np.zeros(N, np.float32)
    lib().orc_w4_column_terms(_ptr(Wp), _ptr(sw), N, int(K), int(G), _ptr(c))
    return c


def qlinear_w4a4_asym(X16, Wp, s_w, G: int, rows=None):
    h = _h16(X16)
    M, K = h.shape
    Wp = _c(Wp, np.uint32)
    N = Wp.shape[0]
    sw = _c(s_w, np.float32)
    r, nr = _rows(rows)
    out = np.zeros((nr if r is not None else M, N), np.float64)
    lib().orc_qlinear_w4a4_asym(_ptr(h), M, K, _ptr(Wp), _ptr(sw), N, int(G), _ptr(r), nr, _ptr(out))
    return out
