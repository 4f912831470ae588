"""The C ABI on the CPU: libqa.so loads, exports every entry point that
include/qa.h declares, and rejects bad arguments before any HIP call (so no
GPU is needed: nothing here launches a kernel)."""
import ctypes
import math
import os
import re

import pytest

import bit_quantized_linear_int8_amd as qa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qa.h")

OK, NULL, SHAPE, ALIGN, VALUE, WORKSPACE, UNSUPPORTED = 0, 1, 2, 3, 4, 5, 6

# fake, suitably aligned device addresses: validation never dereferences them
A = ctypes.c_void_p(0x10000)
B = ctypes.c_void_p(0x20000)
OUT = ctypes.c_void_p(0x30000)
WS = ctypes.c_void_p(0x40000)
MIS = ctypes.c_void_p(0x10001)        # misaligned


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(qa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(qa.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(qa.LIB_PATH)
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings():
    L = qa.lib()
    names = [L.qa_status_string(i).decode() for i in range(8)]
    assert names == ["QA_OK", "QA_ERR_NULL", "QA_ERR_SHAPE", "QA_ERR_ALIGN", "QA_ERR_VALUE", "QA_ERR_WORKSPACE",
                     "QA_ERR_UNSUPPORTED", "QA_ERR_DEVICE"]


def test_workspace_sizes_are_monotone_and_cover_the_buffers():
    L = qa.lib()
    for M, K in [(1, 16), (16, 256), (2048, 4096)]:
        ws = L.qa_qlinear_int8_mixed_workspace(M, K)
        assert ws >= M * K + 4 * M + 5 * K + 4
        assert ws % 256 == 0
        assert L.qa_qlinear_w4a4_workspace(M, K) >= M * K // 2 + 4 * M
    assert L.qa_qlinear_int8_mixed_workspace(-1, 16) == 0
    assert L.qa_outlier_cols_workspace(0) == 0


def mixed(**kw):
    a = dict(X=A, M=16, K=256, Wq=B, s_w=OUT, W16=None, N=32, tau=6.0, out=OUT, dt=1, ws=WS, wsb=1 << 30)
    a.update(kw)
    return qa.lib().qa_qlinear_int8_mixed(a["X"], a["M"], a["K"], a["Wq"], a["s_w"], a["W16"], a["N"], a["tau"],
                                          a["out"], a["dt"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(X=None), NULL), (dict(Wq=None), NULL), (dict(s_w=None), NULL), (dict(out=None), NULL),
    (dict(ws=None), NULL),
    (dict(M=-1), SHAPE), (dict(N=-1), SHAPE), (dict(K=0), SHAPE), (dict(K=24), SHAPE), (dict(K=131088), SHAPE),
    (dict(X=MIS), ALIGN), (dict(Wq=MIS), ALIGN), (dict(ws=ctypes.c_void_p(0x40010)), ALIGN),
    (dict(tau=math.nan), VALUE), (dict(dt=3), VALUE), (dict(dt=-1), VALUE),
    (dict(wsb=100), WORKSPACE),
    (dict(M=0), OK), (dict(N=0), OK),          # empty batch / layer: valid no-ops
])
def test_mixed_argument_errors(kw, status):
    assert mixed(**kw) == status
    if status != OK:
        assert qa.last_error()


def test_quantize_argument_errors():
    f = qa.lib().qa_quantize_rowwise_int8
    assert f(None, 4, 64, None, -127, 127, None, None, B, OUT, None) == NULL
    assert f(A, 4, 64, None, -127, 127, None, None, B, None, None) == NULL          # dynamic needs s_out
    assert f(A, 4, 60, None, -127, 127, None, None, B, OUT, None) == SHAPE
    assert f(A, -4, 64, None, -127, 127, None, None, B, OUT, None) == SHAPE
    assert f(A, 4, (1 << 26) + 8, None, -127, 127, None, None, B, OUT, None) == SHAPE
    assert f(MIS, 4, 64, None, -127, 127, None, None, B, OUT, None) == ALIGN
    assert f(A, 4, 64, None, 5, 4, None, None, B, OUT, None) == VALUE
    assert f(A, 4, 64, None, -129, 127, None, None, B, OUT, None) == VALUE
    assert f(A, 4, 64, None, -127, 0, None, None, B, OUT, None) == VALUE             # dynamic q_max <= 0
    assert f(A, 4, 64, None, -127, 127, None, WS, B, OUT, None) == VALUE             # z without s
    assert f(A, 0, 64, None, -127, 127, None, None, B, OUT, None) == OK


def test_outlier_argument_errors():
    f = qa.lib().qa_outlier_cols
    args = [A, 16, 256, 6.0, B, OUT, WS, None, WS, 1 << 20, None]

    def call(i, v):
        a = list(args)
        a[i] = v
        return f(*a)
    assert call(0, None) == NULL
    assert call(8, None) == NULL
    assert call(2, 12) == SHAPE
    assert call(1, -1) == SHAPE
    assert call(0, MIS) == ALIGN
    assert call(3, math.nan) == VALUE
    assert call(9, 16) == WORKSPACE


def test_hadamard_argument_errors():
    f = qa.lib().qa_hadamard_quant_int4
    assert f(None, 4, 256, 128, 0, -7, 7, B, OUT, None) == NULL
    assert f(A, 4, 256, 96, 0, -7, 7, B, OUT, None) == SHAPE          # not a power of two
    assert f(A, 4, 256, 512, 0, -7, 7, B, OUT, None) == SHAPE         # too large
    assert f(A, 4, 200, 16, 0, -7, 7, B, OUT, None) == SHAPE          # K % G
    assert f(A, 4, 256, 4, 1, -7, 7, B, OUT, None) == SHAPE           # per group needs G >= 8
    assert f(A, 4, 256, 128, 2, -7, 7, B, OUT, None) == VALUE         # bad mode
    assert f(A, 4, 256, 128, 0, -9, 7, B, OUT, None) == VALUE
    assert f(A, 4, 256, 128, 0, -7, 8, B, OUT, None) == VALUE
    assert f(MIS, 4, 256, 128, 0, -7, 7, B, OUT, None) == ALIGN
    assert f(A, 0, 256, 128, 0, -7, 7, B, OUT, None) == OK


def test_w4a4_argument_errors():
    f = qa.lib().qa_qlinear_w4a4
    base = [A, 16, 512, B, OUT, 32, 128, OUT, 0, WS, 1 << 30, None]

    def call(i, v):
        a = list(base)
        a[i] = v
        return f(*a)
    assert call(0, None) == NULL
    assert call(6, 4) == SHAPE                                 # G below 8
    assert call(6, 48) == SHAPE                                # not a power of two
    assert call(6, 512) == SHAPE
    assert call(2, 320) == SHAPE
    assert call(3, MIS) == ALIGN
    assert call(8, 7) == VALUE
    assert call(10, 64) == WORKSPACE
    g = qa.lib().qa_gemm_w4a4_group_acc
    assert g(A, B, 4, 512, 4, 100, OUT, None) == SHAPE
    assert g(A, None, 4, 512, 4, 128, OUT, None) == NULL


def test_w4a8_argument_errors():
    h = qa.lib().qa_hadamard_quant_int8
    assert h(None, 4, 256, 128, -127, 127, B, OUT, None) == NULL
    assert h(A, 4, 256, 96, -127, 127, B, OUT, None) == SHAPE           # not a power of two
    assert h(A, 4, 200, 16, -127, 127, B, OUT, None) == SHAPE           # K % G
    assert h(A, 4, 260, 4, -127, 127, B, OUT, None) == SHAPE            # K % 8
    assert h(A, 4, 256, 128, -129, 127, B, OUT, None) == VALUE
    assert h(A, 4, 256, 128, -127, 128, B, OUT, None) == VALUE
    assert h(A, 4, 256, 128, 5, 4, B, OUT, None) == VALUE
    assert h(MIS, 4, 256, 128, -127, 127, B, OUT, None) == ALIGN
    assert h(A, 4, 256, 128, -127, 127, ctypes.c_void_p(0x20004), OUT, None) == ALIGN   # q 8-byte
    assert h(A, 0, 256, 128, -127, 127, B, OUT, None) == OK
    f = qa.lib().qa_qlinear_w4a8
    base = [A, 16, 512, B, OUT, 32, 128, OUT, 0, WS, 1 << 30, None]

    def call(i, v):
        a = list(base)
        a[i] = v
        return f(*a)
    assert call(0, None) == NULL
    assert call(9, None) == NULL
    assert call(6, 4) == SHAPE
    assert call(6, 24) == SHAPE
    assert call(2, 320) == SHAPE
    assert call(3, MIS) == ALIGN
    assert call(8, 7) == VALUE
    assert call(10, 16 * 512) == WORKSPACE                  # the int8 codes alone need M K bytes
    assert call(1, 0) == OK
    L = qa.lib()
    for M, K in [(1, 64), (16, 512), (2048, 4096)]:
        ws = L.qa_qlinear_w4a8_workspace(M, K)
        assert ws >= M * K + 4 * M and ws % 256 == 0
    g = qa.lib().qa_gemm_w4a8_group_acc
    assert g(A, B, 4, 512, 4, 100, OUT, None) == SHAPE
    assert g(A, None, 4, 512, 4, 128, OUT, None) == NULL
    assert g(MIS, B, 4, 512, 4, 128, OUT, None) == ALIGN


def test_w4a4_asym_argument_errors():
    h = qa.lib().qa_hadamard_quant_int4_asym
    assert h(None, 4, 256, 128, B, OUT, WS, None) == NULL
    assert h(A, 4, 256, 128, B, OUT, None, None) == NULL
    assert h(A, 4, 256, 96, B, OUT, WS, None) == SHAPE
    assert h(A, 4, 200, 16, B, OUT, WS, None) == SHAPE
    assert h(MIS, 4, 256, 128, B, OUT, WS, None) == ALIGN
    assert h(A, 0, 256, 128, B, OUT, WS, None) == OK
    c = qa.lib().qa_w4_column_terms
    assert c(A, B, 16, 512, 4, OUT, None) == SHAPE                     # G < 8
    assert c(A, B, 16, 500, 128, OUT, None) == SHAPE
    assert c(None, B, 16, 512, 128, OUT, None) == NULL
    assert c(A, B, 0, 512, 128, None, None) == OK
    f = qa.lib().qa_qlinear_w4a4_asym
    base = [A, 16, 512, B, OUT, OUT, 32, 128, OUT, 0, WS, 1 << 30, None]

    def call(i, v):
        a = list(base)
        a[i] = v
        return f(*a)
    assert call(0, None) == NULL
    assert call(5, None) == NULL                                      # c_w
    assert call(7, 4) == SHAPE
    assert call(7, 1024) == SHAPE
    assert call(2, 320) == SHAPE
    assert call(3, MIS) == ALIGN
    assert call(9, 7) == VALUE
    assert call(11, 16 * 256) == WORKSPACE                            # codes fit, scales and zero-points do not
    assert call(1, 0) == OK
    for M, K in [(1, 64), (2048, 4096)]:
        assert qa.lib().qa_qlinear_w4a4_asym_workspace(M, K) >= M * K // 2 + 8 * M


def test_gemm_i8_argument_errors():
    f = qa.lib().qa_gemm_i8_i32
    assert f(None, B, 4, 64, 4, OUT, None) == NULL
    assert f(A, B, 4, 40, 4, OUT, None) == SHAPE
    assert f(A, MIS, 4, 64, 4, OUT, None) == ALIGN
    assert f(A, B, 0, 64, 4, OUT, None) == OK


def test_col_absmax_argument_errors():
    f = qa.lib().qa_col_absmax
    args = [A, 16, 256, OUT, 0, WS, 1 << 20, None]

    def call(i, v):
        a = list(args)
        a[i] = v
        return f(*a)
    assert call(0, None) == NULL
    assert call(3, None) == NULL
    assert call(5, None) == NULL
    assert call(2, 12) == SHAPE
    assert call(2, 0) == SHAPE
    assert call(1, -1) == SHAPE
    assert call(2, (1 << 22) + 8) == SHAPE
    assert call(0, MIS) == ALIGN
    assert call(6, 16) == WORKSPACE
    assert call(1, 0) == OK                                    # no rows: no-op
    assert qa.lib().qa_col_absmax_workspace(256) == qa.lib().qa_outlier_cols_workspace(256)


def test_smooth_factors_argument_errors():
    f = qa.lib().qa_smooth_factors
    assert f(None, B, 64, 0.5, OUT, None) == NULL
    assert f(A, B, 64, 0.5, None, None) == NULL
    assert f(A, B, -1, 0.5, OUT, None) == SHAPE
    assert f(A, B, 64, -0.1, OUT, None) == VALUE
    assert f(A, B, 64, 1.5, OUT, None) == VALUE
    assert f(A, B, 64, math.nan, OUT, None) == VALUE
    assert f(ctypes.c_void_p(0x10002), B, 64, 0.5, OUT, None) == ALIGN
    assert f(A, B, 0, 0.5, OUT, None) == OK


def test_quantize_smooth_argument_errors():
    f = qa.lib().qa_quantize_smooth_int8
    args = [A, 4, 64, B, 0, 0, OUT, WS, None]

    def call(i, v):
        a = list(args)
        a[i] = v
        return f(*a)
    assert call(0, None) == NULL
    assert call(3, None) == NULL
    assert call(7, None) == NULL
    assert call(2, 60) == SHAPE
    assert call(2, (1 << 26) + 8) == SHAPE
    assert call(1, -1) == SHAPE
    assert call(4, 2) == VALUE                                 # bad op
    assert call(5, 1) == VALUE                                 # per-group is not a mode here
    assert call(0, MIS) == ALIGN
    assert call(6, MIS) == ALIGN
    assert call(1, 0) == OK
    a = list(args)
    a[1], a[5] = 0, 2                                          # per tensor is a valid mode
    assert f(*a) == OK


def test_smooth_linear_argument_errors():
    f = qa.lib().qa_qlinear_int8_smooth
    base = [A, 16, 256, B, 0, B, OUT, 32, OUT, 1, WS, 1 << 30, None]

    def call(i, v):
        a = list(base)
        a[i] = v
        return f(*a)
    assert call(0, None) == NULL
    assert call(3, None) == NULL
    assert call(10, None) == NULL
    assert call(2, 24) == SHAPE
    assert call(2, 131088) == SHAPE
    assert call(1, -1) == SHAPE
    assert call(4, 1) == VALUE
    assert call(9, 3) == VALUE
    assert call(0, MIS) == ALIGN
    assert call(10, ctypes.c_void_p(0x40010)) == ALIGN
    assert call(11, 100) == WORKSPACE
    assert call(1, 0) == OK and call(7, 0) == OK
    L = qa.lib()
    for M, K in [(1, 16), (2048, 4096)]:
        assert L.qa_qlinear_int8_smooth_workspace(M, K) >= M * K + 4 * M + 4


def test_outlier_topk_argument_errors():
    f = qa.lib().qa_outlier_topk
    args = [A, 16, 256, 3, B, OUT, WS, None, WS, 1 << 20, None]

    def call(i, v):
        a = list(args)
        a[i] = v
        return f(*a)
    assert call(0, None) == NULL
    assert call(8, None) == NULL
    assert call(2, 12) == SHAPE
    assert call(2, 32776) == SHAPE                             # beyond the LDS-resident selection
    assert call(1, -1) == SHAPE
    assert call(3, -1) == VALUE
    assert call(3, 257) == VALUE
    assert call(0, MIS) == ALIGN
    assert call(9, 16) == WORKSPACE


def test_topk_linear_argument_errors():
    f = qa.lib().qa_qlinear_int8_topk
    base = [A, 16, 256, 4, B, OUT, None, 32, OUT, 1, WS, 1 << 30, None]

    def call(i, v):
        a = list(base)
        a[i] = v
        return f(*a)
    assert call(0, None) == NULL
    assert call(10, None) == NULL
    assert call(2, 24) == SHAPE
    assert call(2, 32784) == SHAPE
    assert call(3, -2) == VALUE
    assert call(3, 300) == VALUE
    assert call(9, 5) == VALUE
    assert call(4, MIS) == ALIGN
    assert call(11, 64) == WORKSPACE
    assert call(1, 0) == OK and call(7, 0) == OK
    assert qa.lib().qa_qlinear_int8_topk_workspace(64, 512) == qa.lib().qa_qlinear_int8_mixed_workspace(64, 512)
    assert qa.topk_count(0.01, 4096) == 41 and qa.topk_count(0.02, 4096) == 82 and qa.topk_count(0.0, 64) == 0


def test_asym_quantize_argument_errors():
    f = qa.lib().qa_quantize_rowwise_int8_asym
    args = [A, 4, 64, -128, 127, B, OUT, WS, None, None]

    def call(i, v):
        a = list(args)
        a[i] = v
        return f(*a)
    assert call(0, None) == NULL
    assert call(6, None) == NULL
    assert call(7, None) == NULL
    assert call(2, 60) == SHAPE
    assert call(1, -1) == SHAPE
    assert f(A, 4, 64, 5, 5, B, OUT, WS, None, None) == VALUE    # q_min == q_max
    assert f(A, 4, 64, -129, 127, B, OUT, WS, None, None) == VALUE
    assert call(0, MIS) == ALIGN
    assert call(1, 0) == OK
    g = qa.lib().qa_int8_row_sums
    assert g(None, 4, 64, OUT, None) == NULL
    assert g(A, 4, 72, OUT, None) == SHAPE
    assert g(MIS, 4, 64, OUT, None) == ALIGN
    assert g(A, 0, 64, OUT, None) == OK


def test_asym_linear_argument_errors():
    f = qa.lib().qa_qlinear_int8_asym
    base = [A, 16, 256, B, OUT, None, OUT, 32, OUT, 1, WS, 1 << 30, None]

    def call(i, v):
        a = list(base)
        a[i] = v
        return f(*a)
    assert call(0, None) == NULL
    assert call(6, None) == NULL                               # the weight row sums are required
    assert call(10, None) == NULL
    assert call(2, 24) == SHAPE
    assert call(2, 32784) == SHAPE                             # int32 bound of the zero-point sum
    assert call(9, 4) == VALUE
    assert call(3, MIS) == ALIGN
    assert call(11, 64) == WORKSPACE
    assert call(1, 0) == OK and call(7, 0) == OK
    assert qa.lib().qa_qlinear_int8_asym_workspace(64, 512) >= 64 * 512 + 12 * 64


def test_kron_argument_errors():
    f = qa.lib().qa_kron_quant_int4
    base = [A, 4, 4096, 64, 64, B, OUT, 0, 0, -7, 7, OUT, WS, None]

    def call(i, v):
        a = list(base)
        a[i] = v
        return f(*a)
    assert call(0, None) == NULL
    assert call(5, None) == NULL
    assert call(4, 32) == SHAPE                                # n1 n2 != K
    assert call(1, -1) == SHAPE
    assert f(A, 4, 96, 8, 12, B, OUT, 0, 0, -7, 7, OUT, WS, None) == UNSUPPORTED
    assert call(7, 2) == VALUE                                 # per-tensor is not a mode here
    assert call(9, -9) == VALUE
    assert f(A, 4, 4096, 64, 64, B, OUT, 1, 100, -7, 7, OUT, WS, None) == SHAPE   # K % G
    assert call(5, ctypes.c_void_p(0x20004)) == ALIGN
    assert call(1, 0) == OK
    g = qa.lib().qa_qlinear_kron_w4a4
    gb = [A, 16, 4096, 64, 64, B, OUT, B, OUT, 32, 128, OUT, 0, WS, 1 << 30, None]

    def callg(i, v):
        a = list(gb)
        a[i] = v
        return g(*a)
    assert callg(0, None) == NULL
    assert callg(10, 96) == SHAPE
    assert callg(3, 32) == SHAPE
    assert g(A, 16, 96, 8, 12, B, OUT, B, OUT, 32, 4, OUT, 0, WS, 1 << 30, None) == SHAPE      # G below 8
    assert g(A, 16, 96, 8, 12, B, OUT, B, OUT, 32, 64, OUT, 0, WS, 1 << 30, None) == SHAPE     # K % G
    assert callg(12, 5) == VALUE
    assert callg(14, 64) == WORKSPACE
    assert callg(1, 0) == OK


def test_kron_sizes():
    # the two splits the pages print (tests/golden/kron_sizes.json), then a
    # brute-force minimal-sum search over every n up to 5000, then the oracle
    import json
    import oracle
    with open(os.path.join(ROOT, "tests", "golden", "kron_sizes.json")) as f:
        for c in json.load(f)["cases"]:
            assert qa.qa_kron_sizes(c["n"]) == (c["n1_printed"], c["n2_printed"], True)
    for n in range(1, 5001):
        best = min((a + n // a, a) for a in range(1, n + 1) if n % a == 0 and a * a <= n)
        n1, n2, _ = qa.qa_kron_sizes(n)
        assert (n1, n2) == (best[1], n // best[1]), n
    for n in (64, 96, 4096, 4224, 6144, 8192, 1 << 20, 3 * 5 * 7 * 11 * 13, 2 ** 31 - 1, (1 << 40) + 4):
        assert qa.qa_kron_sizes(n)[:2] == oracle.kron_sizes(n), n
    # a kernel exists for the minimal-sum splits of 64 .. 8192 (powers of two)
    for k in range(6, 14):
        assert qa.qa_kron_sizes(1 << k)[2], k
    assert not qa.qa_kron_sizes(4224)[2] and not qa.qa_kron_sizes(1 << 14)[2]
    n1, n2 = ctypes.c_int64(-5), ctypes.c_int64(-5)
    L = qa.lib()
    assert L.qa_kron_sizes(0, ctypes.byref(n1), ctypes.byref(n2), None) == SHAPE
    assert L.qa_kron_sizes(-3, ctypes.byref(n1), ctypes.byref(n2), None) == SHAPE
    assert (n1.value, n2.value) == (-5, -5)                    # untouched on error
    assert L.qa_kron_sizes(12, None, ctypes.byref(n2), None) == NULL
    assert L.qa_kron_sizes(12, ctypes.byref(n1), ctypes.byref(n2), None) == OK and (n1.value, n2.value) == (3, 4)


def test_mixed_offsets():
    """The workspace offsets of the integer stages: inside the workspace, 256-byte
    aligned, non-overlapping, and the same for the top-k call; bad sizes and a
    NULL array are rejected."""
    L = qa.lib()
    for M, K in [(1, 16), (8, 4096), (2048, 4096), (4096, 8192)]:
        i, c, s, x = qa.qa_qlinear_int8_mixed_offsets(M, K)
        ws = L.qa_qlinear_int8_mixed_workspace(M, K)
        assert ws == L.qa_qlinear_int8_topk_workspace(M, K)
        spans = sorted([(i, 4 * K), (c, 4), (s, 4 * M), (x, M * K)])
        for (a, n), (b, _) in zip(spans, spans[1:]):
            assert a + n <= b
        assert spans[-1][0] + spans[-1][1] <= ws
        assert all(v % 256 == 0 for v in (i, c, s, x))
    off = (ctypes.c_size_t * 4)()
    assert L.qa_qlinear_int8_mixed_offsets(0, 16, off) == SHAPE
    assert L.qa_qlinear_int8_mixed_offsets(4, 0, off) == SHAPE
    assert L.qa_qlinear_int8_mixed_offsets(4, 16, None) == NULL
    assert qa.last_error()


def test_noalloc_argument_errors():
    """The workspace-free LLM.int8() call checks its arguments, and the size of
    the static scratch, before any HIP call."""
    L = qa.lib()

    def call(X=A, M=16, K=256, Wq=B, s_w=OUT, N=32, tau=6.0, out=OUT, dt=1):
        return L.qa_qlinear_int8_mixed_noalloc(X, M, K, Wq, s_w, None, N, tau, out, dt, None)

    assert call(X=None) == NULL and call(out=None) == NULL
    assert call(M=-1) == SHAPE and call(K=24) == SHAPE
    assert call(X=MIS) == ALIGN
    assert call(tau=math.nan) == VALUE and call(dt=3) == VALUE
    assert call(M=0) == OK and call(N=0) == OK
    assert L.qa_qlinear_int8_mixed_workspace(4096, 16384) > qa.NOALLOC_SCRATCH_BYTES
    assert call(M=4096, K=16384) == WORKSPACE
    assert "static scratch" in qa.last_error()
    assert L.qa_qlinear_int8_mixed_workspace(4096, 8192) <= qa.NOALLOC_SCRATCH_BYTES


def test_probe_stream_read_argument_errors():
    p = qa.lib().qa_probe_stream_read
    assert p(A, 1 << 20, 0, 16, 4, OUT, None) == SHAPE
    assert p(A, 1 << 20, 65537, 16, 4, OUT, None) == SHAPE
    assert p(A, 1 << 20, 256, 12, 4, OUT, None) == VALUE
    assert p(A, 1 << 20, 256, 16, 3, OUT, None) == VALUE
    assert p(None, 1 << 20, 256, 16, 4, OUT, None) == NULL
    assert p(A, 1 << 20, 256, 16, 4, None, None) == NULL
    assert p(MIS, 1 << 20, 256, 16, 4, OUT, None) == ALIGN
