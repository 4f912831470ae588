"""GPU parity of the SmoothQuant entry points against the CPU oracle.

Column maxima, smoothed codes and scales match bit for bit (the smoothing is
one IEEE fp32 operation on both sides, given the same factors).  The
migration factors come from an fp64 pow on each side, so they may differ by
one rounding: at most one fp32 ulp.  Linear outputs satisfy
max |got - ref| <= 1e-3 * max |ref| (bf16: or one bf16 ulp of the element).
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from test_parity_gpu import DEV, ODT, as_f64, assert_float_parity, dev, host, tile_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qa():
    import bit_quantized_linear_int8_amd as qa
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    qa.lib()
    return qa


def factors(X, W, alpha=0.5):
    return oracle.smooth_factors(oracle.col_absmax(X), oracle.col_absmax(W), alpha)


# ============================================================ column maxima
@pytest.mark.parametrize("rows,K", [(1, 8), (3, 40), (37, 520), (300, 1032), (257, 4096), (1000, 8)])
def test_col_absmax_shapes(qa, rows, K):
    A, _, _ = synthetic.mixed_inputs(rows, K, 1, seed=rows * 3 + K, n_dims=min(5, K // 8), p_token=0.5)
    got = qa.qa_col_absmax(dev(A))
    assert np.array_equal(host(got), oracle.col_absmax(A))


def test_col_absmax_accumulates_over_batches(qa):
    A1, _, _ = synthetic.mixed_inputs(40, 1024, 1, seed=31, n_dims=4)
    A2, _, _ = synthetic.mixed_inputs(70, 1024, 1, seed=32, n_dims=4)
    scratch = torch.full((qa.qa_col_absmax_workspace(1024),), 255, dtype=torch.uint8, device=DEV)
    cm = qa.qa_col_absmax(dev(A1), scratch=scratch)
    qa.qa_col_absmax(dev(A2), colmax=cm, accumulate=True, scratch=scratch)
    assert np.array_equal(host(cm), oracle.col_absmax(np.concatenate([A1, A2])))


def test_col_absmax_of_weight_config(qa):
    # the weight statistic of the prefill layer: max over 11008 output channels
    c = synthetic.config("prefill_mixed")
    assert np.array_equal(host(qa.qa_col_absmax(dev(c["W"]))), oracle.col_absmax(c["W"]))
    assert np.array_equal(host(qa.qa_col_absmax(dev(c["X"]))), oracle.col_absmax(c["X"]))


# ============================================================ migration factors
@pytest.mark.parametrize("alpha", [0.0, 0.25, 0.5, 0.8, 1.0])
def test_smooth_factors_within_one_ulp(qa, alpha):
    X, W, _ = synthetic.mixed_inputs(64, 4096, 512, seed=33, n_dims=6)
    cx, cw = oracle.col_absmax(X), oracle.col_absmax(W)
    cx[5] = 0.0
    cw[9] = 0.0
    a32 = float(np.float32(alpha))
    ref = oracle.smooth_factors(cx, cw, a32)
    got = host(qa.qa_smooth_factors(dev(cx), dev(cw), alpha))
    assert got[5] == 1.0 and got[9] == 1.0
    ulps = np.abs(got.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
    assert ulps.max() <= 1
    assert (ulps == 0).mean() > 0.99


# ============================================================ smoothing + quantization
SHAPES = [(1, 8), (5, 24), (9, 520), (33, 1032), (17, 2056), (6, 4096), (4, 8200), (3, 8192), (2, 16392),
          (7, 6000)]


@pytest.mark.parametrize("rows,K", SHAPES)
@pytest.mark.parametrize("multiply", [False, True])
@pytest.mark.parametrize("per_tensor", [False, True])
def test_quantize_smooth_bit_exact(qa, rows, K, multiply, per_tensor):
    X, W, _ = synthetic.mixed_inputs(rows, K, 16, seed=rows * 5 + K, n_dims=min(4, K // 8), p_token=0.75)
    s = factors(X, W)
    A = W if multiply else X
    if not multiply and rows > 1:
        A[1, :] = 0                                       # an all-zero row -> safe scale 1.0
    op = oracle.SMOOTH_MULTIPLY if multiply else oracle.SMOOTH_DIVIDE
    q, so = qa.qa_quantize_smooth_int8(dev(A), dev(s), multiply=multiply, per_tensor=per_tensor)
    oq, os_ = oracle.smooth_quantize(A, s, op, per_tensor=per_tensor)
    assert np.array_equal(host(so), os_)
    assert np.array_equal(host(q), oq)


def test_quantize_smooth_zero_tensor_per_tensor(qa):
    A = np.zeros((7, 256), np.float16)
    s = np.linspace(0.5, 3.0, 256).astype(np.float32)
    q, so = qa.qa_quantize_smooth_int8(dev(A), dev(s), per_tensor=True)
    assert np.array_equal(host(so), np.ones(7, np.float32))
    assert not host(q).any()


def test_quantize_smooth_many_rows_per_tensor(qa):
    # more rows than the per-tensor reduction block has threads
    X, W, _ = synthetic.mixed_inputs(2500, 64, 8, seed=34, n_dims=2)
    s = factors(X, W)
    q, so = qa.qa_quantize_smooth_int8(dev(X), dev(s), per_tensor=True)
    oq, os_ = oracle.smooth_quantize(X, s, oracle.SMOOTH_DIVIDE, per_tensor=True)
    assert np.array_equal(host(so), os_) and np.array_equal(host(q), oq)


# ============================================================ SmoothQuant linear
@pytest.mark.parametrize("M,K,N", [(1, 16, 1), (5, 48, 7), (16, 256, 256), (33, 528, 70), (130, 1040, 300),
                                   (257, 4096, 520)])
@pytest.mark.parametrize("per_tensor", [False, True])
@pytest.mark.parametrize("odt", [0, 1, 2])
def test_qlinear_smooth_shapes(qa, M, K, N, per_tensor, odt):
    X, W, _ = synthetic.mixed_inputs(M, K, N, seed=M + 3 * K + 7 * N, n_dims=min(5, K // 16))
    s = factors(X, W)
    Wq, s_w = oracle.smooth_quantize(W, s, oracle.SMOOTH_MULTIPLY)
    out = qa.qa_qlinear_int8_smooth(dev(X), dev(s), dev(Wq), dev(s_w), per_tensor=per_tensor, out_dtype=ODT[odt])
    ref = oracle.qlinear_int8_smooth(X, s, Wq, s_w, per_tensor=per_tensor)
    assert_float_parity(as_f64(out), ref, ODT[odt])


@pytest.mark.parametrize("M", [1, 8, 16])
def test_qlinear_smooth_decode_shapes(qa, M):
    X, W, _ = synthetic.mixed_inputs(M, 4096, 4096, seed=35 + M, n_dims=6, magnitude=("abs_normal", 20.0),
                                     p_token=1.0)
    s = factors(X, W)
    Wq, s_w = oracle.smooth_quantize(W, s, oracle.SMOOTH_MULTIPLY)
    out = qa.qa_qlinear_int8_smooth(dev(X), dev(s), dev(Wq), dev(s_w), out_dtype=torch.float16)
    ref = oracle.qlinear_int8_smooth(X, s, Wq, s_w)
    assert_float_parity(as_f64(out), ref, torch.float16)


@pytest.mark.parametrize("M", [1, 3, 4, 5, 8])
@pytest.mark.parametrize("K,N", [(256, 1), (1024, 40), (3072, 100), (4096, 33)])
@pytest.mark.parametrize("per_tensor", [False, True])
def test_qlinear_smooth_decode_kernel_shapes(qa, M, K, N, per_tensor):
    # M <= 8 with K % 256 == 0, K <= 4096 runs the fused single-kernel path (smoothed values held)
    X, W, _ = synthetic.mixed_inputs(M, K, N, seed=M * 7 + K + N, n_dims=5, p_token=1.0)
    if M > 2:
        X[1, :] = 0                                        # an all-zero token: scale 1 (per token)
    s = factors(X, W)
    Wq, s_w = oracle.smooth_quantize(W, s, oracle.SMOOTH_MULTIPLY)
    odt = 2 if M == 5 else 0
    out = qa.qa_qlinear_int8_smooth(dev(X), dev(s), dev(Wq), dev(s_w), per_tensor=per_tensor, out_dtype=ODT[odt])
    ref = oracle.qlinear_int8_smooth(X, s, Wq, s_w, per_tensor=per_tensor)
    assert_float_parity(as_f64(out), ref, ODT[odt])


@pytest.mark.parametrize("M", [1, 3, 4])
@pytest.mark.parametrize("K,N", [(4352, 17), (8192, 48)])
@pytest.mark.parametrize("per_tensor", [False, True])
def test_qlinear_smooth_decode_kernel_k8192(qa, M, K, N, per_tensor):
    # M <= 4 with K up to 8192 (the pages' hidden size): two chunks per lane,
    # the division redone in the codes pass instead of held
    X, W, _ = synthetic.mixed_inputs(M, K, N, seed=M * 11 + K + N, n_dims=5, p_token=1.0)
    s = factors(X, W)
    Wq, s_w = oracle.smooth_quantize(W, s, oracle.SMOOTH_MULTIPLY)
    out = qa.qa_qlinear_int8_smooth(dev(X), dev(s), dev(Wq), dev(s_w), per_tensor=per_tensor, out_dtype=torch.float32)
    ref = oracle.qlinear_int8_smooth(X, s, Wq, s_w, per_tensor=per_tensor)
    assert_float_parity(as_f64(out), ref, torch.float32)


def test_qlinear_smooth_decode_k8192_one_hot_codes(qa):
    """4 tokens at K = 8192 against a one-hot int8 weight: every smoothed
    code and scale of the fused kernel's two-chunk path, bit for bit."""
    M, K = 4, 8192
    X, W, _ = synthetic.mixed_inputs(M, K, 64, seed=81, n_dims=6, magnitude=("abs_normal", 20.0), p_token=1.0)
    s = factors(X, W)
    Wq = np.zeros((K, K), np.int8)
    Wq[np.arange(K), np.arange(K)] = 127
    out = host(qa.qa_qlinear_int8_smooth(dev(X), dev(s), dev(Wq), dev(np.ones(K, np.float32)),
                                         out_dtype=torch.float32))
    oq, os_ = oracle.smooth_quantize(X, s, oracle.SMOOTH_DIVIDE)
    want = (127 * oq.astype(np.int32)).astype(np.float32) * np.asarray(os_, np.float32).reshape(-1, 1)
    bad = np.argwhere(out != want)
    assert bad.size == 0, "%d outputs differ, first at %s" % (len(bad), bad[:4].tolist())


@pytest.mark.parametrize("per_tensor", [False, True])
def test_qlinear_smooth_decode_one_hot_codes(qa, per_tensor):
    """The decode workload's X (8 x 4096) smoothed by its factors against a
    one-hot int8 weight Wq[n][n] = 127 with s_w = 1: output (m, n) is
    fl32(127 code(m, n)) * s_x[m] exactly, so every smoothed code and every
    scale of the fused decode kernel is compared bit for bit."""
    c = synthetic.config("decode_mixed")
    X, W, K = c["X"], c["W"], c["K"]
    s = factors(X, W)
    Wq = np.zeros((K, K), np.int8)
    Wq[np.arange(K), np.arange(K)] = 127
    s_w = np.ones(K, np.float32)
    out = host(qa.qa_qlinear_int8_smooth(dev(X), dev(s), dev(Wq), dev(s_w), per_tensor=per_tensor,
                                         out_dtype=torch.float32))
    oq, os_ = oracle.smooth_quantize(X, s, oracle.SMOOTH_DIVIDE, per_tensor=per_tensor)
    want = (127 * oq.astype(np.int32)).astype(np.float32) * np.asarray(os_, np.float32).reshape(-1, 1)
    bad = np.argwhere(out != want)
    assert bad.size == 0, "%d outputs differ, first at %s" % (len(bad), bad[:4].tolist())


@pytest.mark.parametrize("M,K,N", [(5, 8192, 33), (12, 3072, 50), (9, 8192, 100), (16, 5120, 40)])
def test_qlinear_smooth_gemv_shapes(qa, M, K, N):
    # decode-size calls that the fused decode kernel does not take (M > 8, or
    # M > 4 with K > 4096) run the int8 GEMM as a GEMV: codes staged in LDS while
    # M K <= 64 KB (K = 8192: two batches of K steps per wave, K = 3072: one),
    # else loaded per wave
    X, W, _ = synthetic.mixed_inputs(M, K, N, seed=M + K + N, n_dims=5, p_token=1.0)
    s = factors(X, W)
    Wq, s_w = oracle.smooth_quantize(W, s, oracle.SMOOTH_MULTIPLY)
    out = qa.qa_qlinear_int8_smooth(dev(X), dev(s), dev(Wq), dev(s_w), out_dtype=torch.float16)
    ref = oracle.qlinear_int8_smooth(X, s, Wq, s_w)
    assert_float_parity(as_f64(out), ref, torch.float16)


def _full_size(qa, name, per_tensor, rows):
    c = synthetic.config(name)
    X, W = c["X"], c["W"]
    # calibration and the offline weight on the device, checked exactly
    cx = qa.qa_col_absmax(dev(X))
    cw = qa.qa_col_absmax(dev(W))
    assert np.array_equal(host(cx), oracle.col_absmax(X)) and np.array_equal(host(cw), oracle.col_absmax(W))
    s_dev = qa.qa_smooth_factors(cx, cw, 0.5)
    s = host(s_dev)
    Wq_d, s_w_d = qa.qa_quantize_smooth_int8(dev(W), s_dev, multiply=True)
    Wq, s_w = oracle.smooth_quantize(W, s, oracle.SMOOTH_MULTIPLY)
    assert np.array_equal(host(s_w_d), s_w)
    assert np.array_equal(host(Wq_d), Wq)
    odt = c["out_dtype"]
    out = qa.qa_qlinear_int8_smooth(dev(X), s_dev, Wq_d, s_w_d, per_tensor=per_tensor, out_dtype=ODT[odt])
    got = as_f64(out)[rows]
    ref = oracle.qlinear_int8_smooth(X, s, Wq, s_w, per_tensor=per_tensor, rows=rows)
    assert_float_parity(got, ref, ODT[odt])


@pytest.mark.parametrize("per_tensor", [False, True])
def test_qlinear_smooth_prefill_size_sampled(qa, per_tensor):
    _full_size(qa, "prefill_mixed", per_tensor, tile_rows(2048, 256, extra=2))


def test_qlinear_smooth_ffn_size_sampled(qa):
    _full_size(qa, "w8a8_ffn", True, tile_rows(4096, 256))


def test_smoothing_lowers_error_on_device(qa):
    """On outlier-heavy activations the smoothed W8A8 output is closer to the
    exact product than plain vector-wise W8A8 (both computed on the GPU)."""
    X, W, _ = synthetic.mixed_inputs(256, 2048, 512, seed=36, n_dims=7, magnitude=("uniform", 20.0, 100.0))
    exact = X.astype(np.float64) @ W.astype(np.float64).T
    s = factors(X, W)
    Wq, s_w = oracle.smooth_quantize(W, s, oracle.SMOOTH_MULTIPLY)
    out_s = as_f64(qa.qa_qlinear_int8_smooth(dev(X), dev(s), dev(Wq), dev(s_w), out_dtype=torch.float32))
    Wq0, s_w0 = oracle.quant_rows(W)
    out_p = as_f64(qa.qa_qlinear_int8_mixed(dev(X), dev(Wq0), dev(s_w0[:, 0]), threshold=float("inf"),
                                            out_dtype=torch.float32))
    assert np.abs(out_s - exact).mean() < np.abs(out_p - exact).mean() / 2
