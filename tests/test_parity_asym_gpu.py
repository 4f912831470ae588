"""GPU parity of the zero-point (asymmetric) entry points against the CPU oracle.

Codes, scales, zero-points and code sums match bit for bit; linear outputs
satisfy max |got - ref| <= 1e-3 * max |ref| (bf16: or one bf16 ulp of the
element).
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


def check_asym_rows(qa, X, q_min=-128, q_max=127):
    q, s, z, rs = qa.qa_quantize_rowwise_int8_asym(dev(X), q_min, q_max)
    oq, os_, oz, ors = oracle.quant_rows_asym(X, q_min, q_max)
    assert np.array_equal(host(s), os_)
    assert np.array_equal(host(z), oz)
    assert np.array_equal(host(q), oq)
    assert np.array_equal(host(rs), ors)


# ============================================================ quantizer
@pytest.mark.parametrize("rows,K", [(1, 8), (5, 24), (9, 520), (33, 1032), (17, 2056), (6, 4096), (4, 8200),
                                    (3, 8192), (2, 16392),
                                    # 16 chunks per lane over four waves, the last wave's chunks past the row
                                    (7, 6000)])
def test_asym_quant_shapes(qa, rows, K):
    X, _, _ = synthetic.mixed_inputs(rows, K, 1, seed=rows * 3 + K, n_dims=min(4, K // 8), p_token=0.75)
    if rows > 2:
        X[1, :] = 0                                        # zero row: s = 1, z = q_min
        X[2, :] = np.abs(X[2, :]) + np.float16(0.5)        # one-sided row
    check_asym_rows(qa, X)


@pytest.mark.parametrize("K", [4096, 8192])
def test_asym_quant_zero_parts(qa, K):
    # a row's parts are quantized by different waves (halves at K = 4096,
    # quarters at K = 8192): the negative end of a row held by one part while
    # another part is all +0.0 or all -0.0 must still set the row's range
    rng = np.random.default_rng(K)
    X = np.zeros((6, K), np.float16)
    h = K // 4
    X[0, :h] = rng.normal(0, 3, h)                    # values in the first part only
    X[1, -h:] = rng.normal(0, 3, h)                   # values in the last part only
    X[2, :h] = -np.abs(rng.normal(0, 3, h))           # negative first part, -0.0 elsewhere
    X[2, h:] = np.float16(-0.0)
    X[3, h:2 * h] = -np.abs(rng.normal(0, 3, h))      # negative second part only
    X[4, :] = np.float16(-0.0)                        # all -0.0: the zero row's scale and zero point
    X[5, -1] = np.float16(-7.0)                       # one negative value at the end
    check_asym_rows(qa, X)


@pytest.mark.parametrize("q_min,q_max", [(-128, 127), (-127, 127), (0, 15), (-8, 7), (-1, 0)])
def test_asym_quant_ranges(qa, q_min, q_max):
    rng = np.random.default_rng(q_max + 50)
    X = rng.normal(0.3, 2.0, (12, 264)).astype(np.float16)
    X[3] = np.abs(X[3])
    X[4] = -np.abs(X[4])
    check_asym_rows(qa, X, q_min, q_max)


def test_asym_quant_ties(qa):
    # rows whose scale is exactly 1/2 or 1 and whose values sit on x.5 steps
    X = np.zeros((3, 64), np.float16)
    X[0, :2] = [-127.5, 0.0]                              # hi - lo = 127.5, s = 0.5
    X[0, 2:10] = [0.25, 0.75, 1.25, -0.25, -0.75, 10.25, -60.75, 63.25]
    X[1, :2] = [0.0, 255.0]                               # s = 1, z = -128
    X[1, 2:8] = [0.5, 1.5, 2.5, 100.5, 254.5, 127.5]
    X[2, :] = np.float16(-3.0)
    check_asym_rows(qa, X)


def test_int8_row_sums(qa):
    rng = np.random.default_rng(7)
    for rows, K in [(1, 16), (9, 4096), (37, 1040), (5, 8208)]:
        A = rng.integers(-128, 128, (rows, K), dtype=np.int8)
        assert np.array_equal(host(qa.qa_int8_row_sums(dev(A))), A.astype(np.int64).sum(axis=1))


# ============================================================ zero-point linear
def _asym_case(qa, X, W, asym_w, out_dtype, rows=None):
    if asym_w:
        Wq, s_w, z_w, rw = qa.qa_quantize_rowwise_int8_asym(dev(W))
        oWq, os_w, oz_w, orw = oracle.quant_rows_asym(W)
        assert np.array_equal(host(Wq), oWq) and np.array_equal(host(z_w), oz_w) and np.array_equal(host(rw), orw)
    else:
        Wq, s_w = qa.qa_quantize_rowwise_int8(dev(W))
        z_w = None
        rw = qa.qa_int8_row_sums(Wq)
        oWq, os_w = oracle.quant_rows(W)
        os_w, oz_w = os_w[:, 0], None
    out = qa.qa_qlinear_int8_asym(dev(X), Wq, s_w, rw, z_w=z_w, out_dtype=ODT[out_dtype])
    ref = oracle.qlinear_int8_asym(X, oWq, os_w, z_w=oz_w, rows=rows)
    got = as_f64(out)
    if rows is not None:
        got = got[rows]
    assert_float_parity(got, ref, ODT[out_dtype])


@pytest.mark.parametrize("M,K,N", [(1, 16, 1), (5, 48, 7), (16, 256, 256), (33, 528, 77), (130, 1040, 300),
                                   (300, 272, 520), (8, 4096, 64)])
@pytest.mark.parametrize("asym_w", [False, True])
def test_asym_linear_shapes(qa, M, K, N, asym_w):
    X, W, _ = synthetic.mixed_inputs(M, K, N, seed=M * 19 + N, n_dims=min(5, K // 16), p_token=0.75)
    X[: max(1, M // 3)] = np.abs(X[: max(1, M // 3)])        # some one-sided tokens
    _asym_case(qa, X, W, asym_w, 0)


@pytest.mark.parametrize("out_dtype", [0, 1, 2])
def test_asym_linear_out_dtypes(qa, out_dtype):
    X, W, _ = synthetic.mixed_inputs(40, 512, 96, seed=61, n_dims=3, x_dist="t3")
    _asym_case(qa, X, W, True, out_dtype)


def test_asym_linear_large_k(qa):
    # the int32 bound: K = 32768 with full-range codes on both sides
    rng = np.random.default_rng(62)
    X = rng.uniform(-1.0, 3.0, (20, 32768)).astype(np.float16)
    W = rng.uniform(-0.5, 1.5, (70, 32768)).astype(np.float16)
    _asym_case(qa, X, W, True, 0)


@pytest.mark.parametrize("asym_w", [False, True])
def test_asym_linear_prefill_size_sampled(qa, asym_w):
    c = synthetic.config("prefill_mixed")
    _asym_case(qa, c["X"], c["W"], asym_w, c["out_dtype"], rows=tile_rows(c["M"], 256, extra=2))


def test_asym_linear_tail_split(qa):
    # 16 x 43 tiles of 256 x 256: two whole rounds over the 256 CUs, the
    # trailing 2816 columns in a second launch of 128 x 256 tiles
    M, K, N = 4096, 64, 11008
    X, W, _ = synthetic.mixed_inputs(M, K, N, seed=63, n_dims=3)
    _asym_case(qa, X, W, True, 1, rows=tile_rows(M, 128, extra=4))


@pytest.mark.parametrize("M,K,N,asym_w,rows", [
    (300, 128, 129 * 256 + 72, True, False),   # 2 x 126 tiles of 256 x 264, ragged M and N
    (3000, 528, 6000, False, True),            # 12 x 21 tiles of 256 x 288, partial last K step
    (2048, 64, 11008, True, True),             # 8 x 32 tiles of 256 x 344
])
def test_asym_linear_wide_tiles(qa, M, K, N, asym_w, rows):
    # one-round wide tiles: each computes 352 columns and stores its stride
    X, W, _ = synthetic.mixed_inputs(M, K, N, seed=M + N, n_dims=3, p_token=0.75)
    X[: M // 4] = np.abs(X[: M // 4])
    _asym_case(qa, X, W, asym_w, 2 if rows else 1, rows=tile_rows(M, 256, extra=6) if rows else None)
