"""GPU parity of the top-k decomposition entry points against the CPU oracle.

The top-k set (mask, ascending list, count) and the column maxima must match
bit for bit, ties included; linear outputs satisfy
max |got - ref| <= 1e-3 * max |ref| (bf16: or one bf16 ulp of the element).
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from test_parity_gpu import DEV, ODT, as_f64, assert_float_parity, check_int8_stages, dev, host, tile_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qa():
    import bit_quantized_linear_int8_amd as qa
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    qa.lib()
    return qa


def check_topk(qa, X, k, scratch=None):
    mask, idx, count, colmax = qa.qa_outlier_topk(dev(X), k, scratch=scratch)
    om, oidx, ocm = oracle.outlier_topk(X, k)
    n = int(host(count)[0])
    assert n == len(oidx) == min(k, X.shape[1])
    assert np.array_equal(host(idx)[:n], oidx)
    assert np.array_equal(host(mask), om)
    assert np.array_equal(host(colmax), ocm)


# ============================================================ top-k set
@pytest.mark.parametrize("M,K,k", [(1, 8, 0), (1, 8, 3), (1, 8, 8), (3, 40, 5), (37, 520, 13), (130, 1032, 40),
                                   (257, 4096, 41), (257, 4096, 82), (300, 8192, 164), (16, 32768, 655),
                                   (5, 32768, 32768), (16, 8192, 300), (7, 8000, 8000), (17, 1000, 30),
                                   (2, 65536 // 2, 100)])
def test_topk_set_shapes(qa, M, K, k):
    X, _, _ = synthetic.mixed_inputs(M, K, 1, seed=M * 11 + K + k, n_dims=min(9, K // 8), p_token=0.5)
    check_topk(qa, X, k)


@pytest.mark.parametrize("k", [1, 7, 100, 255, 256])
def test_topk_set_with_ties(qa, k):
    # small integers: many equal column maxima, so the boundary falls inside a tie
    rng = np.random.default_rng(k)
    X = rng.integers(-6, 7, size=(9, 256)).astype(np.float16)
    check_topk(qa, X, k)


@pytest.mark.parametrize("M", [20, 8])
def test_topk_zero_columns_and_dirty_scratch(qa, M):
    X = np.zeros((M, 1024), np.float16)
    X[3, 700] = 2.0
    X[5, 10] = -2.0
    X[7, 999] = 0.5
    scratch = torch.full((qa.qa_outlier_cols_workspace(1024),), 255, dtype=torch.uint8, device=DEV)
    for k in (5, 2, 0, 1024):                                # ties at 0 go to the lowest columns
        check_topk(qa, X, k, scratch=scratch)


def test_topk_one_bit_apart_maxima(qa):
    # maxima that differ only in the lowest bits of their fp16 patterns
    K = 512
    X = np.zeros((4, K), np.float16)
    base = np.float16(3.0).view(np.uint16)
    X[1, :] = (base + (np.arange(K) % 5).astype(np.uint16)).view(np.float16)
    for k in (1, 102, 103, 300, 511):
        check_topk(qa, X, k)


# ============================================================ top-k linear
def _topk_case(qa, X, W, k, out_dtype, pass_w16, rows=None):
    Wq, s_w = qa.qa_quantize_rowwise_int8(dev(W))
    oWq, os_w = oracle.quant_rows(W)
    assert np.array_equal(host(Wq), oWq)
    M, K = X.shape
    ws = torch.full((qa.qa_qlinear_int8_topk_workspace(M, K),), 0x5A, dtype=torch.uint8, device=DEV)
    out = qa.qa_qlinear_int8_topk(dev(X), Wq, s_w, k, W16=dev(W) if pass_w16 else None, out_dtype=ODT[out_dtype],
                                  workspace=ws)
    om, oidx, _ = oracle.outlier_topk(X, k)
    check_int8_stages(qa, ws, X, om, oidx)
    ref = oracle.qlinear_int8_topk(X, oWq, os_w[:, 0], W16=W if pass_w16 else None, k=k, rows=rows)
    got = as_f64(out)
    if rows is not None:
        got = got[rows]
    assert_float_parity(got, ref, ODT[out_dtype])


@pytest.mark.parametrize("M,K,N,k", [(1, 16, 1, 1), (5, 48, 7, 0), (16, 256, 256, 3), (33, 528, 77, 6),
                                     (130, 1040, 300, 21), (300, 272, 520, 272), (8, 4096, 64, 41)])
@pytest.mark.parametrize("pass_w16", [True, False])
def test_topk_linear_shapes(qa, M, K, N, k, pass_w16):
    X, W, _ = synthetic.mixed_inputs(M, K, N, seed=M * 17 + N + k, n_dims=min(5, K // 16), p_token=0.75)
    _topk_case(qa, X, W, k, 0, pass_w16)


@pytest.mark.parametrize("M,K,N,k,pass_w16", [(12, 8192, 24, 140, False), (5, 4096, 50, 300, False),
                                              (16, 2048, 70, 257, True), (2, 4112, 33, 20, False)])
def test_topk_linear_gemv_shapes(qa, M, K, N, k, pass_w16):
    # decode sizes outside the fused kernel (M > 8 at K > 4096, k > 256, K not
    # a multiple of 256): the GEMV with codes in LDS (or per wave past 64 KB),
    # one or two staging passes of the fp16 product
    X, W, _ = synthetic.mixed_inputs(M, K, N, seed=M * 3 + k, n_dims=6, p_token=0.9)
    _topk_case(qa, X, W, k, 1, pass_w16)


@pytest.mark.parametrize("M,K,N,k,pass_w16", [(4, 8192, 40, 30, False), (3, 8192, 20, 200, True),
                                              (16, 2048, 70, 100, False), (8, 8192, 48, 256, False),
                                              (1, 256, 16, 1, True), (9, 4096, 100, 82, False)])
def test_topk_linear_decode_shapes(qa, M, K, N, k, pass_w16):
    # the fused decode kernel (M <= 16, K <= 4096, or M <= 8, K <= 8192, k <= 256)
    X, W, _ = synthetic.mixed_inputs(M, K, N, seed=M * 5 + k, n_dims=6, p_token=0.9)
    _topk_case(qa, X, W, k, 1, pass_w16)


@pytest.mark.parametrize("M,K,k", [(8, 256, 5), (8, 256, 256), (3, 1024, 100), (16, 4096, 256), (5, 8192, 77),
                                   (8, 8192, 256), (2, 512, 0), (4, 768, 13)])
def test_topk_linear_decode_ties(qa, M, K, k):
    # small integers: few distinct column maxima, so the k-th falls inside a
    # run of equal keys that the fused kernel must split in column order
    rng = np.random.default_rng(M * 1000 + K + k)
    X = rng.integers(-5, 6, size=(M, K)).astype(np.float16)
    _, W, _ = synthetic.mixed_inputs(1, K, 40, seed=k, n_dims=0)
    _topk_case(qa, X, W, k, 0, False)


@pytest.mark.parametrize("k", [0, 3, 256])
def test_topk_linear_decode_zero_input(qa, k):
    # every key 0: all ties, taken from column 0 up
    X = np.zeros((6, 1024), np.float16)
    _, W, _ = synthetic.mixed_inputs(1, 1024, 24, seed=3, n_dims=0)
    _topk_case(qa, X, W, k, 1, True)


@pytest.mark.parametrize("out_dtype", [0, 1, 2])
def test_topk_linear_out_dtypes(qa, out_dtype):
    X, W, _ = synthetic.mixed_inputs(40, 512, 96, seed=45, n_dims=3, x_dist="t3")
    _topk_case(qa, X, W, 11, out_dtype, False)


@pytest.mark.parametrize("share", [0.01, 0.02])
def test_topk_linear_prefill_size_sampled(qa, share):
    c = synthetic.config("prefill_mixed")
    k = qa.topk_count(share, c["K"])
    rows = tile_rows(c["M"], 256)
    _topk_case(qa, c["X"], c["W"], k, c["out_dtype"], False, rows=rows)


def test_topk_linear_decode_config(qa):
    c = synthetic.config("decode_mixed")
    _topk_case(qa, c["X"], c["W"], qa.topk_count(0.02, c["K"]), c["out_dtype"], False)
