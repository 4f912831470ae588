"""GPU parity of the Kronecker-transform (FlatQuant apply side) entry points
against the CPU oracle.

The transform is the same sequence of fp32 fused multiply-adds on both sides,
so packed int4 words and scales match bit for bit; linear outputs satisfy
max |got - ref| <= 1e-3 * max |ref|.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from test_parity_gpu import ODT, as_f64, assert_float_parity, dev, host, tile_rows

pytestmark = pytest.mark.gpu

SIZES = [(8, 8), (8, 16), (16, 16), (16, 32), (32, 32), (32, 64), (64, 64), (64, 128)]


@pytest.fixture(scope="module")
def qa():
    import bit_quantized_linear_int8_amd as qa
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    qa.lib()
    return qa


def check_kron(qa, X, P1, P2, G=None, q_min=-7, q_max=7):
    packed, s = qa.qa_kron_quant_int4(dev(X), dev(P1), dev(P2), G=G, q_min=q_min, q_max=q_max)
    op, os_ = oracle.kron_quant_int4(X, P1, P2, per_group_G=G, qmin=q_min, qmax=q_max)
    assert np.array_equal(host(s), os_)
    assert np.array_equal(host(packed).view(np.uint32), op)


@pytest.mark.parametrize("n1,n2", SIZES)
@pytest.mark.parametrize("kind", ["orthogonal", "general"])
def test_kron_quant_per_row(qa, n1, n2, kind):
    rows = 37
    X, _, _ = synthetic.mixed_inputs(rows, n1 * n2, 1, seed=n1 * n2 + rows, n_dims=min(6, n1), p_token=0.6)
    X[3] = 0                                              # zero row: scale 1.0, all codes 0
    P1, P2 = synthetic.kron_factors(n1, n2, seed=n1 + n2, kind=kind)
    check_kron(qa, X, P1, P2)


@pytest.mark.parametrize("n1,n2,G", [(16, 16, 64), (16, 32, 128), (32, 32, 128), (32, 64, 256), (64, 64, 64),
                                     (64, 64, 128), (64, 64, 256), (64, 128, 128), (8, 8, 32)])
def test_kron_quant_per_group(qa, n1, n2, G):
    X, W, _ = synthetic.w4a4_inputs(5, n1 * n2, 33, seed=G + n1)
    P1, P2 = synthetic.kron_factors(n1, n2, seed=G, kind="orthogonal")
    check_kron(qa, W, P1, P2, G=G)


@pytest.mark.parametrize("q_min,q_max", [(-8, 7), (-7, 7), (0, 7), (-3, 3)])
def test_kron_quant_ranges(qa, q_min, q_max):
    X, _, _ = synthetic.mixed_inputs(9, 1024, 1, seed=q_max - q_min, n_dims=3)
    P1, P2 = synthetic.kron_factors(32, 32, seed=5, kind="general")
    check_kron(qa, X, P1, P2, q_min=q_min, q_max=q_max)


def test_kron_identity_and_hadamard_factors(qa):
    # identity: the codes of X itself; Hadamard factors: many exact ties at .5
    rng = np.random.default_rng(81)
    X = rng.integers(-8, 9, (11, 4096)).astype(np.float16)
    eye = np.eye(64, dtype=np.float32)
    check_kron(qa, X, eye, eye)
    import scipy.linalg
    H = scipy.linalg.hadamard(64).astype(np.float32)
    check_kron(qa, X, H, H)


def test_kron_many_rows_ragged(qa):
    # token counts that leave the last workgroup partly empty
    P1, P2 = synthetic.kron_factors(64, 64, seed=9)
    for rows in (1, 3, 5, 258):
        X, _, _ = synthetic.mixed_inputs(rows, 4096, 1, seed=rows, n_dims=6)
        check_kron(qa, X, P1, P2)


def _kron_linear(qa, M, K, N, n1, n2, G, out_dtype, rows=None, seed=0):
    X, W, _ = synthetic.w4a4_inputs(M, K, N, seed=seed)
    P1, P2 = synthetic.kron_factors(n1, n2, seed=seed + 1, kind="general")
    P1w = np.linalg.inv(P1.astype(np.float64)).T.astype(np.float32)
    P2w = np.linalg.inv(P2.astype(np.float64)).T.astype(np.float32)
    Wp, s_w = qa.qa_kron_quant_int4(dev(W), dev(P1w), dev(P2w), G=G)
    oWp, os_w = oracle.kron_quant_int4(W, P1w, P2w, per_group_G=G)
    assert np.array_equal(host(Wp).view(np.uint32), oWp) and np.array_equal(host(s_w), os_w)
    out = qa.qa_qlinear_kron_w4a4(dev(X), dev(P1), dev(P2), Wp, s_w, G=G, out_dtype=ODT[out_dtype])
    ref = oracle.qlinear_kron_w4a4(X, P1, P2, oWp, os_w, G=G, rows=rows)
    got = as_f64(out)
    if rows is not None:
        got = got[rows]
    assert_float_parity(got, ref, ODT[out_dtype])


@pytest.mark.parametrize("M,K,N,n1,n2,G", [(1, 256, 16, 16, 16, 64), (7, 1024, 100, 32, 32, 128),
                                           (130, 2048, 260, 32, 64, 256), (64, 4096, 300, 64, 64, 128),
                                           (33, 8192, 129, 64, 128, 128)])
def test_kron_linear_shapes(qa, M, K, N, n1, n2, G):
    _kron_linear(qa, M, K, N, n1, n2, G, 0, seed=M + N)


@pytest.mark.parametrize("out_dtype", [1, 2])
def test_kron_linear_out_dtypes(qa, out_dtype):
    _kron_linear(qa, 40, 1024, 96, 32, 32, 128, out_dtype, seed=3)


def test_kron_linear_w4a4_size_sampled(qa):
    # the W4A4 workload's shape: 2048 x 4096 x 4096, 64 x 64 factors, G = 128
    _kron_linear(qa, 2048, 4096, 4096, 64, 64, 128, 0, rows=tile_rows(2048, 128), seed=11)
