"""GPU parity of the W4A4 entry points with zero-point activations against
the CPU oracle.

Codes (stored as q - 8), scales and zero-points match bit for bit; the
column terms match the same fp64 sum rounded once; linear outputs satisfy
max |got - ref| <= 1e-3 * max |ref| (bf16: or one bf16 ulp of the element).
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from test_parity_gpu import ODT, as_f64, assert_float_parity, dev, host, tile_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qa():
    import bit_quantized_linear_int8_amd as qa
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    qa.lib()
    return qa


def check_hq4z(qa, X, G):
    p, s, z = qa.qa_hadamard_quant_int4_asym(dev(X), G)
    op, os_, oz = oracle.hadamard_quant_int4_asym(X, G)
    assert np.array_equal(host(s), os_)
    assert np.array_equal(host(z), oz)
    assert np.array_equal(host(p).view(np.uint32), op)


# ============================================================ quantizer
@pytest.mark.parametrize("G", [1, 2, 4, 8, 16, 32, 64, 128, 256])
def test_hadamard_quant_int4_asym_groups(qa, G):
    rows, K = 13, max(G, 8) * 5
    X, _, _ = synthetic.w4a4_inputs(rows, K, 1, seed=G + 200, n_dims=min(3, K // 16))
    X[1, :] = 0                                           # zero row: s = 1, z = 0, every code 0
    X[2, :] = np.abs(X[2, :])                             # one-sided rows
    X[3, :] = -np.abs(X[3, :])
    check_hq4z(qa, X, G)


@pytest.mark.parametrize("K", [1024, 2048, 4096, 8192])
@pytest.mark.parametrize("G", [8, 64, 128, 256])
def test_hadamard_quant_int4_asym_row_in_registers(qa, K, G):
    X, _, _ = synthetic.w4a4_inputs(13, K, 1, seed=K + G + 2)
    X[5, :] = 0
    X[6, :] = np.abs(X[6, :])
    check_hq4z(qa, X, G)


@pytest.mark.parametrize("K", [8, 264, 520, 4224, 8448, 16384])
def test_hadamard_quant_int4_asym_row_lengths(qa, K):
    G = 8 if K % 64 else 64
    X, _, _ = synthetic.w4a4_inputs(9, K, 1, seed=K + 5, n_dims=min(3, K // 8))
    check_hq4z(qa, X, G)


def test_hadamard_quant_int4_asym_worked_examples(qa):
    # G = 1 leaves rows unrotated: [0, 6] over 16 levels (ties 2.5, 7.5, 12.5)
    # and the range [-0.2, 1.7] that puts real 0 on z = 2
    X = np.zeros((3, 8), np.float16)
    X[0] = [0, 1, 2, 3, 4, 5, 6, 0]
    X[1] = [-0.2, 1.7, 0.0, 0.0, 1.0, -0.1, 0.5, 0.0]
    X[2] = 3.0
    check_hq4z(qa, X, 1)


# ============================================================ column terms
@pytest.mark.parametrize("N,K,G", [(1, 64, 64), (37, 512, 128), (300, 1024, 64), (130, 2048, 256), (8, 256, 8)])
def test_w4_column_terms(qa, N, K, G):
    rng = np.random.default_rng(N + K)
    Wp = rng.integers(0, 2 ** 32, (N, K // 8), dtype=np.uint64).astype(np.uint32)
    s_w = rng.uniform(0.001, 0.1, (N, K // G)).astype(np.float32)
    c = host(qa.qa_w4_column_terms(dev(Wp.view(np.int32)), dev(s_w), K, G))
    assert np.array_equal(c, oracle.w4_column_terms(Wp, s_w, K, G))


# ============================================================ linear
def _w4z_case(qa, M, K, N, G, out_dtype=0, rows=None, seed=0, one_sided=True):
    X, W, _ = synthetic.w4a4_inputs(M, K, N, seed=seed)
    if one_sided:
        X = np.abs(X)
    Wp, s_w = qa.qa_hadamard_quant_int4(dev(W), G, True)
    oWp, os_w = oracle.hadamard_quant_int4(W, G, True)
    assert np.array_equal(host(Wp).view(np.uint32), oWp) and np.array_equal(host(s_w), os_w)
    c_w = qa.qa_w4_column_terms(Wp, s_w, K, G)
    out = as_f64(qa.qa_qlinear_w4a4_asym(dev(X), Wp, s_w, c_w, G=G, out_dtype=ODT[out_dtype]))
    ref = oracle.qlinear_w4a4_asym(X, oWp, os_w, G, rows=rows)
    assert_float_parity(out if rows is None else out[rows], ref, ODT[out_dtype])


@pytest.mark.parametrize("M,K,N,G", [(1, 64, 1, 64), (1, 128, 1, 128), (24, 512, 40, 128), (77, 768, 130, 256),
                                     (200, 1024, 300, 64), (33, 192, 17, 64)])
@pytest.mark.parametrize("one_sided", [True, False])
def test_w4a4_asym_linear_shapes(qa, M, K, N, G, one_sided):
    _w4z_case(qa, M, K, N, G, seed=M + K + 7, one_sided=one_sided)


@pytest.mark.parametrize("out_dtype", [1, 2])
def test_w4a4_asym_linear_out_dtypes(qa, out_dtype):
    _w4z_case(qa, 40, 1024, 96, 128, out_dtype, seed=8)


@pytest.mark.parametrize("M,K,N,G", [(1030, 320, 7976, 64), (2100, 384, 4100, 128)])
def test_w4a4_asym_linear_large_sampled(qa, M, K, N, G):
    rng = np.random.default_rng(M + 9)
    rows = tile_rows(M, 128, extra=4)
    _w4z_case(qa, M, K, N, G, rows=rows, seed=M + G)


@pytest.mark.parametrize("M,K,N,G", [(40, 8448, 96, 64), (33, 8192, 70, 128), (20, 16384, 40, 256)])
def test_w4a4_asym_linear_scales_outside_lds(qa, M, K, N, G):
    # K / G x 256 > 8192: the scales are read per group from memory instead of
    # the block's LDS table
    _w4z_case(qa, M, K, N, G, seed=K + G)


def test_w4a4_asym_config_sampled(qa):
    # the W4A4 workload's shape, 2048 x 4096 x 4096, G = 128, activations made one-sided
    c = synthetic.config("w4a4_hadamard")
    G = c["G"]
    X = np.abs(c["X"])
    Wp, s_w = qa.qa_hadamard_quant_int4(dev(c["W"]), G, True)
    oWp, os_w = oracle.hadamard_quant_int4(c["W"], G, True)
    assert np.array_equal(host(Wp).view(np.uint32), oWp)
    c_w = qa.qa_w4_column_terms(Wp, s_w, c["K"], G)
    out = as_f64(qa.qa_qlinear_w4a4_asym(dev(X), Wp, s_w, c_w, G=G))
    rng = np.random.default_rng(6)
    rows = tile_rows(c["M"], 128, extra=8)
    assert_float_parity(out[rows], oracle.qlinear_w4a4_asym(X, oWp, os_w, G, rows=rows), torch.float32)
    p, s, z = qa.qa_hadamard_quant_int4_asym(dev(X), G)
    op, os_, oz = oracle.hadamard_quant_int4_asym(X[rows[:8]], G)
    assert np.array_equal(host(p).view(np.uint32)[rows[:8]], op)
    assert np.array_equal(host(s)[rows[:8]], os_) and np.array_equal(host(z)[rows[:8]], oz)
