"""GPU parity of the W4A8 entry points (group-Hadamard int8 activations
against the offline per-group int4 weight) with the CPU oracle.

Codes, scales and int32 group sums match bit for bit; linear outputs satisfy
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


def check_hq8(qa, X, G, q_min=-127, q_max=127):
    q, s = qa.qa_hadamard_quant_int8(dev(X), G, q_min, q_max)
    oq, os_ = oracle.hadamard_quant_int8(X, G, q_min, q_max)
    assert np.array_equal(host(s), os_)
    assert np.array_equal(host(q), oq)


# ============================================================ quantizer
@pytest.mark.parametrize("G", [1, 2, 4, 8, 16, 32, 64, 128, 256])
def test_hadamard_quant_int8_groups(qa, G):
    rows, K = 13, max(G, 8) * 5
    X, _, _ = synthetic.w4a4_inputs(rows, K, 1, seed=G + 100, n_dims=min(3, K // 16))
    X[1, :] = 0                                            # zero row: s = 1, codes 0
    check_hq8(qa, X, G)


@pytest.mark.parametrize("K", [1024, 2048, 4096, 8192])
@pytest.mark.parametrize("G", [8, 32, 64, 128, 256])
def test_hadamard_quant_int8_row_in_registers(qa, K, G):
    # K = 512 NC WPR: the row held in registers by one or two waves; 13 rows
    # leave the last workgroup partly past the end
    X, _, _ = synthetic.w4a4_inputs(13, K, 1, seed=K + G + 1)
    X[5, :] = 0
    check_hq8(qa, X, G)


@pytest.mark.parametrize("K", [8, 264, 520, 4224, 8448, 16384])
def test_hadamard_quant_int8_row_lengths(qa, K):
    G = 8 if K % 64 else 64
    X, _, _ = synthetic.w4a4_inputs(9, K, 1, seed=K, n_dims=min(3, K // 8))
    check_hq8(qa, X, G)


@pytest.mark.parametrize("q_min,q_max", [(-128, 127), (-127, 127), (-100, 50), (0, 127), (-7, 7)])
def test_hadamard_quant_int8_ranges(qa, q_min, q_max):
    X, _, _ = synthetic.w4a4_inputs(11, 1024, 1, seed=q_max - q_min)
    check_hq8(qa, X, 128, q_min, q_max)


def test_hadamard_quant_int8_ties(qa):
    # G = 1 leaves X unrotated: rows whose scale is exactly 1 (absmax 127)
    # put values on x.5, which round half to even
    X = np.zeros((3, 64), np.float16)
    X[0, :9] = [127.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, -126.5]
    X[1, :4] = [-127.0, 63.5, -63.5, 100.5]
    X[2, :] = np.float16(-3.0)
    check_hq8(qa, X, 1)


# ============================================================ group accumulators
@pytest.mark.parametrize("M,K,N,G", [(1, 64, 1, 64), (20, 256, 33, 128), (64, 384, 64, 128), (130, 512, 70, 256),
                                     (300, 1024, 500, 64), (2048, 256, 2048, 128),
                                     # >= 256 tiles of 128 x 256, ragged M and N, K ending half-way
                                     # through a 128-element stage
                                     (1030, 320, 7976, 64), (2100, 384, 4100, 128), (1100, 512, 7700, 256)])
def test_w4a8_group_acc(qa, M, K, N, G):
    rng = np.random.default_rng(M + N + 1)
    Xq = rng.integers(-128, 128, (M, K)).astype(np.int8)   # full int8 range, -128 included
    Wp = rng.integers(0, 2 ** 32, (N, K // 8), dtype=np.uint64).astype(np.uint32)
    acc = host(qa.qa_gemm_w4a8_group_acc(dev(Xq), dev(Wp), G))
    rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, size=min(M, 16), replace=False)]))
    assert np.array_equal(acc[rows], oracle.w4a8_group_acc(Xq, Wp, G, rows=rows))


# ============================================================ linear
def _w4a8_case(qa, M, K, N, G, out_dtype=0, rows=None, seed=0):
    X, W, _ = synthetic.w4a4_inputs(M, K, N, seed=seed)
    Wp, s_w = qa.qa_hadamard_quant_int4(dev(W), G, True)
    oWp, os_w = oracle.hadamard_quant_int4(W, G, True)
    assert np.array_equal(host(Wp).view(np.uint32), oWp) and np.array_equal(host(s_w), os_w)
    out = as_f64(qa.qa_qlinear_w4a8(dev(X), Wp, s_w, G=G, out_dtype=ODT[out_dtype]))
    ref = oracle.qlinear_w4a8(X, oWp, os_w, G, rows=rows)
    assert_float_parity(out if rows is None else out[rows], ref, ODT[out_dtype])


@pytest.mark.parametrize("M,K,N,G", [(1, 64, 1, 64), (1, 128, 1, 128), (24, 512, 40, 128), (77, 768, 130, 256),
                                     (200, 1024, 300, 64), (33, 192, 17, 64)])
def test_w4a8_linear_shapes(qa, M, K, N, G):
    _w4a8_case(qa, M, K, N, G, seed=M + K + 2)


@pytest.mark.parametrize("M,K,N,G", [(40, 8448, 96, 64), (33, 8192, 70, 128), (20, 16384, 40, 256)])
def test_w4a8_linear_scales_outside_lds(qa, M, K, N, G):
    # K / G x 256 > 8192: the scales are read per group from memory instead of
    # the block's LDS table
    _w4a8_case(qa, M, K, N, G, seed=K + G)


@pytest.mark.parametrize("out_dtype", [1, 2])
def test_w4a8_linear_out_dtypes(qa, out_dtype):
    _w4a8_case(qa, 40, 1024, 96, 128, out_dtype, seed=5)


@pytest.mark.parametrize("M,K,N,G", [(1030, 320, 7976, 64), (2100, 384, 4100, 128), (1100, 512, 7700, 256)])
def test_w4a8_linear_large_sampled(qa, M, K, N, G):
    rng = np.random.default_rng(M + 3)
    rows = tile_rows(M, 128, extra=4)
    _w4a8_case(qa, M, K, N, G, rows=rows, seed=M + G)


def test_w4a8_config_sampled(qa):
    # the W4A4 workload's shape, 2048 x 4096 x 4096, G = 128, as the bench runs it
    c = synthetic.config("w4a4_hadamard")
    G = c["G"]
    Wp, s_w = qa.qa_hadamard_quant_int4(dev(c["W"]), G, True)
    oWp, os_w = oracle.hadamard_quant_int4(c["W"], G, True)
    assert np.array_equal(host(Wp).view(np.uint32), oWp)
    out = as_f64(qa.qa_qlinear_w4a8(dev(c["X"]), Wp, s_w, G=G))
    rng = np.random.default_rng(4)
    rows = tile_rows(c["M"], 128, extra=8)
    assert_float_parity(out[rows], oracle.qlinear_w4a8(c["X"], oWp, os_w, G, rows=rows), torch.float32)
    Xq, s_x = qa.qa_hadamard_quant_int8(dev(c["X"]), G)
    oXq, os_x = oracle.hadamard_quant_int8(c["X"][rows[:8]], G)
    assert np.array_equal(host(Xq)[rows[:8]], oXq) and np.array_equal(host(s_x)[rows[:8]], os_x)
    acc = host(qa.qa_gemm_w4a8_group_acc(Xq, Wp, G))
    assert np.array_equal(acc[rows[:8]], oracle.w4a8_group_acc(host(Xq), oWp, G, rows=rows[:8]))
