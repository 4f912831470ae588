"""GPU parity of the W4 linears and group accumulators with groups smaller
than one 64-deep MFMA step (G = 8, 16, 32; the pages treat the group size as
a free knob: "模型推理量化" §7.3-§7.4, and the group-rotation page's §二 "分组处理").
Group accumulators are compared bit for bit, linear outputs within
1e-3 * max |ref| (bf16: or one bf16 ulp of the element)."""
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


SHAPES = [(1, 64, 1), (37, 520, 45), (64, 544, 70), (130, 1024, 200), (65, 96, 63)]


def _ok(K, G):
    return K % G == 0


@pytest.mark.parametrize("G", [8, 16, 32])
@pytest.mark.parametrize("M,K,N", SHAPES)
def test_w4a4_group_acc_small_groups(qa, M, K, N, G):
    if not _ok(K, G):
        K = (K // G + 1) * G
    rng = np.random.default_rng(M + K + N + G)
    Xp = rng.integers(0, 2 ** 32, (M, K // 8), dtype=np.uint64).astype(np.uint32)
    Wp = rng.integers(0, 2 ** 32, (N, K // 8), dtype=np.uint64).astype(np.uint32)
    acc = host(qa.qa_gemm_w4a4_group_acc(dev(Xp), dev(Wp), K, G))
    assert np.array_equal(acc, oracle.w4a4_group_acc(Xp, Wp, K, G))


@pytest.mark.parametrize("G", [8, 16, 32])
@pytest.mark.parametrize("M,K,N", SHAPES)
def test_w4a8_group_acc_small_groups(qa, M, K, N, G):
    if not _ok(K, G):
        K = (K // G + 1) * G
    rng = np.random.default_rng(M + K + N + G + 1)
    Xq = rng.integers(-128, 128, (M, K)).astype(np.int8)       # -128 included
    Wp = rng.integers(0, 2 ** 32, (N, K // 8), dtype=np.uint64).astype(np.uint32)
    acc = host(qa.qa_gemm_w4a8_group_acc(dev(Xq), dev(Wp), G))
    assert np.array_equal(acc, oracle.w4a8_group_acc(Xq, Wp, G))


def _weight(qa, W, G):
    Wp, s_w = qa.qa_hadamard_quant_int4(dev(W), G, True)
    oWp, os_w = oracle.hadamard_quant_int4(W, G, True)
    assert np.array_equal(host(Wp).view(np.uint32), oWp) and np.array_equal(host(s_w), os_w)
    return Wp, s_w, oWp, os_w


@pytest.mark.parametrize("G", [8, 16, 32])
@pytest.mark.parametrize("M,K,N,out_dtype", [(1, 64, 1, 0), (24, 512, 40, 0), (77, 768, 130, 1), (200, 1024, 300, 2)])
def test_w4_linears_small_groups(qa, M, K, N, G, out_dtype):
    X, W, _ = synthetic.w4a4_inputs(M, K, N, seed=M + K + G)
    Wp, s_w, oWp, os_w = _weight(qa, W, G)
    odt = ODT[out_dtype]
    out = as_f64(qa.qa_qlinear_w4a4(dev(X), Wp, s_w, G=G, out_dtype=odt))
    assert_float_parity(out, oracle.qlinear_w4a4(X, oWp, os_w, G), odt)
    out = as_f64(qa.qa_qlinear_w4a8(dev(X), Wp, s_w, G=G, out_dtype=odt))
    assert_float_parity(out, oracle.qlinear_w4a8(X, oWp, os_w, G), odt)
    Xa = np.abs(X)                                        # one-sided: the zero-point case
    c_w = qa.qa_w4_column_terms(Wp, s_w, K, G)
    out = as_f64(qa.qa_qlinear_w4a4_asym(dev(Xa), Wp, s_w, c_w, G=G, out_dtype=odt))
    assert_float_parity(out, oracle.qlinear_w4a4_asym(Xa, oWp, os_w, G), odt)


@pytest.mark.parametrize("G", [8, 32])
def test_w4_linears_small_groups_large_sampled(qa, G):
    """The W4A4 workload's shape (2048 x 4096 x 4096) with small groups: every
    row tile sampled, all columns."""
    M, K, N = 2048, 4096, 4096
    X, W, _ = synthetic.w4a4_inputs(M, K, N, seed=G)
    Wp, s_w, oWp, os_w = _weight(qa, W, G)
    rows = tile_rows(M, 128, extra=4, seed=G)
    out = as_f64(qa.qa_qlinear_w4a4(dev(X), Wp, s_w, G=G))
    assert_float_parity(out[rows], oracle.qlinear_w4a4(X, oWp, os_w, G, rows=rows), torch.float32)
    out = as_f64(qa.qa_qlinear_w4a8(dev(X), Wp, s_w, G=G))
    assert_float_parity(out[rows], oracle.qlinear_w4a8(X, oWp, os_w, G, rows=rows), torch.float32)
