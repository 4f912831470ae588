"""Edge cases of the entry points on the GPU: empty batches (M = 0) and empty
layers (N = 0) for every linear and quantizer, and the LLM.int8() linear at
the largest K the boundary accepts (131072), against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from test_parity_gpu import DEV, _mixed_case, dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qa():
    import bit_quantized_linear_int8_amd as qa
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    qa.lib()
    return qa


def test_quantizers_with_no_rows(qa):
    K, G = 256, 128
    X0 = torch.zeros((0, K), dtype=torch.float16, device=DEV)
    q, s = qa.qa_quantize_rowwise_int8(X0)
    assert q.shape == (0, K) and s.shape == (0,)
    r = qa.qa_quantize_rowwise_int8_asym(X0)
    assert r[0].shape == (0, K)
    p, s = qa.qa_hadamard_quant_int4(X0, G, True)
    assert p.shape == (0, K // 8) and s.shape == (0, K // G)
    p, s = qa.qa_hadamard_quant_int4(X0, G, False)
    assert p.shape == (0, K // 8)
    q, s = qa.qa_hadamard_quant_int8(X0, G)
    assert q.shape == (0, K)
    r = qa.qa_hadamard_quant_int4_asym(X0, G)
    assert r[0].shape == (0, K // 8)
    P1, P2 = (dev(p) for p in synthetic.kron_factors(16, 16, seed=1))
    p, s = qa.qa_kron_quant_int4(X0, P1, P2)
    assert p.shape == (0, K // 8)
    smooth = torch.ones(K, dtype=torch.float32, device=DEV)
    q, s = qa.qa_quantize_smooth_int8(X0, smooth)
    assert q.shape == (0, K)
    torch.cuda.synchronize()


def test_linears_with_empty_batch_or_layer(qa):
    M, K, N, G = 6, 512, 40, 128
    X, W, _ = synthetic.mixed_inputs(M, K, N, seed=2)
    X, W16 = dev(X), dev(W)
    Wq, s_w = qa.qa_quantize_rowwise_int8(W16)
    Waq, s_wa, z_w, rw = qa.qa_quantize_rowwise_int8_asym(W16)
    sm = qa.qa_smooth_factors(qa.qa_col_absmax(X), qa.qa_col_absmax(W16), 0.5)
    Wsq, s_ws = qa.qa_quantize_smooth_int8(W16, sm, multiply=True)
    Wp, s_w4 = qa.qa_hadamard_quant_int4(W16, G, True)
    c_w = qa.qa_w4_column_terms(Wp, s_w4, K, G)
    P1, P2 = (dev(p) for p in synthetic.kron_factors(16, 32, seed=3))
    Wpk, s_wk = qa.qa_kron_quant_int4(W16, P1, P2, G=G)

    def run(X, n):                               # every linear on X against the first n output channels
        return [
            qa.qa_qlinear_int8_mixed(X, Wq[:n], s_w[:n]),
            qa.qa_qlinear_int8_topk(X, Wq[:n], s_w[:n], 5),
            qa.qa_qlinear_int8_asym(X, Waq[:n], s_wa[:n], rw[:n], z_w=z_w[:n]),
            qa.qa_qlinear_int8_smooth(X, sm, Wsq[:n], s_ws[:n]),
            qa.qa_qlinear_int8_smooth(X, sm, Wsq[:n], s_ws[:n], per_tensor=True),
            qa.qa_qlinear_w4a4(X, Wp[:n], s_w4[:n], G=G),
            qa.qa_qlinear_w4a8(X, Wp[:n], s_w4[:n], G=G),
            qa.qa_qlinear_w4a4_asym(X.abs(), Wp[:n], s_w4[:n], c_w[:n], G=G),
            qa.qa_qlinear_kron_w4a4(X, P1, P2, Wpk[:n], s_wk[:n], G=G),
        ]

    for out in run(X[:0], N):                    # no tokens
        assert out.shape == (0, N)
    for out in run(X, 0):                        # no output channels
        assert out.shape == (M, 0)
    torch.cuda.synchronize()
    full = run(X, N)                             # and the same objects still give full-size results
    for out in full:
        assert out.shape == (M, N) and torch.isfinite(out.float()).all()


@pytest.mark.parametrize("M", [8, 40])
def test_mixed_largest_k(qa, M):
    # K = 131072, the boundary's largest: past the fused decode kernel's K, so
    # both token counts take the general path (scan, row quantizer, GEMM)
    K, N = 131072, 48
    X, W, dims = synthetic.mixed_inputs(M, K, N, seed=M + 7, n_dims=9)
    _mixed_case(qa, X, W, 6.0, 1, False)
    _mixed_case(qa, X, W, 6.0, 0, True)
