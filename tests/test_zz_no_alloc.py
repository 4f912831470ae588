"""The LLM.int8() entry point without a workspace (static per-GPU scratch)
against qa_qlinear_int8_mixed with a workspace: the same kernels, so the
outputs must agree bit for bit -- on consecutive calls through the one
scratch, each later call smaller than the one before (stale contents of a
larger call must not leak into a smaller one), on the general path (outlier
scan, row quantizer, GEMM) and the fused decode kernel."""
import ctypes

import numpy as np
import pytest
import torch

import synthetic

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def qa():
    import bit_quantized_linear_int8_amd as qa
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    qa.lib()
    return qa


def _bits(t):
    torch.cuda.synchronize()
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32).cpu().numpy()


def _inputs(qa, M, K, N, seed, n_dims):
    X, W, _ = synthetic.mixed_inputs(M, K, N, seed=seed, n_dims=n_dims, magnitude=("uniform", 6.5, 60.0))
    X = torch.from_numpy(X).to(DEV)
    W16 = torch.from_numpy(W).to(DEV)
    Wq, s_w = qa.qa_quantize_rowwise_int8(W16)
    return X, W16, Wq, s_w


@pytest.mark.parametrize("shapes", [
    [(1100, 2048, 1500, 12), (300, 1024, 520, 5)],           # general path, then a smaller general call
    [(8, 4096, 1024, 6), (3, 1024, 200, 4)],                 # fused decode kernel twice
    [(2048, 4096, 1024, 7), (8, 4096, 512, 6)],              # general path, then the decode kernel
])
def test_noalloc_matches_workspace_call(qa, shapes):
    L = qa.lib()
    for i, (M, K, N, n_dims) in enumerate(shapes):
        X, W16, Wq, s_w = _inputs(qa, M, K, N, seed=M + i, n_dims=n_dims)
        for dt, w16 in ((torch.float16, None), (torch.float32, W16)):
            ref = qa.qa_qlinear_int8_mixed(X, Wq, s_w, W16=w16, threshold=6.0, out_dtype=dt)
            out = torch.full((M, N), 7.0, dtype=dt, device=DEV)
            st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            s = L.qa_qlinear_int8_mixed_noalloc(ctypes.c_void_p(X.data_ptr()), M, K, ctypes.c_void_p(Wq.data_ptr()),
                                                ctypes.c_void_p(s_w.data_ptr()),
                                                None if w16 is None else ctypes.c_void_p(w16.data_ptr()), N, 6.0,
                                                ctypes.c_void_p(out.data_ptr()), {torch.float16: 1, torch.float32: 0}[dt],
                                                st)
            assert s == 0, qa.last_error()
            assert np.array_equal(_bits(out), _bits(ref)), "call %d %s" % (i, (M, K, N, dt))
            assert np.isfinite(out.float().cpu().numpy()).all()


def test_noalloc_binding_and_size_limit(qa):
    X, W16, Wq, s_w = _inputs(qa, 64, 512, 96, seed=3, n_dims=3)
    out = torch.empty((64, 96), dtype=torch.float16, device=DEV)
    qa.qa_qlinear_int8_mixed_noalloc(X, Wq, s_w, out, threshold=6.0)
    ref = qa.qa_qlinear_int8_mixed(X, Wq, s_w, threshold=6.0)
    assert np.array_equal(_bits(out), _bits(ref))
    # beyond the static scratch: rejected before anything runs
    assert qa.qa_qlinear_int8_mixed_workspace(4096, 16384) > qa.NOALLOC_SCRATCH_BYTES
    L = qa.lib()
    P = ctypes.c_void_p(0x10000)
    assert L.qa_qlinear_int8_mixed_noalloc(P, 4096, 16384, P, P, None, 64, 6.0, P, 1, None) == 5
    assert "static scratch" in qa.last_error()
