"""Every linear entry point gives one output, bit for bit, whether it runs
eagerly on the current stream, on a second stream, or from a captured HIP
graph replayed several times with other device work and synchronizations in
between.  The library allocates nothing and records no memset, so a graph
holds only its kernels and each replay must reproduce the eager result.
"""
import numpy as np
import pytest
import torch

import synthetic

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qa():
    import bit_quantized_linear_int8_amd as qa
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    qa.lib()
    return qa


def _ws(qa, name, M, K):
    return torch.empty(getattr(qa, name + "_workspace")(M, K), dtype=torch.uint8, device="cuda:0")


def _cases(qa):
    """(name, out tensor, call) with every input, output and workspace allocated up front."""
    dev = "cuda:0"
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    cases = []

    # LLM.int8() mixed: decode-sized (the single-launch decode kernel) and
    # prefill-sized (outlier scan, row quantizer, GEMM with the fp16 product)
    for M, K, N in [(8, 1024, 512), (520, 1024, 1040)]:
        X, W, _ = synthetic.mixed_inputs(M, K, N, seed=M)
        X, W16 = d(X), d(W)
        Wq, s_w = qa.qa_quantize_rowwise_int8(W16)
        out = torch.empty((M, N), dtype=torch.float16, device=dev)
        ws = _ws(qa, "qa_qlinear_int8_mixed", M, K)
        cases.append(("int8_mixed_%d" % M, out,
                      lambda X=X, Wq=Wq, s_w=s_w, out=out, ws=ws:
                      qa.qa_qlinear_int8_mixed(X, Wq, s_w, None, 6.0, out=out, workspace=ws)))

    M, K, N = 300, 1024, 520
    X, W, _ = synthetic.mixed_inputs(M, K, N, seed=3)
    X, W16 = d(X), d(W)
    Wq, s_w = qa.qa_quantize_rowwise_int8(W16)

    out_t = torch.empty((M, N), dtype=torch.float16, device=dev)
    ws_t = _ws(qa, "qa_qlinear_int8_topk", M, K)
    k = qa.topk_count(0.02, K)
    cases.append(("int8_topk", out_t, lambda: qa.qa_qlinear_int8_topk(X, Wq, s_w, k, out=out_t, workspace=ws_t)))

    s = qa.qa_smooth_factors(qa.qa_col_absmax(X), qa.qa_col_absmax(W16), 0.5)
    Wsq, s_ws = qa.qa_quantize_smooth_int8(W16, s, multiply=True)
    for per_tensor in (False, True):
        out_s = torch.empty((M, N), dtype=torch.float16, device=dev)
        ws_s = _ws(qa, "qa_qlinear_int8_smooth", M, K)
        cases.append(("int8_smooth_%s" % per_tensor, out_s,
                      lambda pt=per_tensor, out=out_s, ws=ws_s:
                      qa.qa_qlinear_int8_smooth(X, s, Wsq, s_ws, per_tensor=pt, out=out, workspace=ws)))

    Waq, s_wa, z_w, rw = qa.qa_quantize_rowwise_int8_asym(W16)
    out_a = torch.empty((M, N), dtype=torch.float16, device=dev)
    ws_a = _ws(qa, "qa_qlinear_int8_asym", M, K)
    cases.append(("int8_asym", out_a,
                  lambda: qa.qa_qlinear_int8_asym(X, Waq, s_wa, rw, z_w=z_w, out=out_a, workspace=ws_a)))

    # W4 paths; 2048 x 4096 x 4096 at G = 128 puts W4A4 on its LDS-DMA kernel
    for M, K, N, G in [(96, 1024, 384, 128), (2048, 1024, 4096, 128)]:
        X4, W4, _ = synthetic.w4a4_inputs(M, K, N, seed=K + M)
        X4 = d(X4)
        Wp, s_w4 = qa.qa_hadamard_quant_int4(d(W4), G, True)
        out4 = torch.empty((M, N), dtype=torch.float32, device=dev)
        ws4 = _ws(qa, "qa_qlinear_w4a4", M, K)
        cases.append(("w4a4_%d" % M, out4,
                      lambda X4=X4, Wp=Wp, s_w4=s_w4, out=out4, ws=ws4, G=G:
                      qa.qa_qlinear_w4a4(X4, Wp, s_w4, G=G, out=out, workspace=ws)))
        out8 = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        ws8 = _ws(qa, "qa_qlinear_w4a8", M, K)
        cases.append(("w4a8_%d" % M, out8,
                      lambda X4=X4, Wp=Wp, s_w4=s_w4, out=out8, ws=ws8, G=G:
                      qa.qa_qlinear_w4a8(X4, Wp, s_w4, G=G, out=out, workspace=ws)))
        Xa = X4.abs()
        c_w = qa.qa_w4_column_terms(Wp, s_w4, K, G)
        outz = torch.empty((M, N), dtype=torch.float16, device=dev)
        wsz = _ws(qa, "qa_qlinear_w4a4_asym", M, K)
        cases.append(("w4a4_asym_%d" % M, outz,
                      lambda Xa=Xa, Wp=Wp, s_w4=s_w4, c_w=c_w, out=outz, ws=wsz, G=G:
                      qa.qa_qlinear_w4a4_asym(Xa, Wp, s_w4, c_w, G=G, out=out, workspace=ws)))

    M, K, N, G = 200, 1024, 256, 128
    Xk, Wk, _ = synthetic.w4a4_inputs(M, K, N, seed=11)
    P1, P2 = (d(p) for p in synthetic.kron_factors(32, 32, seed=5))
    Xk = d(Xk)
    Wpk, s_wk = qa.qa_kron_quant_int4(d(Wk), P1, P2, G=G)
    outk = torch.empty((M, N), dtype=torch.float32, device=dev)
    wsk = _ws(qa, "qa_qlinear_kron_w4a4", M, K)
    cases.append(("kron_w4a4", outk,
                  lambda: qa.qa_qlinear_kron_w4a4(Xk, P1, P2, Wpk, s_wk, G=G, out=outk, workspace=wsk)))
    return cases


def _bits(t):
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32).cpu().numpy()


def test_side_stream_and_graph_replays(qa):
    cases = _cases(qa)
    torch.cuda.synchronize()
    eager = {}
    for name, out, call in cases:
        out.fill_(7)
        call()
        torch.cuda.synchronize()
        eager[name] = _bits(out)
        assert np.isfinite(out.float().cpu().numpy()).all(), name

    side = torch.cuda.Stream()                       # default priority
    for name, out, call in cases:
        out.fill_(7)
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            call()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(out), eager[name]), "second stream: " + name

    # capture every call into one graph (warmed up on a side stream first, as
    # torch requires), then replay it with eager work between the replays
    warm = torch.cuda.Stream()
    warm.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(warm):
        for _, _, call in cases:
            call()
    torch.cuda.current_stream().wait_stream(warm)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _, _, call in cases:
            call()
    scratch = torch.empty(1 << 22, dtype=torch.float32, device="cuda:0")
    for rep in range(4):
        for _, out, _ in cases:
            out.fill_(rep + 1.0)                     # eager work that the replay must overwrite
        scratch.normal_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, out, _ in cases:
            assert np.array_equal(_bits(out), eager[name]), "graph replay %d: %s" % (rep, name)


def test_stream_argument_keeps_internal_buffers_on_that_stream(qa):
    """A call given stream= (not the current stream) allocates its output and
    workspace on that stream, so when the workspace is released at return the
    caching allocator does not hand it to work queued on the current stream
    while the call's kernels, held back on the busy side stream, still use
    it.  The current stream re-allocates and overwrites blocks of the
    workspace's size right after each call; every result must equal the
    eager one bit for bit."""
    dev = "cuda:0"
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    M, K, N = 520, 1024, 1040
    X, W, _ = synthetic.mixed_inputs(M, K, N, seed=17, n_dims=5)
    X, W16 = d(X), d(W)
    Wq, s_w = qa.qa_quantize_rowwise_int8(W16)
    ref = _bits(qa.qa_qlinear_int8_mixed(X, Wq, s_w, threshold=6.0, out_dtype=torch.float16))
    nbytes = qa.qa_qlinear_int8_mixed_workspace(M, K)
    side = torch.cuda.Stream()                       # default priority
    a = torch.randn(3072, 3072, device=dev)
    torch.cuda.synchronize()
    for trial in range(3):
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            busy = a @ a                             # the side stream is still busy when the call returns
        out = qa.qa_qlinear_int8_mixed(X, Wq, s_w, threshold=6.0, out_dtype=torch.float16, stream=side)
        junk = [torch.full((nbytes,), 0xA5, dtype=torch.uint8, device=dev) for _ in range(4)]
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(out), ref), "trial %d" % trial
        del busy, junk
