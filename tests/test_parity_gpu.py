"""GPU parity: every libqa entry point against the CPU oracle on the same
seeded inputs.

Integer results (outlier sets, codes, scales, packed words, int32
accumulators) must match bit for bit.  Float outputs must satisfy
max |got - ref| <= 1e-3 * max |ref| (fp32 / fp16), and for bf16 outputs each
element may also differ by one bf16 ulp of its reference value.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def qa():
    import bit_quantized_linear_int8_amd as qa
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    qa.lib()
    return qa


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(a).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def as_f64(t):
    torch.cuda.synchronize()
    return t.float().cpu().numpy().astype(np.float64)


def tile_rows(M, tile=128, extra=0, seed=0):
    """First and last row of every `tile`-row block (so every row tile of a
    128-, 256- or larger-row tiling is reached), plus `extra` random rows."""
    rng = np.random.default_rng(seed)
    r = [np.arange(0, M, tile), np.arange(tile - 1, M, tile), [M - 1]]
    if extra:
        r.append(rng.choice(M, min(M, extra), replace=False))
    return np.unique(np.concatenate(r)).astype(np.int64)


def assert_float_parity(got, ref, dtype):
    ref = np.asarray(ref, np.float64)
    tol = 1e-3 * np.abs(ref).max()
    if dtype == torch.bfloat16:
        mag = np.abs(ref)
        ulp = np.where(mag > 0, 2.0 ** (np.floor(np.log2(np.maximum(mag, 1e-300))) - 7), 0.0)
        tol = np.maximum(tol, ulp)
    err = np.abs(got - ref)
    bad = err > tol
    assert not bad.any(), "max|diff| %g vs tol %g (%d elements over)" % (err.max(), np.max(tol), bad.sum())


ODT = {0: torch.float32, 1: torch.float16, 2: torch.bfloat16}


# ============================================================ outlier columns
@pytest.mark.parametrize("M,K", [(1, 8), (3, 40), (37, 520), (64, 512), (130, 1032), (257, 4096)])
@pytest.mark.parametrize("tau", [6.0, 0.5, -1.0, float("inf")])
def test_outlier_cols_shapes(qa, M, K, tau):
    X, _, _ = synthetic.mixed_inputs(M, K, 1, seed=M * 7 + K, n_dims=min(5, K // 8), p_token=0.5)
    X[0, 0] = 6.0                                   # exactly at the threshold
    mask, idx, count, colmax = qa.qa_outlier_cols(dev(X), tau)
    om, oidx, ocm = oracle.outlier_cols(X, tau)
    n = int(host(count)[0])
    assert n == len(oidx)
    assert np.array_equal(host(idx)[:n], oidx)
    assert np.array_equal(host(mask), om)
    assert np.array_equal(host(colmax), ocm)


@pytest.mark.parametrize("name", ["tiny_mixed", "decode_mixed", "prefill_mixed"])
def test_outlier_cols_configs(qa, name):
    c = synthetic.config(name)
    mask, idx, count, colmax = qa.qa_outlier_cols(dev(c["X"]), c["tau"])
    om, oidx, ocm = oracle.outlier_cols(c["X"], c["tau"])
    n = int(host(count)[0])
    assert np.array_equal(host(idx)[:n], oidx)
    assert np.array_equal(host(mask), om) and np.array_equal(host(colmax), ocm)
    assert set(c["dims"].tolist()) <= set(oidx.tolist())


def test_outlier_cols_reuses_dirty_scratch(qa):
    X, _, _ = synthetic.mixed_inputs(50, 1024, 1, seed=3, n_dims=4)
    scratch = torch.full((qa.qa_outlier_cols_workspace(1024),), 255, dtype=torch.uint8, device=DEV)
    for _ in range(2):
        mask, idx, count, colmax = qa.qa_outlier_cols(dev(X), 6.0, scratch=scratch)
        om, oidx, ocm = oracle.outlier_cols(X, 6.0)
        assert np.array_equal(host(idx)[: int(host(count)[0])], oidx)
        assert np.array_equal(host(colmax), ocm)


# ============================================================ row quantization
@pytest.mark.parametrize("rows,K", [(1, 8), (5, 24), (9, 520), (33, 1032), (17, 2056), (6, 4096), (4, 8200),
                                    (3, 8192), (2, 16392),
                                    # 16 chunks per lane over four waves, the last wave's chunks past the row
                                    (7, 6000)])
@pytest.mark.parametrize("with_mask", [False, True])
def test_rowquant_dynamic(qa, rows, K, with_mask):
    X, _, _ = synthetic.mixed_inputs(rows, K, 1, seed=rows + K, n_dims=min(4, K // 8), p_token=0.75)
    X[0, :] = 0                                          # an all-zero row -> safe scale 1.0
    mask = None
    if with_mask:
        mask = oracle.outlier_cols(X, 6.0)[0]
    Xq, s = qa.qa_quantize_rowwise_int8(dev(X), mask=None if mask is None else dev(mask))
    oq, os_ = oracle.quant_rows(X, mask=mask)
    assert np.array_equal(host(Xq), oq)
    assert np.array_equal(host(s), os_[:, 0])


def test_rowquant_ties_take_the_even_code(qa):
    # rows whose absmax is 127 (s = 1.0) and whose values sit exactly on x.5
    K = 64
    X = np.zeros((3, K), np.float16)
    X[:, 0] = 127.0
    X[0, 1:12] = [0.5, 1.5, 2.5, 3.5, -0.5, -1.5, -2.5, 100.5, -126.5, 63.5, 0.25]
    X[1, 0] = 63.5                                       # s = fl32(63.5 / 127) = 0.5
    X[1, 1:6] = [0.25, 0.75, 1.25, -0.25, 31.75]
    X[2, 1:4] = [126.5, -126.5, 125.5]
    Xq, s = qa.qa_quantize_rowwise_int8(dev(X))
    oq, os_ = oracle.quant_rows(X)
    assert np.array_equal(host(Xq), oq) and np.array_equal(host(s), os_[:, 0])
    assert host(Xq)[0, 1:8].tolist() == [0, 2, 2, 4, 0, -2, -2]


@pytest.mark.parametrize("q_min,q_max", [(-128, 127), (-127, 127), (0, 15), (-8, 7)])
# K = 264: one wave per row; 4096 and 6000: rows split over two and four waves
@pytest.mark.parametrize("K", [264, 4096, 6000])
def test_rowquant_static_affine(qa, q_min, q_max, K):
    rng = np.random.default_rng(q_max + K)
    X = (rng.normal(0, 4, (7, K))).astype(np.float16)
    X[0, :6] = [0.5, 1.5, 2.5, -0.5, -1.5, -2.5]
    s_in = rng.uniform(0.01, 1.0, 7).astype(np.float32)
    s_in[0] = 1.0
    z_in = rng.integers(-20, 20, 7).astype(np.int32)
    z_in[0] = 0
    mask = (rng.random(K) < 0.05).astype(np.uint8)
    Xq, _ = qa.qa_quantize_rowwise_int8(dev(X), mask=dev(mask), q_min=q_min, q_max=q_max, s_in=dev(s_in),
                                        z_in=dev(z_in))
    oq, _ = oracle.quant_rows(X, mask=mask, qmin=q_min, qmax=q_max, s_in=s_in, z_in=z_in)
    assert np.array_equal(host(Xq), oq)


@pytest.mark.parametrize("name", ["decode_mixed", "prefill_mixed"])
def test_weight_quant_configs(qa, name):
    c = synthetic.config(name)
    Wq, s_w = qa.qa_quantize_rowwise_int8(dev(c["W"]))
    oq, os_ = oracle.quant_rows(c["W"])
    assert np.array_equal(host(s_w), os_[:, 0])
    assert np.array_equal(host(Wq), oq)


# ============================================================ int8 GEMM, int32 accumulators
@pytest.mark.parametrize("M,K,N", [(1, 16, 1), (37, 80, 45), (64, 128, 64), (130, 272, 140), (300, 528, 200),
                                   (2048, 64, 2048), (1000, 400, 3000)])
def test_gemm_i8_i32(qa, M, K, N):
    rng = np.random.default_rng(M + K + N)
    A = rng.integers(-128, 128, (M, K), dtype=np.int8)
    B = rng.integers(-128, 128, (N, K), dtype=np.int8)
    C = host(qa.qa_gemm_i8_i32(dev(A), dev(B)))
    rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, size=min(M, 40), replace=False)]))
    assert np.array_equal(C[rows], oracle.gemm_i8_i32(A, B, rows=rows))


def test_gemm_i8_i32_big_tiles(qa):
    # enough 256 x 256 tiles to select the large-tile kernel, ragged in M, N, K
    M, K, N = 4100, 144, 8200
    rng = np.random.default_rng(11)
    A = rng.integers(-127, 128, (M, K), dtype=np.int8)
    B = rng.integers(-127, 128, (N, K), dtype=np.int8)
    C = host(qa.qa_gemm_i8_i32(dev(A), dev(B)))
    rows = tile_rows(M, 256, extra=8, seed=11)
    assert np.array_equal(C[rows], oracle.gemm_i8_i32(A, B, rows=rows))


@pytest.mark.parametrize("K", [64, 128, 192, 256, 320, 528])
def test_gemm_i8_i32_largest_tiles(qa, K):
    # >= 1024 tiles of 256 x 256 selects the largest tile; ragged M and N, and
    # every parity of the stage count of the software pipeline
    M, N = 8200, 8230
    rng = np.random.default_rng(K)
    A = rng.integers(-128, 128, (M, K), dtype=np.int8)
    B = rng.integers(-128, 128, (N, K), dtype=np.int8)
    C = host(qa.qa_gemm_i8_i32(dev(A), dev(B)))
    rows = tile_rows(M, 256, extra=8, seed=K)
    assert np.array_equal(C[rows], oracle.gemm_i8_i32(A, B, rows=rows))


# ============================================================ LLM.int8() mixed linear
def check_int8_stages(qa, ws, X, mask, oidx):
    """The integer stages a call left in its workspace -- outlier list and
    count, per-token scales, int8 codes (0 in the outlier columns) -- bit for
    bit against the oracle's outlier set and its row quantization with that
    mask."""
    M, K = X.shape
    o_idx, o_cnt, o_sx, o_xq = qa.qa_qlinear_int8_mixed_offsets(M, K)
    w = host(ws)
    cnt = int(w[o_cnt:o_cnt + 4].view(np.int32)[0])
    assert cnt == len(oidx), "outlier count %d vs %d" % (cnt, len(oidx))
    assert np.array_equal(w[o_idx:o_idx + 4 * cnt].view(np.int32), oidx)
    oq, os_ = oracle.quant_rows(X, mask=mask)
    assert np.array_equal(w[o_sx:o_sx + 4 * M].view(np.float32), os_[:, 0])
    got = w[o_xq:o_xq + M * K].view(np.int8).reshape(M, K)
    bad = np.argwhere(got != oq)
    assert bad.size == 0, "%d codes differ, first at %s" % (len(bad), bad[:4].tolist())


def _mixed_case(qa, X, W, tau, out_dtype, pass_w16, rows=None):
    Wq, s_w = qa.qa_quantize_rowwise_int8(dev(W))
    oWq, os_w = oracle.quant_rows(W)
    assert np.array_equal(host(Wq), oWq) and np.array_equal(host(s_w), os_w[:, 0])
    M, K = X.shape
    ws = torch.full((qa.qa_qlinear_int8_mixed_workspace(M, K),), 0x5A, dtype=torch.uint8, device=DEV)
    out = qa.qa_qlinear_int8_mixed(dev(X), Wq, s_w, W16=dev(W) if pass_w16 else None, threshold=tau,
                                   out_dtype=ODT[out_dtype], workspace=ws)
    om, oidx, _ = oracle.outlier_cols(X, tau)
    check_int8_stages(qa, ws, X, om, oidx)
    ref = oracle.qlinear_int8_mixed(X, oWq, os_w[:, 0], W16=W if pass_w16 else None, tau=tau, rows=rows)
    got = as_f64(out)
    if rows is not None:
        got = got[rows]
    assert_float_parity(got, ref, ODT[out_dtype])
    return out


@pytest.mark.parametrize("M,K,N", [(1, 16, 1), (5, 48, 7), (16, 256, 256), (33, 528, 77), (130, 1040, 300),
                                   (300, 272, 520)])
@pytest.mark.parametrize("tau", [6.0, float("inf"), -1.0])
@pytest.mark.parametrize("pass_w16", [True, False])
def test_mixed_shapes(qa, M, K, N, tau, pass_w16):
    X, W, _ = synthetic.mixed_inputs(M, K, N, seed=M * 31 + N, n_dims=min(5, K // 16), p_token=0.75)
    _mixed_case(qa, X, W, tau, 0, pass_w16)


@pytest.mark.parametrize("out_dtype", [0, 1, 2])
def test_mixed_out_dtypes(qa, out_dtype):
    X, W, _ = synthetic.mixed_inputs(40, 512, 96, seed=5, n_dims=3)
    _mixed_case(qa, X, W, 6.0, out_dtype, False)


def test_mixed_many_outliers(qa):
    # more than 32 outlier columns: several fp16 MFMA passes in the epilogue
    X, W, dims = synthetic.mixed_inputs(70, 1024, 130, seed=9, n_dims=75, p_token=0.5)
    _mixed_case(qa, X, W, 6.0, 0, True)


@pytest.mark.parametrize("M,K,N,n_dims,pass_w16", [
    (300, 2048, 520, 150, False),    # 96 < count <= 256: several staging passes from the compact rows
    (300, 2048, 520, 150, True),
    (600, 4096, 300, 256, False),    # exactly the compact-row capacity
    (70, 1024, 260, 300, False),     # count > 256: X gathered as well
    (40, 8208, 96, 20, True),        # K > 8192: rows not held in registers, X gathered
    (513, 1024, 1030, 40, False),    # big tiles with a tail launch, count between the prefetch and one pass
    (37, 8192, 130, 40, True),       # rows of 16 chunks per lane quantized by four waves each, compact rows
    (100, 6144, 260, 12, False),     # the same with a row shorter than the four waves' chunks
])
def test_mixed_outlier_staging_paths(qa, M, K, N, n_dims, pass_w16):
    X, W, dims = synthetic.mixed_inputs(M, K, N, seed=M + n_dims, n_dims=n_dims, p_token=0.6,
                                        magnitude=("uniform", 6.5, 60.0))
    _mixed_case(qa, X, W, 6.0, 1, pass_w16)


@pytest.mark.parametrize("M,K,N,n_dims,pass_w16,out_dtype", [
    (8, 8208, 100, 20, True, 1),     # K % 64 = 16: a partial last K step; three batches of steps (odd)
    (16, 12288, 33, 6, False, 0),    # K past the fused decode kernel: three batches, 16 tokens, ragged N
    (3, 1040, 300, 150, False, 1),   # more outlier columns than one staging pass (128)
    (13, 2064, 70, 300, True, 2),    # three staging passes, bf16 out
    (1, 8192, 17, 0, False, 1),      # no outlier columns, one token
])
def test_mixed_gemv_shapes(qa, M, K, N, n_dims, pass_w16, out_dtype):
    # decode-size calls (M <= 16) that the fused decode kernel does not take
    # run the int8 GEMM as a weight-streaming GEMV
    X, W, _ = synthetic.mixed_inputs(M, K, N, seed=M * 5 + K + n_dims, n_dims=n_dims, p_token=0.8,
                                     magnitude=("uniform", 6.5, 60.0))
    _mixed_case(qa, X, W, 6.0, out_dtype, pass_w16)


@pytest.mark.parametrize("M,K,N", [(1, 256, 1), (3, 512, 17), (4, 768, 40), (7, 1024, 33), (8, 4096, 64),
                                   (9, 2048, 48), (12, 256, 100), (16, 4096, 20),
                                   # K above 4096 (M <= 8): two 8-column chunks per thread
                                   (8, 8192, 48), (5, 6144, 40), (3, 4352, 17), (1, 8192, 100)])
@pytest.mark.parametrize("tau", [6.0, float("inf"), -1.0])
@pytest.mark.parametrize("pass_w16", [True, False])
def test_mixed_decode_kernel_shapes(qa, M, K, N, tau, pass_w16):
    # M <= 16 with K % 256 == 0, K <= 4096 (or M <= 8, K <= 8192) runs the fused single-kernel path
    X, W, _ = synthetic.mixed_inputs(M, K, N, seed=M * 13 + K + N, n_dims=6, magnitude=("abs_normal", 20.0),
                                     p_token=1.0)
    _mixed_case(qa, X, W, tau, 1, pass_w16)


@pytest.mark.parametrize("tau", [float("inf"), 90.0])
def test_mixed_decode_kernel_ties(qa, tau):
    # the fused decode kernel's exact fallback: rows whose scale is exactly 1
    # or 1/2 put many quotients on .5 ties, which round half to even
    rng = np.random.default_rng(23)
    M, K, N = 6, 1024, 48
    X = (rng.integers(-200, 201, (M, K)) * 0.5).astype(np.float16)     # multiples of 0.5 in [-100, 100]
    X[:, 7] = 127.0                                                      # absmax 127: s = 1
    X[1] = (rng.integers(-127, 128, K) * 0.25 + 0.25).astype(np.float16) # s = 1/2 with x / s = k + 0.5
    X[1, 7] = 63.5
    # one-hot weight rows: output (m, n) is s_x[m] * code(m, k_n) * s_w[n] * 127,
    # so a code off by one moves it by 1/127 of the largest output
    W = np.zeros((N, K), np.float16)
    W[np.arange(N), 20 * np.arange(N) + 3] = 1.0
    _mixed_case(qa, X, W, tau, 0, False)


@pytest.mark.parametrize("K", [4096, 8192])
def test_mixed_decode_kernel_many_outliers(qa, K):
    X, W, _ = synthetic.mixed_inputs(8, K, 96, seed=21 + K, n_dims=300, p_token=0.6)
    for dt in (0, 1, 2):
        _mixed_case(qa, X, W, 6.0, dt, False)


@pytest.mark.parametrize("tau", [6.0, 1e-3, 0.0, 65504.0, 100.0])
def test_mixed_decode_kernel_thresholds(qa, tau):
    """Thresholds that are and are not fp16 values, zero, the largest finite
    fp16 and values just below magnitudes present in X: the decode kernel
    compares fp16 patterns against the threshold's pattern, which must pick
    exactly the columns with max |x| > tau."""
    X, W, _ = synthetic.mixed_inputs(6, 1024, 40, seed=int(tau * 7) % 1000 + 3, n_dims=5,
                                     magnitude=("uniform", 6.0, 120.0))
    X[1, 5] = np.float16(6.0)
    X[2, 9] = np.float16(100.0)
    X[3, 11] = np.float16(np.nextafter(np.float16(100.0), np.float16(0)))
    X[0, 12] = np.float16(1e-3)
    _mixed_case(qa, X, W, tau, 0, True)


def test_mixed_decode_k8192_one_hot_codes(qa):
    """The pages' 8192 hidden size at decode (8 tokens), six planted outlier
    dims, threshold 6, a one-hot weight: every int8 code is visible in the
    output, and the integer stages are compared bit for bit."""
    X, _, _ = synthetic.mixed_inputs(8, 8192, 1, seed=77, n_dims=6, magnitude=("abs_normal", 20.0), p_token=1.0)
    N = 2048
    W = np.zeros((N, 8192), np.float16)
    W[np.arange(N), 4 * np.arange(N) + 1] = 1.0
    _mixed_case(qa, X, W, 6.0, 0, False)


def test_mixed_tiny_config(qa):
    c = synthetic.config("tiny_mixed")
    _mixed_case(qa, c["X"], c["W"], c["tau"], c["out_dtype"], c["pass_w16"])


def test_mixed_decode_config(qa):
    c = synthetic.config("decode_mixed")
    _mixed_case(qa, c["X"], c["W"], c["tau"], c["out_dtype"], c["pass_w16"])


def test_mixed_prefill_config_sampled(qa):
    c = synthetic.config("prefill_mixed")
    rows = tile_rows(c["M"], 128, extra=16)
    _mixed_case(qa, c["X"], c["W"], c["tau"], c["out_dtype"], c["pass_w16"], rows=rows)


@pytest.mark.parametrize("out_dtype", [0, 1])
def test_mixed_decode_config_one_hot_codes(qa, out_dtype):
    """The decode workload's X (8 x 4096, six planted outlier dims) with
    threshold 6 against a one-hot weight W[n][n] = 1 (N = K = 4096): output
    (m, n) is code(m, n) * s_x[m] (times w~ = 1 plus x in an outlier column),
    so one code off by one moves an output by s_x[m], about 1/127 of the row's
    largest output -- far outside the tolerance."""
    c = synthetic.config("decode_mixed")
    K = c["K"]
    W = np.zeros((K, K), np.float16)
    W[np.arange(K), np.arange(K)] = 1.0
    _mixed_case(qa, c["X"], W, 6.0, out_dtype, False)


@pytest.mark.parametrize("pass_w16", [False, True])
def test_mixed_tail_split(qa, pass_w16):
    """More 256 x 256 tiles than whole rounds over the 256 CUs: the trailing
    output columns go to a second launch of 128 x 128 tiles writing into the
    same output rows (ragged M and a ragged tail width)."""
    M, K, N = 300, 128, 129 * 256 + 72
    X, W, _ = synthetic.mixed_inputs(M, K, N, seed=5, n_dims=3, magnitude=("uniform", 6.0, 60.0))
    _mixed_case(qa, X, W, 6.0, 1, pass_w16)               # fp16 output


@pytest.mark.parametrize("M,K,N,n_dims,pass_w16,tau", [
    (2100, 528, 9000, 6, False, 6.0),        # 324 tiles, last K step partial, ragged M and N
    (768, 4112, 22000, 5, True, 6.0),        # 258 tiles, 65 K steps
    (1024, 1024, 17000, 150, False, 6.0),    # 268 tiles, 150 outlier columns: several staging passes
    (1030, 2048, 16500, 0, False, float("inf")),  # 325 tiles, no outlier columns
    (2048, 64, 11008, 0, True, -1.0),        # 344 tiles, K below one staging pass: every column an outlier
])
def test_mixed_partial_rounds(qa, M, K, N, n_dims, pass_w16, tau):
    """More 256 x 256 tiles than one round over the 256 CUs but not whole
    rounds (the trailing columns take a second launch of smaller tiles), with
    a partial last K step, ragged M and N and up to 150 outlier columns.
    Sampled rows from every tile row, all columns."""
    X, W, _ = synthetic.mixed_inputs(M, K, N, seed=M + N, n_dims=n_dims, p_token=0.7,
                                     magnitude=("uniform", 6.5, 60.0))
    rng = np.random.default_rng(M)
    rows = np.unique(np.concatenate([np.arange(0, M, 256), np.arange(255, M, 256), [M - 1],
                                     rng.choice(M, 6, replace=False)]))
    _mixed_case(qa, X, W, tau, 1, pass_w16, rows=rows)


def test_mixed_repeated_calls_one_workspace(qa):
    # consecutive calls with different data through the same workspace
    M, K, N = 600, 256, 30000
    ws = torch.empty(qa.qa_qlinear_int8_mixed_workspace(M, K), dtype=torch.uint8, device=DEV)
    for seed in (1, 2, 3):
        X, W, _ = synthetic.mixed_inputs(M, K, N, seed=seed, n_dims=4, magnitude=("uniform", 6.5, 60.0))
        Wq, s_w = qa.qa_quantize_rowwise_int8(dev(W))
        out = qa.qa_qlinear_int8_mixed(dev(X), Wq, s_w, out_dtype=torch.float32, workspace=ws)
        oWq, os_w = oracle.quant_rows(W)
        rows = np.array([0, 255, 256, 511, 599])
        ref = oracle.qlinear_int8_mixed(X, oWq, os_w[:, 0], tau=6.0, rows=rows)
        assert_float_parity(as_f64(out)[rows], ref, torch.float32)


def test_mixed_w8a8_config_sampled(qa):
    c = synthetic.config("w8a8_ffn")
    rows = tile_rows(c["M"], 256, extra=4, seed=1)
    _mixed_case(qa, c["X"], c["W"], c["tau"], c["out_dtype"], c["pass_w16"], rows=rows)


def test_mixed_empty_batch_and_layer(qa):
    W = np.zeros((8, 64), np.float16)
    Wq, s_w = qa.qa_quantize_rowwise_int8(dev(W))
    out = qa.qa_qlinear_int8_mixed(torch.zeros((0, 64), dtype=torch.float16, device=DEV), Wq, s_w)
    assert out.shape == (0, 8)
    out = qa.qa_qlinear_int8_mixed(torch.zeros((4, 64), dtype=torch.float16, device=DEV), Wq[:0], s_w[:0])
    assert out.shape == (4, 0)


def test_mixed_is_deterministic(qa):
    X, W, _ = synthetic.mixed_inputs(200, 1024, 300, seed=13, n_dims=6)
    Wq, s_w = qa.qa_quantize_rowwise_int8(dev(W))
    a = host(qa.qa_qlinear_int8_mixed(dev(X), Wq, s_w, out_dtype=torch.float32))
    b = host(qa.qa_qlinear_int8_mixed(dev(X), Wq, s_w, out_dtype=torch.float32))
    assert np.array_equal(a, b)


# ============================================================ Hadamard + int4
@pytest.mark.parametrize("G,per_group", [(G, False) for G in (1, 2, 4, 8, 16, 32, 64, 128, 256)] +
                         [(G, True) for G in (8, 16, 32, 64, 128, 256)])          # per-group scales need G >= 8
def test_hadamard_quant_int4(qa, G, per_group):
    rows, K = 13, max(G, 8) * 5
    X, _, _ = synthetic.w4a4_inputs(rows, K, 1, seed=G, n_dims=min(3, K // 16))
    X[1, :] = 0
    packed, s = qa.qa_hadamard_quant_int4(dev(X), G, per_group)
    op, os_ = oracle.hadamard_quant_int4(X, G, per_group)
    assert np.array_equal(host(s), os_)
    assert np.array_equal(host(packed).view(np.uint32), op)


@pytest.mark.parametrize("K", [1024, 2048, 4096, 8192])
@pytest.mark.parametrize("G", [8, 16, 32, 64, 128, 256])
def test_hadamard_quant_int4_row_in_registers(qa, K, G):
    """Per-row scales at K = 512 * NC * WPR: the row is held in registers by
    one or two waves, and all but the lowest chunk bits of a block are
    in-lane; 13 rows leave the last workgroup partly past the end."""
    X, _, _ = synthetic.w4a4_inputs(13, K, 1, seed=K + G)
    X[5, :] = 0
    packed, s = qa.qa_hadamard_quant_int4(dev(X), G, False)
    op, os_ = oracle.hadamard_quant_int4(X, G, False)
    assert np.array_equal(host(s), os_)
    assert np.array_equal(host(packed).view(np.uint32), op)


@pytest.mark.parametrize("K", [4096, 8192, 8448, 16384])
def test_hadamard_quant_int4_row_lengths(qa, K):
    X, _, _ = synthetic.w4a4_inputs(9, K, 1, seed=K)
    packed, s = qa.qa_hadamard_quant_int4(dev(X), 128, False)
    op, os_ = oracle.hadamard_quant_int4(X, 128, False)
    assert np.array_equal(host(s), os_) and np.array_equal(host(packed).view(np.uint32), op)


def test_hadamard_quant_int4_config(qa):
    c = synthetic.config("w4a4_hadamard")
    Wp, s_w = qa.qa_hadamard_quant_int4(dev(c["W"]), c["G"], True)
    oWp, os_w = oracle.hadamard_quant_int4(c["W"], c["G"], True)
    assert np.array_equal(host(s_w), os_w) and np.array_equal(host(Wp).view(np.uint32), oWp)
    Xp, s_x = qa.qa_hadamard_quant_int4(dev(c["X"]), c["G"], False)
    oXp, os_x = oracle.hadamard_quant_int4(c["X"], c["G"], False)
    assert np.array_equal(host(s_x), os_x) and np.array_equal(host(Xp).view(np.uint32), oXp)


# ============================================================ W4A4 GEMM
@pytest.mark.parametrize("M,K,N,G", [(1, 64, 1, 64), (20, 256, 33, 128), (64, 384, 64, 128), (130, 512, 70, 256),
                                     (300, 1024, 500, 64), (2048, 256, 2048, 128),
                                     # >= 256 tiles of 128 x 256 (eight-wave LDS-DMA kernel), ragged M and N,
                                     # K ending half-way through a 128-element stage
                                     (1030, 320, 7976, 64), (2100, 384, 4100, 128), (1100, 512, 7700, 256)])
def test_w4a4_group_acc(qa, M, K, N, G):
    rng = np.random.default_rng(M + N)
    Xp = rng.integers(0, 2 ** 32, (M, K // 8), dtype=np.uint64).astype(np.uint32)
    Wp = rng.integers(0, 2 ** 32, (N, K // 8), dtype=np.uint64).astype(np.uint32)
    acc = host(qa.qa_gemm_w4a4_group_acc(dev(Xp), dev(Wp), K, G))
    rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, size=min(M, 16), replace=False)]))
    assert np.array_equal(acc[rows], oracle.w4a4_group_acc(Xp, Wp, K, G, rows=rows))


@pytest.mark.parametrize("M,K,N,G", [(1, 128, 1, 128), (24, 512, 40, 128), (77, 768, 130, 256),
                                     (200, 1024, 300, 64)])
def test_w4a4_linear_shapes(qa, M, K, N, G):
    X, W, _ = synthetic.w4a4_inputs(M, K, N, seed=M + K)
    Wp, s_w = qa.qa_hadamard_quant_int4(dev(W), G, True)
    oWp, os_w = oracle.hadamard_quant_int4(W, G, True)
    assert np.array_equal(host(Wp).view(np.uint32), oWp)
    out = qa.qa_qlinear_w4a4(dev(X), Wp, s_w, G=G)
    assert_float_parity(as_f64(out), oracle.qlinear_w4a4(X, oWp, os_w, G), torch.float32)


@pytest.mark.parametrize("M,K,N,G", [(1030, 320, 7976, 64), (2100, 384, 4100, 128), (1100, 512, 7700, 256),
                                     # K / G x 256 > 8192: the block's scales do not fit the LDS table
                                     (2048, 8448, 4096, 64), (2050, 8192, 4100, 128)])
def test_w4a4_linear_large_sampled(qa, M, K, N, G):
    """Shapes with >= 256 tiles of 128 x 256 (the eight-wave LDS-DMA kernel):
    ragged M and N, K ending half-way through a stage; sampled rows."""
    X, W, _ = synthetic.w4a4_inputs(M, K, N, seed=M + G)
    Wp, s_w = qa.qa_hadamard_quant_int4(dev(W), G, True)
    oWp, os_w = oracle.hadamard_quant_int4(W, G, True)
    assert np.array_equal(host(Wp).view(np.uint32), oWp)
    out = as_f64(qa.qa_qlinear_w4a4(dev(X), Wp, s_w, G=G))
    rng = np.random.default_rng(M)
    rows = tile_rows(M, 128, extra=4, seed=M)
    assert_float_parity(out[rows], oracle.qlinear_w4a4(X, oWp, os_w, G, rows=rows), torch.float32)


def test_w4a4_config_sampled(qa):
    c = synthetic.config("w4a4_hadamard")
    G = c["G"]
    Wp, s_w = qa.qa_hadamard_quant_int4(dev(c["W"]), G, True)
    oWp, os_w = oracle.hadamard_quant_int4(c["W"], G, True)
    assert np.array_equal(host(Wp).view(np.uint32), oWp)
    out = as_f64(qa.qa_qlinear_w4a4(dev(c["X"]), Wp, s_w, G=G))
    rows = tile_rows(c["M"], 128, extra=8, seed=2)
    ref = oracle.qlinear_w4a4(c["X"], oWp, os_w, G, rows=rows)
    assert_float_parity(out[rows], ref, torch.float32)
    # int32 group accumulators of the same call, bit exact on sampled rows
    Xp, _ = qa.qa_hadamard_quant_int4(dev(c["X"]), G, False)
    acc = host(qa.qa_gemm_w4a4_group_acc(Xp, Wp, c["K"], G))
    oXp, _ = oracle.hadamard_quant_int4(c["X"], G, False)
    r = rows[::3]
    assert np.array_equal(acc[r], oracle.w4a4_group_acc(oXp, oWp, c["K"], G, rows=r))
