"""Pins of the CPU oracle to what the pages and the mathematics fix.

Nothing here compares the oracle with itself: every check goes against a
value printed on a page (tests/golden), a closed form, a library routine
(numpy, scipy, torch CPU) computing the same quantity another way, a special
case that reduces to a textbook operation, or a rigorous error bound.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.linalg
from hypothesis import given, settings, strategies as st

import oracle
import synthetic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------ formats
def test_f16_decode_all_bit_patterns_match_numpy():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_f16_encode_matches_numpy_rounding():
    rng = np.random.default_rng(1)
    vals = np.concatenate([
        rng.normal(0, 1, 4000), rng.normal(0, 3e4, 2000), rng.normal(0, 1e-5, 2000),
        rng.normal(0, 1e-7, 1000),
        # exact ties between neighbouring fp16 values, normal and subnormal
        1.0 + np.arange(1, 200, 2) * 2.0 ** -11, np.arange(1, 200, 2) * 2.0 ** -25,
        [65504.0, 65519.99, 65520.0, 70000.0, -65520.0, 0.0, -0.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26],
    ])
    ref = vals.astype(np.float16).view(np.uint16)
    got = np.array([oracle.f64_to_f16_bits(v) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, ref)
    # ties go to the even neighbour
    assert oracle.f64_to_f16_bits(1.0 + 2.0 ** -11) == 0x3C00
    assert oracle.f64_to_f16_bits(1.0 + 3 * 2.0 ** -11) == 0x3C02


def test_bf16_encode_matches_torch_rounding():
    import torch
    rng = np.random.default_rng(2)
    f32 = np.concatenate([rng.normal(0, 1, 4000), rng.normal(0, 1e30, 500), rng.normal(0, 1e-39, 500),
                          1.0 + np.arange(1, 100, 2) * 2.0 ** -8]).astype(np.float32)
    ref = torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.f64_to_bf16_bits(float(v)) for v in f32], dtype=np.uint16)
    assert np.array_equal(got, ref)
    assert oracle.f64_to_bf16_bits(1.0 + 2.0 ** -8) == 0x3F80          # tie -> even
    assert oracle.f64_to_bf16_bits(3.4e38) == 0x7F80 or oracle.f64_to_bf16_bits(3.4e38) == 0x7F7F
    assert oracle.f64_to_bf16_bits(1e39) == 0x7F80                     # overflow -> inf


# ------------------------------------------------------------------ worked examples
@pytest.mark.parametrize("as_f16", [False, True])
def test_scale_example_int4(as_f16):
    g = golden("scale_example.json")
    x = np.array(g["W"], np.float16 if as_f16 else np.float32)
    q, s = oracle.quant_rows(x, qmin=g["q_min"], qmax=g["q_max"])
    s = float(s[0, 0])
    assert round(s, g["s_printed_digits"]) == g["s_printed"]
    assert s == np.float32(np.float32(np.abs(x.astype(np.float32)).max()) / np.float32(7))
    i = g["W"].index(g["x_printed"])
    assert q[0, i] == g["q_printed"]
    assert round(q[0, i] * s, g["dequant_printed_digits"]) == g["dequant_printed"]
    # the remaining codes follow from the same rule: -0.7/s = -5.44, -0.3/s = -2.33, 0.1/s = 0.78, 0.9/s = 7
    assert q[0].tolist() == [-5, -2, 1, 3, 7]


def test_outlier_collapse_example():
    g = golden("outlier_example.json")
    q, s = oracle.quant_rows(np.array(g["x"], np.float32), qmin=g["q_min"], qmax=g["q_max"])
    assert round(float(s[0, 0]), g["s_printed_digits"]) == g["s_printed"]
    assert q[0].tolist() == g["codes_printed"]


def test_llm_int8_4096_example():
    g = golden("llm_int8_4096.json")
    rng = np.random.default_rng(3)
    x = rng.uniform(-1, 1, g["hidden"]).astype(np.float16)
    x[0], x[1] = 1.0, -1.0                       # ordinary channels reach exactly +-1
    x[g["outlier_dim"]] = g["outlier_value"]
    X = x[None, :]
    # undecomposed: one scale over everything
    q, s = oracle.quant_rows(X)
    s = float(s[0, 0])
    assert round(s, g["s_undecomposed_digits"]) == g["s_undecomposed_printed"]
    assert abs(int(q[0, 0])) in g["levels_undecomposed_printed"] and q[0, 0] == -q[0, 1]
    assert set(np.abs(q[0, 2:g["outlier_dim"]]).tolist()) <= {0, 1, 2}
    # decomposed at threshold 6.0
    mask, idx, colmax = oracle.outlier_cols(X, g["threshold"])
    assert idx.tolist() == [g["outlier_dim"]]
    q2, s2 = oracle.quant_rows(X, mask=mask)
    s2 = float(s2[0, 0])
    assert round(s2, g["s_split_digits"]) == g["s_split_printed"]
    assert q2[0, 0] == g["level_split_printed"] and q2[0, 1] == -g["level_split_printed"]
    assert q2[0, g["outlier_dim"]] == 0


def test_affine_static_mode_closed_form():
    # q = clip(round(x/s) + z, qmin, qmax) with ties to even (模型推理量化 §6.2)
    q, _ = oracle.quant_rows(np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5], np.float32),
                             s_in=[1.0], z_in=[0], qmin=-128, qmax=127)
    assert q[0].tolist() == [0, 2, 2, 0, -2, -2]
    q, _ = oracle.quant_rows(np.array([1.0, -1.0, 100.0, -300.0], np.float32),
                             s_in=[0.5], z_in=[3], qmin=-128, qmax=127)
    assert q[0].tolist() == [5, 1, 127, -128]


def test_zero_row_gets_safe_scale():
    q, s = oracle.quant_rows(np.zeros((2, 16), np.float16))
    assert s.ravel().tolist() == [1.0, 1.0] and not q.any()


def test_int4_packing_words():
    # codes of the two 模型推理量化 examples (§4, §5), zero-padded to 8, plus a
    # sign pattern; element i of a word sits in bits [4i+3:4i].
    cases = [([-5, -2, 1, 3, 7, 0, 0, 0], 0x000731EB),
             ([0, 0, 0, 0, 0, 7, 0, 0], 0x00700000),
             ([1, -1, 2, -2, 3, -3, 7, -7], 0x97D3E2F1),
             ([-8, 7, 0, 0, 0, 0, 0, -1], 0xF0000078)]
    for codes, word in cases:
        assert int(oracle.pack_int4(np.array(codes))[0, 0]) == word
        assert oracle.unpack_int4(np.array([word], np.uint32), 8)[0].tolist() == codes


def test_int4_quant_via_identity_rotation_matches_examples():
    g = golden("scale_example.json")
    x = np.zeros(8, np.float16)
    x[:5] = g["W"]
    packed, s = oracle.hadamard_quant_int4(x, G=1, per_group=False)
    assert int(packed[0, 0]) == 0x000731EB
    assert round(float(s[0, 0]), 4) == g["s_printed"]


# ------------------------------------------------------------------ outlier set
def test_outlier_cols_match_numpy_definition():
    rng = np.random.default_rng(4)
    for M, K in [(1, 8), (7, 64), (33, 300)]:
        X = rng.normal(0, 3, (M, K)).astype(np.float16)
        X[0, 0] = 6.0                 # exactly at the threshold: not an outlier
        X[-1, -1] = np.float16(-6.0039)
        for tau in (6.0, 0.0, -1.0, float("inf")):
            mask, idx, colmax = oracle.outlier_cols(X, tau)
            cm = np.abs(X.astype(np.float32)).max(axis=0)
            assert np.array_equal(colmax, cm)
            assert idx.tolist() == np.nonzero(cm > np.float32(tau))[0].tolist()
            assert np.array_equal(mask, (cm > np.float32(tau)).astype(np.uint8))
        assert 0 not in oracle.outlier_cols(X[:, :1] * 0 + np.float16(6.0), 6.0)[1]


def test_planted_outlier_sets():
    c = synthetic.config("tiny_mixed")
    assert oracle.outlier_cols(c["X"], 6.0)[1].tolist() == [17, 200]
    X, W, dims = synthetic.mixed_inputs(64, 1024, 8, seed=5, n_dims=7)
    assert set(dims.tolist()) <= set(oracle.outlier_cols(X, 6.0)[1].tolist())


# ------------------------------------------------------------------ integer GEMM
@settings(max_examples=40, deadline=None)
@given(M=st.integers(1, 40), K=st.integers(1, 300), N=st.integers(1, 70), seed=st.integers(0, 2 ** 31))
def test_gemm_i8_bruteforce(M, K, N, seed):
    rng = np.random.default_rng(seed)
    A = rng.integers(-128, 128, (M, K), dtype=np.int8)
    B = rng.integers(-128, 128, (N, K), dtype=np.int8)
    C = oracle.gemm_i8_i32(A, B)
    assert np.array_equal(C, A.astype(np.int64) @ B.astype(np.int64).T)
    rows = rng.choice(M, size=min(M, 3), replace=False)
    assert np.array_equal(oracle.gemm_i8_i32(A, B, rows=rows), C[rows])


def test_gemm_i8_overflow_detected():
    K = 131073                               # 131073 * 128^2 > 2^31 - 1
    A = np.full((1, K), -128, np.int8)
    with pytest.raises(OverflowError):
        oracle.gemm_i8_i32(A, A)


# ------------------------------------------------------------------ mixed linear
def _w8(W):
    Wq, s_w = oracle.quant_rows(W)
    return Wq, s_w[:, 0]


def test_mixed_tau_inf_is_plain_vectorwise_w8a8():
    X, W, _ = synthetic.mixed_inputs(24, 512, 40, seed=6, n_dims=3)
    Wq, s_w = _w8(W)
    out = oracle.qlinear_int8_mixed(X, Wq, s_w, tau=float("inf"))
    Xq, s_x = oracle.quant_rows(X)
    C = Xq.astype(np.int64) @ Wq.astype(np.int64).T
    ref = C.astype(np.float64) * s_x.astype(np.float64) * s_w.astype(np.float64)[None, :]
    assert np.array_equal(out, ref)


def test_mixed_all_outliers_is_plain_fp16_gemm():
    X, W, _ = synthetic.mixed_inputs(12, 256, 30, seed=7, n_dims=2)
    Wq, s_w = _w8(W)
    X64, W64 = X.astype(np.float64), W.astype(np.float64)
    out = oracle.qlinear_int8_mixed(X, Wq, s_w, W16=W, tau=-1.0)
    mag = np.abs(X64) @ np.abs(W64).T
    assert np.all(np.abs(out - X64 @ W64.T) <= 1e-13 * mag + 1e-300)
    # without W16 the fp16 weights are fp16(fp32(s_w * Wq))
    wt = (s_w[:, None] * Wq.astype(np.float32)).astype(np.float16).astype(np.float64)
    out2 = oracle.qlinear_int8_mixed(X, Wq, s_w, tau=-1.0)
    assert np.all(np.abs(out2 - X64 @ wt.T) <= 1e-13 * (np.abs(X64) @ np.abs(wt).T) + 1e-300)


def _mixed_error_bound(X, W, tau, w16_given):
    """Rigorous bound on |out - X W^T| from |x - s q| <= s/2 per code."""
    X32 = X.astype(np.float32)
    W32 = W.astype(np.float32)
    cm = np.abs(X32).max(axis=0)
    O = cm > np.float32(tau)
    a_x = np.where(O[None, :], 0, np.abs(X32)).max(axis=1)
    s_x = np.where(a_x == 0, np.float32(1), a_x / np.float32(127)).astype(np.float64)
    a_w = np.abs(W32).max(axis=1)
    s_w = np.where(a_w == 0, np.float32(1), a_w / np.float32(127)).astype(np.float64)
    aX = np.abs(X.astype(np.float64))
    aW = np.abs(W.astype(np.float64))
    nonO = (~O).astype(np.float64)
    B = 0.5 * s_x[:, None] * ((aW * nonO) @ np.ones(X.shape[1]) + 0.5 * s_w * nonO.sum())[None, :] \
        + 0.5 * (aX * nonO) @ np.ones(X.shape[1])[:, None] * s_w[None, :]
    if not w16_given:
        On = O.astype(np.float64)
        B = B + (aX * On) @ (0.5 * s_w[:, None] + (aW + 0.5 * s_w[:, None]) * 2.0 ** -10).T * On.any()
    return B * (1 + 1e-5) + 1e-12


@pytest.mark.parametrize("w16_given", [True, False])
def test_mixed_within_quantization_error_bound(w16_given):
    X, W, dims = synthetic.mixed_inputs(40, 768, 56, seed=8, n_dims=5, p_token=0.75)
    Wq, s_w = _w8(W)
    out = oracle.qlinear_int8_mixed(X, Wq, s_w, W16=W if w16_given else None, tau=6.0)
    exact = X.astype(np.float64) @ W.astype(np.float64).T
    B = _mixed_error_bound(X, W, 6.0, w16_given)
    assert np.all(np.abs(out - exact) <= B)
    # the bound is tight enough that dropping the outlier part breaks it
    Xn = X.copy()
    Xn[:, dims] = 0
    no_outl = oracle.qlinear_int8_mixed(Xn, Wq, s_w, W16=W, tau=6.0)
    assert np.any(np.abs(no_outl - exact) > B)


def test_mixed_row_sampling_matches_full():
    X, W, _ = synthetic.mixed_inputs(20, 256, 24, seed=9, n_dims=3)
    Wq, s_w = _w8(W)
    full = oracle.qlinear_int8_mixed(X, Wq, s_w, tau=6.0)
    rows = np.array([19, 0, 7])
    assert np.array_equal(oracle.qlinear_int8_mixed(X, Wq, s_w, tau=6.0, rows=rows), full[rows])


def test_decomposition_lowers_error():
    c = synthetic.config("tiny_mixed")
    X, W = c["X"], c["W"]
    Wq, s_w = _w8(W)
    exact = X.astype(np.float64) @ W.astype(np.float64).T
    e_split = np.abs(oracle.qlinear_int8_mixed(X, Wq, s_w, W16=W, tau=6.0) - exact).max()
    e_plain = np.abs(oracle.qlinear_int8_mixed(X, Wq, s_w, W16=W, tau=float("inf")) - exact).max()
    assert e_split < e_plain / 3


def test_output_rounding():
    x = np.array([1.0, 1.0 + 2.0 ** -11, -70000.0, 1e-8, 3.0 + 2.0 ** -30])
    assert np.array_equal(oracle.round_output(x, oracle.F16), x.astype(np.float16).view(np.uint16))
    assert np.array_equal(oracle.round_output(x, oracle.F32), x.astype(np.float32))


# ------------------------------------------------------------------ Hadamard
@pytest.mark.parametrize("G", [1, 2, 4, 8, 16, 32, 64, 128, 256])
def test_hadamard_orthogonal_and_sylvester(G):
    H = np.array([[oracle.hadamard_entry(i, j) for j in range(G)] for i in range(G)], np.int64)
    assert np.array_equal(H @ H.T, G * np.eye(G, dtype=np.int64))
    assert np.array_equal(H, scipy.linalg.hadamard(G))


@pytest.mark.parametrize("G", [1, 8, 64, 128, 256])
def test_hadamard_rows_match_scipy_exactly(G):
    X, _, _ = synthetic.mixed_inputs(6, 512, 1, seed=10 + G, n_dims=4, magnitude=("uniform", 50, 60000))
    X[0, :8] = [65504, -65504, 2 ** -24, -(2 ** -24), 6e-5, 1, -1, 0]
    H = scipy.linalg.hadamard(G).astype(np.float64)
    c = 1.0 / math.sqrt(G)
    ref = ((X.astype(np.float64).reshape(6, -1, G) @ H) * c).astype(np.float32).reshape(6, 512)
    assert np.array_equal(oracle.hadamard_rows(X, G), ref)


def test_hadamard_constant_row():
    x = np.ones(128, np.float16)
    y = oracle.hadamard_rows(x, 128)[0]
    assert y[0] == np.float32(128 * (1.0 / math.sqrt(128.0))) and not y[1:].any()
    packed, s = oracle.hadamard_quant_int4(x, 128, per_group=False)
    codes = oracle.unpack_int4(packed, 128)[0]
    assert codes[0] == 7 and not codes[1:].any()


def test_rotation_cancels_in_the_product():
    X, W = synthetic.w4a4_inputs(16, 512, 24, seed=11)[:2]
    Xr = oracle.hadamard_rows(X, 128).astype(np.float64)
    Wr = oracle.hadamard_rows(W, 128).astype(np.float64)
    exact = X.astype(np.float64) @ W.astype(np.float64).T
    mag = np.abs(X.astype(np.float64)) @ np.abs(W.astype(np.float64)).T
    assert np.all(np.abs(Xr @ Wr.T - exact) <= 2.0 ** -21 * mag * 16)


# ------------------------------------------------------------------ W4A4
def _unpack_np(p, K):
    p = p.astype(np.uint64)
    nib = ((p[..., None] >> (4 * np.arange(8, dtype=np.uint64))) & 0xF).astype(np.int64)
    nib = np.where(nib >= 8, nib - 16, nib)
    return nib.reshape(p.shape[0], K)


def test_pack_roundtrip_random():
    rng = np.random.default_rng(12)
    q = rng.integers(-8, 8, (9, 64)).astype(np.int8)
    p = oracle.pack_int4(q)
    assert np.array_equal(_unpack_np(p, 64), q)
    assert np.array_equal(oracle.unpack_int4(p, 64), q)


@pytest.mark.parametrize("G", [8, 64, 128])
def test_hadamard_quant_int4_matches_library_composition(G):
    X, _, _ = synthetic.mixed_inputs(5, 256, 1, seed=13, n_dims=3, magnitude=("abs_normal", 50.0))
    H = scipy.linalg.hadamard(G).astype(np.float64)
    xr = ((X.astype(np.float64).reshape(5, -1, G) @ H) * (1.0 / math.sqrt(G))).astype(np.float32)
    for per_group in (False, True):
        packed, s = oracle.hadamard_quant_int4(X, G, per_group=per_group)
        a = np.abs(xr).max(axis=2) if per_group else np.abs(xr).reshape(5, -1).max(axis=1, keepdims=True)
        s_ref = np.where(a == 0, np.float32(1), a / np.float32(7)).astype(np.float32)
        assert np.array_equal(s, s_ref)
        sb = s_ref[:, :, None] if per_group else s_ref[:, :, None]
        q_ref = np.clip(np.rint(xr / sb), -7, 7).reshape(5, 256)
        assert np.array_equal(_unpack_np(packed, 256), q_ref)


@settings(max_examples=15, deadline=None)
@given(M=st.integers(1, 12), N=st.integers(1, 20), groups=st.integers(1, 4), G=st.sampled_from([8, 64, 128]),
       seed=st.integers(0, 2 ** 31))
def test_w4a4_group_acc_bruteforce(M, N, groups, G, seed):
    K = G * groups
    rng = np.random.default_rng(seed)
    Xp = rng.integers(0, 2 ** 32, (M, K // 8), dtype=np.uint64).astype(np.uint32)
    Wp = rng.integers(0, 2 ** 32, (N, K // 8), dtype=np.uint64).astype(np.uint32)
    acc = oracle.w4a4_group_acc(Xp, Wp, K, G)
    x = _unpack_np(Xp, K).reshape(M, groups, G)
    w = _unpack_np(Wp, K).reshape(N, groups, G)
    assert np.array_equal(acc, np.einsum("mgk,ngk->mng", x, w))


def test_w4a4_output_matches_dequant_matmul_and_error_bound():
    M, K, N, G = 12, 512, 20, 128
    X, W, _ = synthetic.w4a4_inputs(M, K, N, seed=14)
    Wp, s_w = oracle.hadamard_quant_int4(W, G, per_group=True)
    out = oracle.qlinear_w4a4(X, Wp, s_w, G)
    Xp, s_x = oracle.hadamard_quant_int4(X, G, per_group=False)
    xd = _unpack_np(Xp, K) * s_x.astype(np.float64)
    wd = _unpack_np(Wp, K) * np.repeat(s_w.astype(np.float64), G, axis=1)
    mag = np.abs(xd) @ np.abs(wd).T
    assert np.all(np.abs(out - xd @ wd.T) <= 1e-12 * mag)
    # error bound against the unquantized product (rotation is orthogonal)
    H = scipy.linalg.hadamard(G).astype(np.float64) / math.sqrt(G)
    xr = (X.astype(np.float64).reshape(M, -1, G) @ H).reshape(M, K)
    wr = (W.astype(np.float64).reshape(N, -1, G) @ H).reshape(N, K)
    sx = np.abs(xr.astype(np.float32)).max(axis=1).astype(np.float64) / 7 * (1 + 1e-6)
    sw = np.repeat(np.abs(wr.astype(np.float32)).reshape(N, -1, G).max(axis=2) / 7, G, axis=1) * (1 + 1e-6)
    B = 0.5 * sx[:, None] * ((np.abs(wr) + 0.5 * sw).sum(axis=1))[None, :] + 0.5 * np.abs(xr) @ sw.T
    exact = X.astype(np.float64) @ W.astype(np.float64).T
    slack = 2.0 ** -20 * (np.abs(xr) @ np.abs(wr).T)
    assert np.all(np.abs(out - exact) <= B + slack)
    # a mis-grouped weight scale breaks the dequantize-then-matmul identity
    out_bad = oracle.qlinear_w4a4(X, Wp, s_w[:, ::-1].copy(), G)
    assert not np.all(np.abs(out_bad - xd @ wd.T) <= 1e-6 * mag)


def test_rotation_lowers_w4a4_error():
    # qualitative claim of the group-rotation page (§二): rotating before int4
    # quantization lowers the error; compared with the identity rotation and
    # the same 128-wide weight groups.
    M, K, N = 16, 512, 24
    X, W, _ = synthetic.w4a4_inputs(M, K, N, seed=15)
    exact = X.astype(np.float64) @ W.astype(np.float64).T
    Wp, s_w = oracle.hadamard_quant_int4(W, 128, per_group=True)
    err_rot = np.abs(oracle.qlinear_w4a4(X, Wp, s_w, 128) - exact).mean()
    qx, sx = oracle.quant_rows(X, qmin=-7, qmax=7)
    qw, sw = oracle.quant_rows(W, gsize=128, qmin=-7, qmax=7)
    plain = (qx * sx.astype(np.float64)) @ (qw * np.repeat(sw.astype(np.float64), 128, axis=1)).T
    assert err_rot < np.abs(plain - exact).mean() / 2


# ------------------------------------------------------------------ W4A8
@pytest.mark.parametrize("G", [64, 256])
def test_hadamard_quant_int8_unit_vectors(G):
    # x = v e_i in one block: the rotated block is v/sqrt(G) times row i of H_G
    # (exact for G = 64, 256), every other block is 0, so the codes are
    # +-127 in H_G's sign pattern and s = fl32(|v|/sqrt(G) / 127)
    K = 2 * G
    for i, v, b in [(0, 8.0, 0), (5, -24.0, 1), (G - 1, 0.5, 0), (G // 2 + 3, 1000.0, 1)]:
        x = np.zeros(K, np.float16)
        x[b * G + i] = v
        q, s = oracle.hadamard_quant_int8(x, G)
        a = np.float32(abs(v) / math.sqrt(G))
        assert s[0] == a / np.float32(127)
        H = scipy.linalg.hadamard(G)
        want = np.zeros(K, np.int64)
        want[b * G:(b + 1) * G] = 127 * np.sign(v) * H[i]
        assert np.array_equal(q[0], want)


@pytest.mark.parametrize("G", [8, 64, 128])
def test_hadamard_quant_int8_matches_library_composition(G):
    X, _, _ = synthetic.mixed_inputs(5, 256, 1, seed=16, n_dims=3, magnitude=("abs_normal", 50.0))
    X[2] = 0
    H = scipy.linalg.hadamard(G).astype(np.float64)
    xr = ((X.astype(np.float64).reshape(5, -1, G) @ H) * (1.0 / math.sqrt(G))).astype(np.float32).reshape(5, 256)
    q, s = oracle.hadamard_quant_int8(X, G)
    a = np.abs(xr).max(axis=1)
    s_ref = np.where(a == 0, np.float32(1), a / np.float32(127)).astype(np.float32)
    assert np.array_equal(s, s_ref) and s[2] == 1.0
    assert np.array_equal(q, np.clip(np.rint(xr / s_ref[:, None]), -127, 127))
    # rounding to nearest: each code is within half a step of the rotated value
    err = np.abs(q * s.astype(np.float64)[:, None] - xr.astype(np.float64))
    assert np.all(err <= 0.5 * s.astype(np.float64)[:, None] * (1 + 1e-6))
    assert np.all(np.abs(q[[0, 1, 3, 4]]).max(axis=1) == 127)


@settings(max_examples=15, deadline=None)
@given(M=st.integers(1, 12), N=st.integers(1, 20), groups=st.integers(1, 4), G=st.sampled_from([8, 64, 256]),
       seed=st.integers(0, 2 ** 31))
def test_w4a8_group_acc_bruteforce(M, N, groups, G, seed):
    K = G * groups
    rng = np.random.default_rng(seed)
    Xq = rng.integers(-128, 128, (M, K)).astype(np.int8)
    Wp = rng.integers(0, 2 ** 32, (N, K // 8), dtype=np.uint64).astype(np.uint32)
    acc = oracle.w4a8_group_acc(Xq, Wp, G)
    w = _unpack_np(Wp, K).reshape(N, groups, G)
    assert np.array_equal(acc, np.einsum("mgk,ngk->mng", Xq.astype(np.int64).reshape(M, groups, G), w))
    rows = np.array([M - 1, 0])
    assert np.array_equal(oracle.w4a8_group_acc(Xq, Wp, G, rows=rows), acc[rows])


def test_w4a8_output_matches_dequant_matmul_and_error_bound():
    M, K, N, G = 12, 512, 20, 128
    X, W, _ = synthetic.w4a4_inputs(M, K, N, seed=17)
    Wp, s_w = oracle.hadamard_quant_int4(W, G, per_group=True)
    out = oracle.qlinear_w4a8(X, Wp, s_w, G)
    q, s_x = oracle.hadamard_quant_int8(X, G)
    xd = q * s_x.astype(np.float64)[:, None]
    wd = _unpack_np(Wp, K) * np.repeat(s_w.astype(np.float64), G, axis=1)
    mag = np.abs(xd) @ np.abs(wd).T
    assert np.all(np.abs(out - xd @ wd.T) <= 1e-12 * mag)
    # error bound against the unquantized product (rotation is orthogonal)
    H = scipy.linalg.hadamard(G).astype(np.float64) / math.sqrt(G)
    xr = (X.astype(np.float64).reshape(M, -1, G) @ H).reshape(M, K)
    wr = (W.astype(np.float64).reshape(N, -1, G) @ H).reshape(N, K)
    sx = np.abs(xr.astype(np.float32)).max(axis=1).astype(np.float64) / 127 * (1 + 1e-6)
    sw = np.repeat(np.abs(wr.astype(np.float32)).reshape(N, -1, G).max(axis=2) / 7, G, axis=1) * (1 + 1e-6)
    B = 0.5 * sx[:, None] * ((np.abs(wr) + 0.5 * sw).sum(axis=1))[None, :] + 0.5 * np.abs(xr) @ sw.T
    exact = X.astype(np.float64) @ W.astype(np.float64).T
    slack = 2.0 ** -20 * (np.abs(xr) @ np.abs(wr).T)
    assert np.all(np.abs(out - exact) <= B + slack)
    rows = np.array([11, 0, 5])
    assert np.array_equal(oracle.qlinear_w4a8(X, Wp, s_w, G, rows=rows), out[rows])


def test_w4a8_error_below_w4a4():
    # the point of 8-bit activations: with the same rotated int4 weight, the
    # output error falls to the weight-only level (rotated activations kept
    # unquantized), clearly below W4A4's
    M, K, N, G = 16, 1024, 24, 128
    X, W, _ = synthetic.w4a4_inputs(M, K, N, seed=18)
    exact = X.astype(np.float64) @ W.astype(np.float64).T
    Wp, s_w = oracle.hadamard_quant_int4(W, G, per_group=True)
    e8 = np.abs(oracle.qlinear_w4a8(X, Wp, s_w, G) - exact).mean()
    e4 = np.abs(oracle.qlinear_w4a4(X, Wp, s_w, G) - exact).mean()
    H = scipy.linalg.hadamard(G).astype(np.float64) / math.sqrt(G)
    xr = (X.astype(np.float64).reshape(M, -1, G) @ H).reshape(M, K)
    wd = _unpack_np(Wp, K) * np.repeat(s_w.astype(np.float64), G, axis=1)
    e_w = np.abs(xr @ wd.T - exact).mean()
    assert e8 < 0.75 * e4
    assert abs(e8 - e_w) < 0.05 * e_w


# ------------------------------------------------------------------ W4A4, zero-point activations
def test_w4a4_asym_worked_examples():
    # G = 1 leaves the row unrotated.  Inference Quantization §6: data in [0, 6]
    # on int4 spreads over all 16 levels with 0 at the bottom: s = 6/15, z = 0;
    # 2.5, 7.5 and 12.5 round half to even
    x = np.array([[0, 1, 2, 3, 4, 5, 6, 0]], np.float16)
    p, s, z = oracle.hadamard_quant_int4_asym(x, 1)
    assert s[0] == np.float32(6.0) / np.float32(15.0) and z[0] == 0
    assert np.array_equal(oracle.unpack_int4(p, 8)[0] + 8, [0, 2, 5, 8, 10, 12, 15, 0])
    assert np.array_equal(_unpack_np(p, 8)[0], [-8, -6, -3, 0, 2, 4, 7, -8])       # stored as q - 8
    # §6.2: the range [-0.2, 1.7] puts real 0 exactly on the code z = 2
    x = np.array([[-0.2, 1.7, 0.0, 0.0, 1.0, -0.1, 0.5, 0.0]], np.float16)
    p, s, z = oracle.hadamard_quant_int4_asym(x, 1)
    q = oracle.unpack_int4(p, 8)[0] + 8
    assert z[0] == 2 and q[2] == 2 and q[0] == 0 and q[1] == 15
    # a constant row: hi = lo after including 0 only when the row is all zero
    p, s, z = oracle.hadamard_quant_int4_asym(np.zeros((1, 16), np.float16), 8)
    assert s[0] == 1.0 and z[0] == 0 and not (oracle.unpack_int4(p, 16) + 8).any()


@pytest.mark.parametrize("G", [8, 64, 128])
def test_w4a4_asym_codes_reconstruct_the_rotated_row(G):
    X, _, _ = synthetic.mixed_inputs(6, 512, 1, seed=31, n_dims=3, magnitude=("abs_normal", 30.0))
    X[1] = np.abs(X[1])                                     # one-sided row
    p, s, z = oracle.hadamard_quant_int4_asym(X, G)
    H = scipy.linalg.hadamard(G).astype(np.float64)
    xr = ((X.astype(np.float64).reshape(6, -1, G) @ H) * (1.0 / math.sqrt(G))).astype(np.float32).reshape(6, 512)
    q = oracle.unpack_int4(p, 512).astype(np.int64) + 8
    assert q.min() >= 0 and q.max() <= 15 and np.all((z >= 0) & (z <= 15))
    lo = np.minimum(xr.min(axis=1), 0).astype(np.float64)
    hi = np.maximum(xr.max(axis=1), 0).astype(np.float64)
    # every value of [lo, hi] is representable: within half a step of s (q - z)
    sd = s.astype(np.float64)[:, None]
    assert np.all(np.abs(sd * (q - z[:, None]) - xr) <= 0.5 * sd * (1 + 1e-5))
    assert np.all(np.abs(s - (hi - lo) / 15) <= 1e-6 * (hi - lo) / 15)
    # real 0 sits within half a step of the grid point z
    assert np.all(np.abs(np.rint(-lo / s.astype(np.float64)) - z) <= 0.5 + 1e-9)


def test_w4a4_asym_linear_is_the_dequantized_product_and_bounded():
    M, K, N, G = 10, 512, 18, 128
    X, W, _ = synthetic.w4a4_inputs(M, K, N, seed=32)
    X = np.abs(X)                                           # one-sided activations
    Wp, s_w = oracle.hadamard_quant_int4(W, G, per_group=True)
    out = oracle.qlinear_w4a4_asym(X, Wp, s_w, G)
    p, s_x, z_x = oracle.hadamard_quant_int4_asym(X, G)
    xd = (oracle.unpack_int4(p, K).astype(np.float64) + 8 - z_x[:, None]) * s_x.astype(np.float64)[:, None]
    wd = _unpack_np(Wp, K) * np.repeat(s_w.astype(np.float64), G, axis=1)
    mag = np.abs(xd) @ np.abs(wd).T
    assert np.all(np.abs(out - xd @ wd.T) <= 1e-12 * mag)
    H = scipy.linalg.hadamard(G).astype(np.float64) / math.sqrt(G)
    xr = (X.astype(np.float64).reshape(M, -1, G) @ H).reshape(M, K)
    wr = (W.astype(np.float64).reshape(N, -1, G) @ H).reshape(N, K)
    sx = s_x.astype(np.float64) * (1 + 1e-6)
    sw = np.repeat(np.abs(wr.astype(np.float32)).reshape(N, -1, G).max(axis=2) / 7, G, axis=1) * (1 + 1e-6)
    B = 0.5 * sx[:, None] * ((np.abs(wr) + 0.5 * sw).sum(axis=1))[None, :] + 0.5 * np.abs(xr) @ sw.T
    exact = X.astype(np.float64) @ W.astype(np.float64).T
    assert np.all(np.abs(out - exact) <= B + 2.0 ** -20 * (np.abs(xr) @ np.abs(wr).T))
    rows = np.array([9, 2])
    assert np.array_equal(oracle.qlinear_w4a4_asym(X, Wp, s_w, G, rows=rows), out[rows])


def test_w4_column_terms_hand_example_and_closed_forms():
    # one column, K = 16, G = 8: nibbles 1..8 (8 reads as -8) in group 0, all -1 in group 1
    q = np.array([[1, 2, 3, 4, 5, 6, 7, -8, -1, -1, -1, -1, -1, -1, -1, -1]], np.int8)
    Wp = oracle.pack_int4(q)
    c = oracle.w4_column_terms(Wp, np.array([[0.5, 0.25]], np.float32), 16, 8)
    assert c[0] == np.float32(0.5 * 20 + 0.25 * -8)              # 8.0
    # one group: a single product, rounded once
    rng = np.random.default_rng(36)
    q = rng.integers(-8, 8, (5, 64)).astype(np.int8)
    s = rng.uniform(0.001, 0.1, (5, 1)).astype(np.float32)
    c = oracle.w4_column_terms(oracle.pack_int4(q), s, 64, 64)
    assert np.array_equal(c, (s[:, 0].astype(np.float64) * q.astype(np.int64).sum(axis=1)).astype(np.float32))
    # an all-zero weight
    assert not oracle.w4_column_terms(oracle.pack_int4(np.zeros((3, 32), np.int8)),
                                      np.ones((3, 4), np.float32), 32, 8).any()


def test_w4_column_terms_split_the_zero_point_linear():
    # the zero-point linear (pinned above to the dequantized product) is the
    # symmetric group products of the stored codes q - 8 minus (z - 8) times
    # the column term; only c's rounding to fp32 separates the two
    M, K, N, G = 6, 512, 14, 128
    X, W, _ = synthetic.w4a4_inputs(M, K, N, seed=35)
    X = np.abs(X)
    Wp, s_w = oracle.hadamard_quant_int4(W, G, per_group=True)
    c = oracle.w4_column_terms(Wp, s_w, K, G).astype(np.float64)
    p, s_x, z_x = oracle.hadamard_quant_int4_asym(X, G)
    acc = oracle.w4a4_group_acc(p, Wp, K, G).astype(np.float64)      # sum_{k in g} (q - 8) qw
    sym = (acc * s_w.astype(np.float64)[None, :, :]).sum(axis=2)
    sx = s_x.astype(np.float64)[:, None]
    zm = (z_x.astype(np.float64) - 8)[:, None]
    split = sx * (sym - zm * c[None, :])
    out = oracle.qlinear_w4a4_asym(X, Wp, s_w, G)
    mag = sx * ((np.abs(acc) * s_w.astype(np.float64)[None, :, :]).sum(axis=2) + np.abs(zm * c[None, :]))
    assert np.all(np.abs(out - split) <= sx * np.abs(zm) * np.abs(c)[None, :] * 2.0 ** -23 + 1e-12 * mag)
    assert np.any(zm != 0)


@pytest.mark.parametrize("seed", [33, 34])
def test_w4a4_asym_lowers_the_error_of_one_sided_activations(seed):
    # the point of the zero-point: one-sided rows (after the rotation their
    # range is still lopsided) get a finer grid, (hi - lo)/15 against the
    # symmetric absmax/7, so both the activation codes and the output are closer
    M, K, N, G = 16, 1024, 24, 128
    X, W, _ = synthetic.w4a4_inputs(M, K, N, seed=seed)
    X = np.abs(X)
    H = scipy.linalg.hadamard(G).astype(np.float64) / math.sqrt(G)
    xr = (X.astype(np.float64).reshape(M, -1, G) @ H).reshape(M, K)
    pa, sa, za = oracle.hadamard_quant_int4_asym(X, G)
    ps, ss = oracle.hadamard_quant_int4(X, G, per_group=False)
    ea = np.abs((oracle.unpack_int4(pa, K) + 8 - za[:, None]) * sa.astype(np.float64)[:, None] - xr).mean()
    es = np.abs(oracle.unpack_int4(ps, K) * ss.astype(np.float64) - xr).mean()
    assert ea < 0.9 * es
    exact = X.astype(np.float64) @ W.astype(np.float64).T
    Wp, s_w = oracle.hadamard_quant_int4(W, G, per_group=True)
    e_asym = np.abs(oracle.qlinear_w4a4_asym(X, Wp, s_w, G) - exact).mean()
    e_sym = np.abs(oracle.qlinear_w4a4(X, Wp, s_w, G) - exact).mean()
    assert e_asym < e_sym


# ------------------------------------------------------------------ SmoothQuant
def _f32_ulp(x):
    x = np.abs(np.asarray(x, np.float32))
    return np.spacing(x).astype(np.float64)


def test_smoothquant_page_example():
    """The printed demonstration of "Quantization explained, part 2" §4.5:
    per-tensor W8A8 error 0.108 without and 0.054 with alpha = 0.5 smoothing,
    and an equivalence error of order 1e-6."""
    g = golden("smoothquant_toy.json")
    X = np.array([[int(v, 16) for v in row] for row in g["X_f32_bits"]], np.uint32).view(np.float32)
    W = np.array([[int(v, 16) for v in row] for row in g["W_f32_bits"]], np.uint32).view(np.float32)
    assert X.shape == (g["T"], g["C_in"]) and W.shape == (g["C_in"], g["C_out"])
    Wt = np.ascontiguousarray(W.T)                     # our layout: [out x in]
    Y = X.astype(np.float64) @ W.astype(np.float64)
    s = oracle.smooth_factors(oracle.col_absmax(X), oracle.col_absmax(Wt), g["alpha"])
    Xh = oracle.smooth_apply(X, s, oracle.SMOOTH_DIVIDE)
    Wh = oracle.smooth_apply(Wt, s, oracle.SMOOTH_MULTIPLY)
    eq = np.abs(Xh.astype(np.float64) @ Wh.astype(np.float64).T - Y).max()
    assert eq < 10 * g["equivalence_printed_order"]

    def w8a8_err(sv):
        qx, sx = oracle.smooth_quantize(X, sv, oracle.SMOOTH_DIVIDE, per_tensor=True)
        qw, sw = oracle.smooth_quantize(Wt, sv, oracle.SMOOTH_MULTIPLY, per_tensor=True)
        deq_x = qx.astype(np.float64) * sx.astype(np.float64)[:, None]
        deq_w = qw.astype(np.float64) * sw.astype(np.float64)[:, None]
        return np.abs(Y - deq_x @ deq_w.T).mean()

    d = g["printed_digits"]
    assert round(w8a8_err(np.ones(g["C_in"], np.float32)), d) == g["err_raw_printed"]
    assert round(w8a8_err(s), d) == g["err_smooth_printed"]


@pytest.mark.parametrize("alpha", [0.25, 0.5, 0.75])
def test_smooth_column_maxima_closed_form(alpha):
    """After migration the column maxima are cx^(1-a) cw^(1-a) (activations)
    and cx^a cw^a (weights); at a = 0.5 both equal sqrt(cx cw)."""
    X, W, _ = synthetic.mixed_inputs(64, 256, 48, seed=21, n_dims=4)
    cx = np.abs(X.astype(np.float64)).max(axis=0)
    cw = np.abs(W.astype(np.float64)).max(axis=0)
    s = oracle.smooth_factors(oracle.col_absmax(X), oracle.col_absmax(W), alpha)
    mx = np.abs(oracle.smooth_apply(X, s, oracle.SMOOTH_DIVIDE)).max(axis=0)
    mw = np.abs(oracle.smooth_apply(W, s, oracle.SMOOTH_MULTIPLY)).max(axis=0)
    ex = cx ** (1 - alpha) * cw ** (1 - alpha)
    ew = cx ** alpha * cw ** alpha
    # s carries one fp32 rounding, the applied value another
    assert np.all(np.abs(mx - ex) <= 2.5 * 2.0 ** -24 * ex)
    assert np.all(np.abs(mw - ew) <= 2.5 * 2.0 ** -24 * ew)
    if alpha == 0.5:
        assert np.all(np.abs(mx - mw) <= 5 * 2.0 ** -24 * ex)


def test_smooth_alpha_extremes():
    """alpha = 1 moves all of the range into the weight (activation column
    maxima become exactly 1); alpha = 0 gives s = 1/max|W_j| (weight column
    maxima 1 up to one rounding), as the formula reads."""
    X, W, _ = synthetic.mixed_inputs(32, 128, 40, seed=22, n_dims=3)
    cx, cw = oracle.col_absmax(X), oracle.col_absmax(W)
    s1 = oracle.smooth_factors(cx, cw, 1.0)
    assert np.array_equal(s1, cx)
    assert np.array_equal(np.abs(oracle.smooth_apply(X, s1, oracle.SMOOTH_DIVIDE)).max(axis=0), np.ones(128, np.float32))
    s0 = oracle.smooth_factors(cx, cw, 0.0)
    assert np.array_equal(s0, (np.float32(1) / cw).astype(np.float32))
    mw = np.abs(oracle.smooth_apply(W, s0, oracle.SMOOTH_MULTIPLY)).max(axis=0).astype(np.float64)
    assert np.all(np.abs(mw - 1.0) <= 2.0 ** -23)


def test_col_absmax_matches_numpy():
    X, W, _ = synthetic.mixed_inputs(37, 200, 11, seed=23, n_dims=2)
    assert np.array_equal(oracle.col_absmax(X), np.abs(X.astype(np.float32)).max(axis=0))
    assert np.array_equal(oracle.col_absmax(W), np.abs(W.astype(np.float32)).max(axis=0))


def test_smooth_zero_columns_keep_factor_one():
    cx = np.array([0.0, 3.0, 0.0, 2.0], np.float32)
    cw = np.array([1.0, 0.0, 0.0, 0.5], np.float32)
    s = oracle.smooth_factors(cx, cw, 0.5)
    assert np.array_equal(s[:3], np.ones(3, np.float32))
    assert s[3] == np.float32(2.0)                                        # sqrt(2 / 0.5)


def test_smoothing_is_an_equivalence_within_rounding():
    """X^ W^T = X W^T up to the two fp32 roundings of each smoothed operand:
    x/s (1 + d1) * w s (1 + d2), |d1|, |d2| <= 2^-24."""
    X, W, _ = synthetic.mixed_inputs(48, 512, 64, seed=24, n_dims=5)
    s = oracle.smooth_factors(oracle.col_absmax(X), oracle.col_absmax(W), 0.5)
    Xh = oracle.smooth_apply(X, s, oracle.SMOOTH_DIVIDE).astype(np.float64)
    Wh = oracle.smooth_apply(W, s, oracle.SMOOTH_MULTIPLY).astype(np.float64)
    X64, W64 = X.astype(np.float64), W.astype(np.float64)
    bound = (2 * 2.0 ** -24 + 2.0 ** -47) * (np.abs(X64) @ np.abs(W64).T) * (1 + 1e-12)
    assert np.all(np.abs(Xh @ Wh.T - X64 @ W64.T) <= bound)
    # a dropped factor on one side breaks it
    assert not np.all(np.abs(X64 @ Wh.T - X64 @ W64.T) <= bound)


def test_smooth_quantize_scales():
    """Per-row scales are the absmax quantizer of the smoothed rows; the
    per-tensor scale is the largest per-row scale (fl32(a/127) is monotone),
    broadcast to every row."""
    X, W, _ = synthetic.mixed_inputs(30, 256, 8, seed=25, n_dims=3)
    s = oracle.smooth_factors(oracle.col_absmax(X), oracle.col_absmax(W), 0.5)
    Xh = oracle.smooth_apply(X, s, oracle.SMOOTH_DIVIDE)
    a = np.abs(Xh).max(axis=1)
    q, sr = oracle.smooth_quantize(X, s, oracle.SMOOTH_DIVIDE)
    assert np.array_equal(sr, (a / np.float32(127)).astype(np.float32))
    assert np.array_equal(q, np.clip(np.rint(Xh / sr[:, None]), -127, 127).astype(np.int8))
    qt, st_ = oracle.smooth_quantize(X, s, oracle.SMOOTH_DIVIDE, per_tensor=True)
    assert np.all(st_ == sr.max())
    assert np.array_equal(qt, np.clip(np.rint(Xh / st_[0]), -127, 127).astype(np.int8))


def test_smooth_linear_with_unit_factors_is_vectorwise_w8a8():
    X, W, _ = synthetic.mixed_inputs(24, 512, 40, seed=26, n_dims=3)
    one = np.ones(512, np.float32)
    Wq, s_w = oracle.smooth_quantize(W, one, oracle.SMOOTH_MULTIPLY)
    Wq_ref, s_w_ref = _w8(W)
    assert np.array_equal(Wq, Wq_ref) and np.array_equal(s_w, s_w_ref)
    out = oracle.qlinear_int8_smooth(X, one, Wq, s_w)
    assert np.array_equal(out, oracle.qlinear_int8_mixed(X, Wq, s_w, tau=float("inf")))


@pytest.mark.parametrize("e", [-3, 5])
def test_smooth_linear_power_of_two_factor_changes_nothing(e):
    """A uniform factor 2^e scales X^ and W^ exactly, so codes are unchanged and
    s_x s_w is the same product: the output is identical."""
    X, W, _ = synthetic.mixed_inputs(20, 256, 30, seed=27, n_dims=2)
    one = np.ones(256, np.float32)
    p2 = np.full(256, 2.0 ** e, np.float32)
    for per_tensor in (False, True):
        Wq1, sw1 = oracle.smooth_quantize(W, one, oracle.SMOOTH_MULTIPLY)
        Wq2, sw2 = oracle.smooth_quantize(W, p2, oracle.SMOOTH_MULTIPLY)
        assert np.array_equal(Wq1, Wq2)
        a = oracle.qlinear_int8_smooth(X, one, Wq1, sw1, per_tensor=per_tensor)
        b = oracle.qlinear_int8_smooth(X, p2, Wq2, sw2, per_tensor=per_tensor)
        assert np.array_equal(a, b)


def test_smooth_linear_matches_integer_matmul_composition():
    X, W, _ = synthetic.mixed_inputs(9, 128, 13, seed=28, n_dims=2)
    s = oracle.smooth_factors(oracle.col_absmax(X), oracle.col_absmax(W), 0.5)
    Wq, s_w = oracle.smooth_quantize(W, s, oracle.SMOOTH_MULTIPLY)
    for per_tensor in (False, True):
        qx, sx = oracle.smooth_quantize(X, s, oracle.SMOOTH_DIVIDE, per_tensor=per_tensor)
        C = qx.astype(np.int64) @ Wq.astype(np.int64).T
        ref = C.astype(np.float64) * sx.astype(np.float64)[:, None] * s_w.astype(np.float64)[None, :]
        out = oracle.qlinear_int8_smooth(X, s, Wq, s_w, per_tensor=per_tensor)
        assert np.array_equal(out, ref)
        rows = np.array([8, 0, 3])
        assert np.array_equal(oracle.qlinear_int8_smooth(X, s, Wq, s_w, per_tensor, rows=rows), out[rows])


@pytest.mark.parametrize("per_tensor", [False, True])
def test_smoothing_lowers_w8a8_error_on_outlier_activations(per_tensor):
    X, W, _ = synthetic.mixed_inputs(64, 1024, 96, seed=29, n_dims=6, magnitude=("uniform", 20.0, 100.0))
    exact = X.astype(np.float64) @ W.astype(np.float64).T
    one = np.ones(1024, np.float32)
    s = oracle.smooth_factors(oracle.col_absmax(X), oracle.col_absmax(W), 0.5)
    errs = []
    for sv in (one, s):
        Wq, s_w = oracle.smooth_quantize(W, sv, oracle.SMOOTH_MULTIPLY)
        errs.append(np.abs(oracle.qlinear_int8_smooth(X, sv, Wq, s_w, per_tensor=per_tensor) - exact).mean())
    assert errs[1] < errs[0] / 2


# ------------------------------------------------------------------ top-k decomposition
def _topk_ref(X, k):
    """The k largest column maxima, ties to the lower column, via a stable sort."""
    cm = np.abs(X.astype(np.float32)).max(axis=0)
    order = np.argsort(-cm.astype(np.float64), kind="stable")
    return np.sort(order[: max(0, min(k, X.shape[1]))]).astype(np.int32)


@pytest.mark.parametrize("k", [0, 1, 3, 17, 64, 200, 256, 300])
def test_topk_set_matches_stable_sort_with_ties(k):
    rng = np.random.default_rng(41)
    # small integers: many equal column maxima
    X = rng.integers(-6, 7, size=(9, 256)).astype(np.float16)
    mask, idx, cm = oracle.outlier_topk(X, k)
    ref = _topk_ref(X, k)
    assert np.array_equal(idx, ref)
    assert mask.sum() == len(ref) and np.all(mask[ref] == 1)
    assert np.array_equal(cm, np.abs(X.astype(np.float32)).max(axis=0))


def test_topk_equals_threshold_set_without_boundary_ties():
    X, _, dims = synthetic.mixed_inputs(64, 1024, 1, seed=42, n_dims=9, magnitude=("uniform", 8.0, 60.0))
    _, idx_t, cm = oracle.outlier_cols(X, 6.0)
    assert len(np.unique(cm[cm > 6.0])) == len(idx_t)            # no ties among the outliers
    _, idx_k, _ = oracle.outlier_topk(X, len(idx_t))
    assert np.array_equal(idx_k, idx_t)
    Wq, s_w = oracle.quant_rows(synthetic.normal_f16(np.random.default_rng(1), (40, 1024), 0.02))
    a = oracle.qlinear_int8_topk(X, Wq, s_w[:, 0], k=len(idx_t))
    b = oracle.qlinear_int8_mixed(X, Wq, s_w[:, 0], tau=6.0)
    assert np.array_equal(a, b)


def test_topk_linear_extremes_reduce_to_pinned_cases():
    X, W, _ = synthetic.mixed_inputs(12, 256, 30, seed=43, n_dims=3)
    Wq, s_w = _w8(W)
    assert np.array_equal(oracle.qlinear_int8_topk(X, Wq, s_w, k=0),
                          oracle.qlinear_int8_mixed(X, Wq, s_w, tau=float("inf")))
    assert np.array_equal(oracle.qlinear_int8_topk(X, Wq, s_w, W16=W, k=256),
                          oracle.qlinear_int8_mixed(X, Wq, s_w, W16=W, tau=-1.0))


def test_raising_the_decomposed_share_lowers_error():
    """The pages advise decomposing the top 1-2% of dimensions rather than
    about 0.1%; on heavy-tailed activations the error drops."""
    X, W, _ = synthetic.mixed_inputs(128, 2048, 64, seed=44, n_dims=0, x_dist="t3")
    Wq, s_w = _w8(W)
    exact = X.astype(np.float64) @ W.astype(np.float64).T
    errs = [np.abs(oracle.qlinear_int8_topk(X, Wq, s_w, W16=W, k=k) - exact).mean() for k in (2, 21, 41)]
    assert errs[2] < errs[1] < errs[0]


# ------------------------------------------------------------------ asymmetric (zero-point)
def test_zero_point_grid_on_a_nonnegative_range():
    """Inference Quantization notes §6: data in [0, 6] wastes half of a signed
    int4 grid; shifted by z it uses all 16 levels, 0 -> q_min = z, 6 -> q_max."""
    x = np.linspace(0.0, 6.0, 61).astype(np.float32)
    s, z = oracle.minmax_params(x, -8, 7)
    assert s == np.float32(np.float32(6.0) / np.float32(15)) and z == -8
    q, sr, zr, _ = oracle.quant_rows_asym(x[None, :], -8, 7)
    assert q[0, 0] == -8 and q[0, -1] == 7
    assert set(q[0].tolist()) == set(range(-8, 8))
    assert sr[0] * (q[0, 0] - zr[0]) == 0.0                       # real 0 is exact


def test_zero_point_grid_on_a_shifted_range():
    """§6.2: a range such as [-0.2, 1.7] gets the whole grid; real 0 maps to z."""
    x = np.array([-0.2, 0.0, 0.35, 1.1, 1.7], np.float32)
    s, z = oracle.minmax_params(x, -128, 127)
    assert s == np.float32(np.float32(np.float32(1.7) - np.float32(-0.2)) / np.float32(255))
    assert z == -128 + int(np.rint(np.float32(0.2) / s))          # -101
    q, sr, zr, _ = oracle.quant_rows_asym(x[None, :])
    assert q[0, 0] == -128 and q[0, 1] == z and q[0, -1] == 127
    assert np.all(np.abs(sr[0] * (q[0].astype(np.float64) - zr[0]) - x) <= sr[0] / 2 * (1 + 1e-6))


def test_zero_point_symmetric_range_and_zero_row():
    a = np.float32(3.0)
    x = np.array([-a, -1.0, 0.5, a], np.float32)
    assert oracle.minmax_params(x, -128, 127)[1] == 0             # -128 - rint(-127.5) = 0 (ties to even)
    q, s, z, rs = oracle.quant_rows_asym(np.zeros((2, 16), np.float32))
    assert np.all(s == 1.0) and np.all(z == -128) and np.all(q == -128) and np.all(rs == -128 * 16)


def test_asymmetric_codes_within_half_a_step():
    X, _, _ = synthetic.mixed_inputs(40, 300, 1, seed=51, n_dims=3, magnitude=("uniform", 10.0, 60.0))
    X[:5] = np.abs(X[:5]) + np.float16(2.0)                     # rows away from 0 on one side
    X[5:10] = -np.abs(X[5:10]) - np.float16(1.0)
    Xf = X.astype(np.float32)
    q, s, z, rs = oracle.quant_rows_asym(X)
    deq = s[:, None].astype(np.float64) * (q.astype(np.float64) - z[:, None])
    assert np.all(np.abs(deq - Xf) <= s[:, None] / 2 * (1 + 1e-6) + 1e-30)
    assert np.array_equal(rs, q.astype(np.int64).sum(axis=1))
    assert np.array_equal(q, np.clip(np.rint(Xf / s[:, None]) + z[:, None], -128, 127).astype(np.int8))


def test_asymmetric_linear_is_the_dequantized_product():
    X, W, _ = synthetic.mixed_inputs(11, 160, 23, seed=52, n_dims=2)
    Wq, s_w = _w8(W)
    qw, sw2, zw, _ = oracle.quant_rows_asym(W)
    for wq, swv, zwv in ((Wq, s_w, None), (qw, sw2, zw)):
        q, s, z, _ = oracle.quant_rows_asym(X)
        dz = zwv if zwv is not None else np.zeros(len(swv), np.int32)
        acc = (q.astype(np.int64) - z[:, None]) @ (wq.astype(np.int64) - dz[:, None]).T
        ref = acc.astype(np.float64) * s.astype(np.float64)[:, None] * swv.astype(np.float64)[None, :]
        out = oracle.qlinear_int8_asym(X, wq, swv, z_w=zwv)
        assert np.array_equal(out, ref)
        rows = np.array([10, 0, 4])
        assert np.array_equal(oracle.qlinear_int8_asym(X, wq, swv, z_w=zwv, rows=rows), out[rows])


def test_zero_point_helps_one_sided_activations():
    """The pages attribute zero-point's edge over absmax to one-sided values:
    on non-negative activations the shifted grid has about half the step
    (max/255 against max/127), so the activation error halves and the W8A8
    output error drops."""
    rng = np.random.default_rng(53)
    X = np.maximum(rng.normal(0.5, 1.0, (64, 512)), 0).astype(np.float16)
    W = synthetic.normal_f16(rng, (48, 512), 0.02)
    X64 = X.astype(np.float64)
    q, s, z, _ = oracle.quant_rows_asym(X)
    qs, ss = oracle.quant_rows(X)
    e_act_asym = np.abs(s[:, None] * (q.astype(np.float64) - z[:, None]) - X64).mean()
    e_act_sym = np.abs(ss * qs.astype(np.float64) - X64).mean()
    assert e_act_asym < 0.6 * e_act_sym
    Wq, s_w = _w8(W)
    exact = X64 @ W.astype(np.float64).T
    e_asym = np.abs(oracle.qlinear_int8_asym(X, Wq, s_w) - exact).mean()
    e_sym = np.abs(oracle.qlinear_int8_mixed(X, Wq, s_w, tau=float("inf")) - exact).mean()
    assert e_asym < e_sym


# ------------------------------------------------------------------ Kronecker transform (FlatQuant)
def test_kron_sizes_page_examples():
    for c in golden("kron_sizes.json")["cases"]:
        assert oracle.kron_sizes(c["n"]) == (c["n1_printed"], c["n2_printed"])


def test_kron_sizes_bruteforce():
    for n in list(range(1, 600)) + [11008, 14336, 28672]:
        pairs = [(a, n // a) for a in range(1, n + 1) if n % a == 0 and a <= n // a]
        best = min(pairs, key=lambda p: p[0] + p[1])
        assert oracle.kron_sizes(n) == best


def _gamma(n):
    u = 2.0 ** -24
    return n * u / (1 - n * u)


@pytest.mark.parametrize("n1,n2", [(4, 8), (8, 8), (16, 32), (64, 64)])
def test_kron_transform_is_the_kronecker_product(n1, n2):
    """x (P1 (x) P2) within the error bound of two fp32 dot-product chains."""
    rng = np.random.default_rng(n1 * 100 + n2)
    X = rng.normal(0, 2.0, (7, n1 * n2)).astype(np.float16)
    P1, P2 = synthetic.kron_factors(n1, n2, seed=n2, kind="general")
    P1 = P1 + rng.normal(0, 0.2, P1.shape).astype(np.float32)   # clearly non-symmetric
    got = oracle.kron_transform(X, P1, P2).astype(np.float64)
    X64, A, B = X.astype(np.float64), P1.astype(np.float64), P2.astype(np.float64)
    ref = X64 @ np.kron(A, B)
    Xt = np.abs(X64).reshape(-1, n1, n2)
    e1 = _gamma(n1) * np.einsum("ia,rij->raj", np.abs(A), Xt)          # stage-1 error bound
    Y = np.abs(np.einsum("ia,rij->raj", A, X64.reshape(-1, n1, n2)))
    bound = (_gamma(n2) * np.einsum("raj,jb->rab", Y + e1, np.abs(B)) + np.einsum("raj,jb->rab", e1, np.abs(B)))
    assert np.all(np.abs(got - ref) <= bound.reshape(got.shape) * (1 + 1e-6) + 1e-30)
    # the other reading of the mode-2 product (P2 transposed) is a different map
    alt = X64 @ np.kron(A, B.T)
    assert np.abs(got - alt).max() > 1e3 * bound.max()


def test_kron_identity_and_permutations_are_exact():
    rng = np.random.default_rng(71)
    X = rng.normal(0, 3.0, (5, 96)).astype(np.float16)
    assert np.array_equal(oracle.kron_transform(X, np.eye(8, dtype=np.float32), np.eye(12, dtype=np.float32)),
                          X.astype(np.float32))
    p1, p2 = rng.permutation(8), rng.permutation(12)
    P1 = np.eye(8, dtype=np.float32)[p1]
    P2 = np.eye(12, dtype=np.float32)[p2]
    ref = (X.astype(np.float64) @ np.kron(P1.astype(np.float64), P2.astype(np.float64))).astype(np.float32)
    assert np.array_equal(oracle.kron_transform(X, P1, P2), ref)


@pytest.mark.parametrize("n1,n2", [(2, 4), (8, 8), (16, 32), (64, 64)])
def test_kron_of_hadamards_is_the_sylvester_hadamard(n1, n2):
    """H_n1 (x) H_n2 = H_n (Sylvester order): on small integers every partial
    sum is exact, so the transform equals the integer product."""
    rng = np.random.default_rng(n1 + n2)
    X = rng.integers(-8, 9, (6, n1 * n2))
    H1 = scipy.linalg.hadamard(n1).astype(np.float32)
    H2 = scipy.linalg.hadamard(n2).astype(np.float32)
    got = oracle.kron_transform(X.astype(np.float16), H1, H2)
    assert np.array_equal(got.astype(np.int64), X @ scipy.linalg.hadamard(n1 * n2))


def test_kron_weight_transform_cancels_in_the_product():
    """(X P)(P^-1 W^T) = X W^T: the weight rows take P1^-T, P2^-T."""
    X, W, _ = synthetic.mixed_inputs(16, 256, 24, seed=72, n_dims=3)
    P1, P2 = synthetic.kron_factors(16, 16, seed=73, kind="general")
    P1w = np.linalg.inv(P1.astype(np.float64)).T.astype(np.float32)
    P2w = np.linalg.inv(P2.astype(np.float64)).T.astype(np.float32)
    Xt = oracle.kron_transform(X, P1, P2).astype(np.float64)
    Wt = oracle.kron_transform(W, P1w, P2w).astype(np.float64)
    exact = X.astype(np.float64) @ W.astype(np.float64).T
    mag = np.abs(X.astype(np.float64)) @ np.abs(W.astype(np.float64)).T
    assert np.all(np.abs(Xt @ Wt.T - exact) <= 1e-5 * mag.max())


def test_kron_quant_int4_is_transform_then_codes():
    X, _, _ = synthetic.mixed_inputs(9, 512, 1, seed=74, n_dims=3)
    P1, P2 = synthetic.kron_factors(16, 32, seed=75)
    for G in (None, 128):
        packed, s = oracle.kron_quant_int4(X, P1, P2, per_group_G=G)
        q, s_ref = oracle.quant_rows(oracle.kron_transform(X, P1, P2), gsize=G, qmin=-7, qmax=7)
        assert np.array_equal(s, s_ref)
        assert np.array_equal(_unpack_np(packed, 512), q)


def test_kron_w4a4_linear_is_the_dequantized_product():
    X, W, _ = synthetic.mixed_inputs(6, 256, 20, seed=76, n_dims=2)
    P1, P2 = synthetic.kron_factors(16, 16, seed=77)
    Wp, s_w = oracle.kron_quant_int4(W, P1, P2, per_group_G=64)
    Xp, s_x = oracle.kron_quant_int4(X, P1, P2)
    qx, qw = _unpack_np(Xp, 256).astype(np.int64), _unpack_np(Wp, 256).astype(np.int64)
    ref = np.zeros((6, 20))
    for g in range(4):
        acc = qx[:, g * 64:(g + 1) * 64] @ qw[:, g * 64:(g + 1) * 64].T
        ref += acc.astype(np.float64) * s_w[:, g].astype(np.float64)[None, :]
    ref *= s_x[:, 0].astype(np.float64)[:, None]
    out = oracle.qlinear_kron_w4a4(X, P1, P2, Wp, s_w, G=64)
    assert np.allclose(out, ref, rtol=1e-12, atol=0)
    rows = np.array([5, 0, 2])
    assert np.array_equal(oracle.qlinear_kron_w4a4(X, P1, P2, Wp, s_w, G=64, rows=rows), out[rows])


def test_orthogonal_kron_transform_lowers_w4a4_error():
    """The flatness argument: an orthogonal transform spreads the outlier
    channels, so W4A4 on (X P, W P) is closer to X W^T than on (X, W)."""
    X, W, _ = synthetic.w4a4_inputs(64, 1024, 48, seed=78)
    exact = X.astype(np.float64) @ W.astype(np.float64).T
    errs = []
    for P1, P2 in ((np.eye(32, dtype=np.float32), np.eye(32, dtype=np.float32)), synthetic.kron_factors(32, 32, 79)):
        Wp, s_w = oracle.kron_quant_int4(W, P1, P2, per_group_G=128)
        errs.append(np.abs(oracle.qlinear_kron_w4a4(X, P1, P2, Wp, s_w, G=128) - exact).mean())
    assert errs[1] < 0.75 * errs[0]
