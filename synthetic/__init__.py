"""Seeded synthetic inputs for the quantized linear layer.

This module only draws numbers: it holds none of the method's arithmetic and
serves both the GPU library's tests / benchmark and the CPU oracle.  Values are
drawn in float64 with ``numpy.random.default_rng(seed)`` and rounded once to
fp16 (round to nearest even).

The shapes and statistics stand in for the pages' workloads (their models and
evaluation sets are not available): hidden sizes 4096 and 8192, 2048-token
sequences, 6-7 fixed outlier feature dimensions covering about 0.1% of values,
one-sided per dimension, at 20x or more the typical magnitude and up to 100x,
present in about 75% of the tokens (AIInfra 05Quantization01, LLM.int8()
analysis of emergent outlier features; FlatQuant blog §1).
"""
from __future__ import annotations

import numpy as np

F32, F16, BF16 = 0, 1, 2

CONFIG_NAMES = ("tiny_mixed", "decode_mixed", "prefill_mixed", "w8a8_ffn", "w4a4_hadamard")


def _f16(a: np.ndarray) -> np.ndarray:
    return np.asarray(a, dtype=np.float64).astype(np.float16)


def normal_f16(rng: np.random.Generator, shape, std: float, chunk_rows: int = 2048) -> np.ndarray:
    """N(0, std) rounded to fp16, drawn in row chunks to bound host memory."""
    rows, cols = shape
    out = np.empty((rows, cols), np.float16)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        out[r0:r1] = _f16(rng.normal(0.0, std, size=(r1 - r0, cols)))
    return out


def plant_outlier_dims(rng, X64: np.ndarray, n_dims: int, magnitude, p_token: float = 1.0):
    """Overwrite n_dims random feature columns of X64 (float64, in place).

    magnitude: ("abs_normal", scale) -> scale * |N(0,1)|, or ("uniform", lo, hi).
    Each dim has one sign for all its tokens (outliers are one-sided); each
    token carries the outlier with probability p_token, else keeps its value.
    Returns the sorted planted dims.
    """
    M, K = X64.shape
    dims = np.sort(rng.choice(K, size=n_dims, replace=False))
    signs = rng.choice(np.array([-1.0, 1.0]), size=n_dims)
    for d, sg in zip(dims, signs):
        if magnitude[0] == "abs_normal":
            mag = magnitude[1] * np.abs(rng.normal(0.0, 1.0, size=M))
        else:
            mag = rng.uniform(magnitude[1], magnitude[2], size=M)
        hit = rng.random(M) < p_token if p_token < 1.0 else np.ones(M, bool)
        X64[hit, d] = sg * mag[hit]
    return dims


def mixed_inputs(M, K, N, seed=0, n_dims=7, magnitude=("uniform", 6.0, 100.0), p_token=0.75,
                 w_std=0.02, x_dist="normal"):
    """Generic LLM.int8()-shaped inputs: X fp16 [M x K] with planted outlier
    dims, W fp16 [N x K] ~ N(0, w_std)."""
    rng = np.random.default_rng(seed)
    if x_dist == "normal":
        X64 = rng.normal(0.0, 1.0, size=(M, K))
    elif x_dist == "t3":
        X64 = np.clip(rng.standard_t(3, size=(M, K)), -30.0, 30.0)
    else:
        raise ValueError(x_dist)
    dims = plant_outlier_dims(rng, X64, n_dims, magnitude, p_token) if n_dims else np.zeros(0, np.int64)
    X = _f16(X64)
    W = normal_f16(rng, (N, K), w_std)
    return X, W, dims


def w4a4_inputs(M, K, N, seed=0, n_dims=6, x_mag=50.0, w_std=0.02, w_spike_p=0.01, w_spike=20.0):
    """W4A4 inputs: W ~ N(0, w_std) with a fraction w_spike_p of entries
    multiplied by w_spike; X ~ N(0,1) with n_dims one-sided dims of
    magnitude x_mag * |N(0,1)|."""
    rng = np.random.default_rng(seed)
    W64 = rng.normal(0.0, w_std, size=(N, K))
    spikes = rng.random((N, K)) < w_spike_p
    W64[spikes] *= w_spike
    W = _f16(W64)
    del W64, spikes
    X64 = rng.normal(0.0, 1.0, size=(M, K))
    dims = plant_outlier_dims(rng, X64, n_dims, ("abs_normal", x_mag)) if n_dims else np.zeros(0, np.int64)
    return _f16(X64), W, dims


def kron_factors(n1, n2, seed=0, kind="orthogonal"):
    """Stand-ins for FlatQuant's learned Kronecker factors (learning them needs
    calibration data): P1 [n1 x n1], P2 [n2 x n2] as float32.  kind:
    "orthogonal" -- Q of the QR factorization of a standard normal matrix;
    "general" -- identity plus N(0, 0.3 / sqrt(n)) noise (invertible, not
    orthogonal, not symmetric)."""
    rng = np.random.default_rng(seed)
    out = []
    for n in (n1, n2):
        if kind == "orthogonal":
            q, r = np.linalg.qr(rng.normal(0.0, 1.0, size=(n, n)))
            q = q * np.sign(np.diag(r))[None, :]
            out.append(q.astype(np.float32))
        else:
            out.append((np.eye(n) + rng.normal(0.0, 0.3 / np.sqrt(n), size=(n, n))).astype(np.float32))
    return out[0], out[1]


def config(name: str) -> dict:
    """The five workloads at full size.  Keys: X (fp16 [M x K]), W (fp16
    [N x K]), dims (planted outlier dims), tau, out_dtype, G, pass_w16, M, K, N."""
    if name == "tiny_mixed":
        rng = np.random.default_rng(0)
        X64 = rng.normal(0.0, 1.0, size=(16, 256))
        X64[:, 17] = rng.uniform(8.0, 70.0, size=16)
        X64[:, 200] = -rng.uniform(8.0, 70.0, size=16)
        W = normal_f16(rng, (256, 256), 0.02)
        return dict(name=name, X=_f16(X64), W=W, dims=np.array([17, 200]), tau=6.0, out_dtype=F32,
                    pass_w16=True, G=None, M=16, K=256, N=256)
    if name == "decode_mixed":
        X, W, dims = mixed_inputs(8, 4096, 4096, seed=0, n_dims=6, magnitude=("abs_normal", 20.0), p_token=1.0)
        return dict(name=name, X=X, W=W, dims=dims, tau=6.0, out_dtype=F16, pass_w16=False, G=None,
                    M=8, K=4096, N=4096)
    if name == "prefill_mixed":
        X, W, dims = mixed_inputs(2048, 4096, 11008, seed=0, n_dims=7, magnitude=("uniform", 6.0, 100.0),
                                  p_token=0.75)
        return dict(name=name, X=X, W=W, dims=dims, tau=6.0, out_dtype=F16, pass_w16=False, G=None,
                    M=2048, K=4096, N=11008)
    if name == "w8a8_ffn":
        X, W, dims = mixed_inputs(4096, 8192, 28672, seed=0, n_dims=0, x_dist="t3")
        return dict(name=name, X=X, W=W, dims=dims, tau=float("inf"), out_dtype=BF16, pass_w16=False,
                    G=None, M=4096, K=8192, N=28672)
    if name == "w4a4_hadamard":
        X, W, dims = w4a4_inputs(2048, 4096, 4096, seed=0)
        return dict(name=name, X=X, W=W, dims=dims, tau=None, out_dtype=F32, pass_w16=False, G=128,
                    M=2048, K=4096, N=4096)
    raise KeyError(name)
