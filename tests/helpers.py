"""Shared helpers of the GPU tests: upload inputs, run a path, compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np

import oracle
import tiled_dense_matrix_amd as tdm
from tiled_dense_matrix_amd import inputs

# Tolerances on the normalized error max|C - R| / (max|A| max|B| K).
TOL_F32 = 1e-5
TOL_BF16 = 4e-3
# Relative Frobenius error gate (also catches gross errors the normalized
# bar is too loose to see for bf16).
TOL_FRO = 1e-5


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(X: np.ndarray):
    import torch
    if X.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(X).view(np.int16)).cuda()
    return torch.from_numpy(np.ascontiguousarray(X)).cuda()


def run(kind: str, A_d, B_d, path=tdm.Path.AUTO, C_d=None, stream=None):
    if kind == "f32":
        return tdm.tdm_gemm_f32_path(A_d, B_d, C_d, path=path, stream=stream)
    return tdm.tdm_gemm_bf16_f32acc_path(A_d, B_d, C_d, path=path, stream=stream)


def max_abs(X: np.ndarray) -> float:
    return float(np.abs(oracle.widen(X)).max()) if X.size else 0.0


def check_full(kind: str, A: np.ndarray, B: np.ndarray, C: np.ndarray, what: str = ""):
    """Compare a full GPU product with the oracle; returns the metrics."""
    R = oracle.gemm(A, B)
    p = oracle.parity(C, R, max_abs(A), max_abs(B), A.shape[1])
    tol = TOL_F32 if kind == "f32" else TOL_BF16
    assert p["norm_max_err"] <= tol, (what, p)
    if np.any(R != 0):
        assert p["rel_fro"] <= TOL_FRO, (what, p)
    return p


def check_tiles(kind: str, A: np.ndarray, B: np.ndarray, C: np.ndarray, tiles, tile=32,
                what: str = ""):
    """Compare sampled output tiles with the oracle (one by one)."""
    tol = TOL_F32 if kind == "f32" else TOL_BF16
    ma, mb, K = max_abs(A), max_abs(B), A.shape[1]
    worst = 0.0
    num = den = 0.0
    for (r, c), R in zip(tiles, oracle.gemm_tiles(A, B, tiles, tile)):
        blk = C[r:r + R.shape[0], c:c + R.shape[1]]
        p = oracle.parity(blk, R, ma, mb, K)
        worst = max(worst, p["norm_max_err"])
        num += float(((blk.astype(np.float64) - R) ** 2).sum())
        den += float((R ** 2).sum())
    assert worst <= tol, (what, worst)
    rel = (num / den) ** 0.5 if den > 0 else 0.0
    assert rel <= TOL_FRO, (what, rel)
    return {"norm_max_err": worst, "rel_fro": rel}


def check_freivalds(A: np.ndarray, B: np.ndarray, C: np.ndarray, seed: int = 7, what: str = ""):
    """Full-coverage check: ||C x - A (B x)|| against the Frobenius gate.

    For a random +-1 vector x, E||(C - R) x||^2 = ||C - R||_F^2, so a product
    within the relative Frobenius gate gives a residual near or below
    TOL_FRO * ||C||_F; a wrong tile or row shows up far above it.
    """
    x = inputs.pm_one_vector(np.random.default_rng(seed), C.shape[1])
    f = oracle.freivalds(A, B, C, x)
    res, fro = f["residual_norm"], f["c_fro"]
    assert res <= 4 * TOL_FRO * fro + 1e-30, (what, res, fro)
    return res / fro if fro else 0.0
