"""Seeded synthetic inputs for the GEMM workloads.

This module is shared by the HIP path's tests/bench and by the CPU oracle's
tests. It holds no GEMM arithmetic: it only draws numbers and encodes them in
the storage formats the library takes (fp32, or bf16 as raw uint16 bits).

Recipe (one fresh PCG64 generator per workload, seeded with the workload's
seed; A is drawn first, row-major, then B):

* fp32 workloads: i.i.d. uniform[-1, 1) drawn in float64, rounded to fp32
  (round-to-nearest-even).
* bf16 workloads: i.i.d. normal(0, sigma) drawn in float64 (sigma is a
  standard deviation), rounded to fp32 and then to bf16, both
  round-to-nearest-even.
* a fused-epilogue workload's bias: normal(0, bias_sigma) from its own
  generator, seeded with (seed, 1), in the output's element type.
* a workload whose B is stored N x K draws B in that order (row n, then k).

The bf16 format is the upper half of an IEEE fp32 word (1 sign, 8 exponent,
7 mantissa bits), as the CS336 Lecture 5 GPU notes describe in §3.1 (table of
floating-point formats). Those notes remark that converting fp32 to bf16 can
be a plain truncation; the inputs here use round-to-nearest-even instead, the
conversion PyTorch applies. Either choice is valid because the oracle and the
GPU read the very same bits.
"""
from __future__ import annotations

import dataclasses
import hashlib

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "fp32_to_bf16_bits",
    "bf16_bits_to_fp32",
    "make_inputs",
    "make_bias",
    "uniform_fp32",
    "normal_bf16",
    "small_int_matrix",
    "pm_one_vector",
    "sample_tiles",
    "digest",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic GEMM workload: C[M,N] = A[M,K] @ B[K,N], row-major."""

    name: str
    kind: str  # "f32" or "bf16"
    M: int
    N: int
    K: int
    seed: int
    dist: str  # "uniform" (fp32 workloads) or "normal" (bf16 workloads)
    sigma_a: float = 1.0
    sigma_b: float = 1.0
    # Fused epilogue (bf16 workloads): bias of this standard deviation (0: no
    # bias), GELU, and the output's element type ("f32" or "bf16").
    bias_sigma: float = 0.0
    gelu: bool = False
    out: str = "f32"
    # How B is stored: "kn" (K x N) or "nk" (N x K, a linear layer's weight;
    # the product is then A @ B.T).
    b_layout: str = "kn"

    @property
    def has_epilogue(self) -> bool:
        return self.bias_sigma > 0 or self.gelu or self.out != "f32"


# The workloads, with their sizes, seeds and value distributions.
WORKLOADS = {
    w.name: w
    for w in (
        Workload("f32_256", "f32", 256, 256, 256, 0, "uniform"),
        Workload("f32_4096", "f32", 4096, 4096, 4096, 1, "uniform"),
        Workload("bf16_4096", "bf16", 4096, 4096, 4096, 2, "normal"),
        Workload("bf16_8192", "bf16", 8192, 8192, 8192, 2, "normal"),
        Workload("bf16_mlp", "bf16", 8192, 14336, 4096, 3, "normal", 1.0, 0.02),
        # The same product as the MLP up-projection above, finished in the
        # kernel: + bias, GELU, bf16 output.
        Workload("bf16_mlp_gelu", "bf16", 8192, 14336, 4096, 3, "normal", 1.0, 0.02,
                 bias_sigma=0.02, gelu=True, out="bf16"),
        # Weights stored N x K, as a linear layer keeps them: the MLP
        # up-projection with bias, GELU and bf16 output, and the small-M shape.
        Workload("bf16_linear_gelu", "bf16", 8192, 14336, 4096, 5, "normal", 1.0, 0.02,
                 bias_sigma=0.02, gelu=True, out="bf16", b_layout="nk"),
        Workload("bf16_skinny_nk", "bf16", 16, 8192, 8192, 6, "normal", 1.0, 0.02,
                 b_layout="nk"),
        Workload("bf16_skinny", "bf16", 16, 8192, 8192, 4, "normal", 1.0, 0.02),
    )
}


def fp32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bits.

    Meant for finite values; +-Inf map to the bf16 infinities and the default
    quiet NaN (0x7FC00000) to a bf16 NaN. A NaN whose payload sits only in the
    low 16 bits would round to Inf: not used here.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_fp32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bits to fp32 (exact)."""
    u = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32)


def uniform_fp32(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.uniform(-1.0, 1.0, size=shape).astype(np.float32)


def normal_bf16(rng: np.random.Generator, shape, sigma: float) -> np.ndarray:
    x = rng.standard_normal(size=shape)
    if sigma != 1.0:
        x *= sigma
    return fp32_to_bf16_bits(x.astype(np.float32))


def make_inputs(w: Workload | str):
    """Return (A, B) for a workload.

    fp32 workloads give float32 arrays; bf16 workloads give uint16 bf16 bits.
    B comes in its stored shape: K x N, or N x K for b_layout "nk" (drawn in
    that order).
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    rng = np.random.default_rng(w.seed)
    if w.kind == "f32":
        if w.dist != "uniform":
            raise ValueError(w.dist)
        A = uniform_fp32(rng, (w.M, w.K))
        B = uniform_fp32(rng, (w.K, w.N))
    elif w.kind == "bf16":
        if w.dist != "normal":
            raise ValueError(w.dist)
        A = normal_bf16(rng, (w.M, w.K), w.sigma_a)
        B = normal_bf16(rng, (w.N, w.K) if w.b_layout == "nk" else (w.K, w.N), w.sigma_b)
    else:
        raise ValueError(w.kind)
    return A, B


def make_bias(w: Workload | str) -> np.ndarray:
    """The bias of an epilogue workload: N values normal(0, bias_sigma) from a
    PCG64 generator seeded with (seed, 1) (independent of A and B), in the
    output's element type (fp32, or bf16 bits rounded to nearest even)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    rng = np.random.default_rng((w.seed, 1))
    x = (rng.standard_normal(w.N) * w.bias_sigma).astype(np.float32)
    return fp32_to_bf16_bits(x) if w.out == "bf16" else x


def small_int_matrix(rng: np.random.Generator, shape, lo: int = -3, hi: int = 3,
                     kind: str = "f32") -> np.ndarray:
    """Integer values in [lo, hi], stored as fp32 or bf16 bits (both exact)."""
    x = rng.integers(lo, hi + 1, size=shape).astype(np.float32)
    return x if kind == "f32" else fp32_to_bf16_bits(x)


def pm_one_vector(rng: np.random.Generator, n: int) -> np.ndarray:
    """A random +-1 vector (float64), e.g. for a Freivalds check."""
    return rng.integers(0, 2, size=n).astype(np.float64) * 2.0 - 1.0


def sample_tiles(M: int, N: int, count: int = 64, tile: int = 32, seed: int = 10_003):
    """`count` distinct tile-aligned output tiles, as (row0, col0) pairs.

    Tiles are drawn without replacement from the tile grid with their own seed,
    so the choice does not depend on the input draws.
    """
    gm, gn = M // tile, N // tile
    count = min(count, gm * gn)
    idx = np.random.default_rng(seed).choice(gm * gn, size=count, replace=False)
    return [(int(i // gn) * tile, int(i % gn) * tile) for i in np.sort(idx)]


def digest(*arrays: np.ndarray) -> str:
    """SHA-256 over the raw bytes of the arrays (pins the recipe)."""
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()
