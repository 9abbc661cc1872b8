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
* a workload whose B is stored N x K draws B in that order (row n, then k);
  one whose A is stored K x M draws A in that order (row k, then m).
* FP8 workloads (B always N x K): normal(0, sigma) in float64, then either
  rounded straight to FP8 (nearest, ties to even, saturating at the largest
  finite value), or block-scaled first as the OCP Microscaling (MX) recipe
  does: per 32 consecutive k of a row, the shared scale is 2^s with
  s = floor(log2(max |x|)) - emax (emax = 8 for E4M3, whose largest value
  is 1.75 * 2^8 = 448; 15 for E5M2, 1.75 * 2^15 = 57344), stored as the
  8-bit exponent s + 127, and every element of the block is x / 2^s rounded
  to FP8 as above. An all-zero block gets s = 0.
* attention workloads: Q, then K, then V, each [batch, heads, seq, head_dim]
  normal(0, 1) rounded to bf16 (as the bf16 workloads).

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
    "make_integer_inputs",
    "pm_one_vector",
    "sample_tiles",
    "digest",
    "encode_fp8",
    "mx_quantize",
    "make_fp8_inputs",
    "AttnWorkload",
    "ATTN_WORKLOADS",
    "make_attention_inputs",
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
    # How A is stored: "mk" (M x K) or "km" (K x M, the product is then
    # A.T @ B, as in x = A.T @ B).
    a_layout: str = "mk"
    # FP8 workloads: the formats of A and B, and whether they carry block
    # scales (one 8-bit power-of-two exponent per 32 k of each row).
    fp8: tuple = ("e4m3", "e4m3")
    scaled: bool = False

    @property
    def has_epilogue(self) -> bool:
        return self.bias_sigma > 0 or self.gelu or self.out != "f32"


# The workloads, with their sizes, seeds and value distributions.
WORKLOADS = {
    w.name: w
    for w in (
        Workload("f32_256", "f32", 256, 256, 256, 0, "uniform"),
        Workload("f32_4096", "f32", 4096, 4096, 4096, 1, "uniform"),
        # The fp32 4096^3 product with a transposed operand: B stored N x K,
        # and A stored K x M.
        Workload("f32_4096_nk", "f32", 4096, 4096, 4096, 11, "uniform", b_layout="nk"),
        Workload("f32_4096_tn", "f32", 4096, 4096, 4096, 12, "uniform", a_layout="km"),
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
        # The square bf16 product with A stored K x M: x = A.T @ B.
        Workload("bf16_8192_tn", "bf16", 8192, 8192, 8192, 10, "normal", a_layout="km"),
        # The MLP up-projection in E4M3 with block scales, weight N x K,
        # bf16 output.
        Workload("fp8_mlp", "fp8", 8192, 14336, 4096, 7, "normal", 1.0, 0.02, out="bf16",
                 b_layout="nk", fp8=("e4m3", "e4m3"), scaled=True),
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
    A and B come in their stored shapes: A M x K, or K x M for a_layout "km";
    B K x N, or N x K for b_layout "nk" (each drawn in that order).
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    rng = np.random.default_rng(w.seed)
    if w.kind == "f32":
        if w.dist != "uniform":
            raise ValueError(w.dist)
        A = uniform_fp32(rng, (w.K, w.M) if w.a_layout == "km" else (w.M, w.K))
        B = uniform_fp32(rng, (w.N, w.K) if w.b_layout == "nk" else (w.K, w.N))
    elif w.kind == "bf16":
        if w.dist != "normal":
            raise ValueError(w.dist)
        A = normal_bf16(rng, (w.K, w.M) if w.a_layout == "km" else (w.M, w.K), w.sigma_a)
        B = normal_bf16(rng, (w.N, w.K) if w.b_layout == "nk" else (w.K, w.N), w.sigma_b)
    elif w.kind == "fp8":
        raise ValueError("FP8 workloads come with scales: use make_fp8_inputs")
    else:
        raise ValueError(w.kind)
    return A, B


# FP8 formats: (exponent bits, mantissa bits, exponent of the largest finite
# value, the largest finite value).
_FP8 = {"e4m3": (4, 3, 8, 448.0), "e5m2": (5, 2, 15, 57344.0)}
SCALE_BLOCK = 32


def encode_fp8(x, fmt: str) -> np.ndarray:
    """FP8 codes (uint8) of finite float64 values: nearest representable
    value, ties to even, magnitudes above the largest finite one saturate to
    it. Exponent bias 2^(E-1) - 1, subnormals below 2^(1 - bias)."""
    E, Mb, _, top = _FP8[fmt]
    bias = (1 << (E - 1)) - 1
    x = np.asarray(x, dtype=np.float64)
    if not np.isfinite(x).all():
        raise ValueError("encode_fp8 takes finite values")
    neg = np.signbit(x)
    a = np.abs(x)
    _, ex = np.frexp(a)                              # a = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex - 1, 1 - bias)                 # exponent of a's binade
    q = np.ldexp(1.0, e - Mb)                        # spacing of values there
    r = np.minimum(np.rint(a / q) * q, top)          # rint: ties to even
    _, ex2 = np.frexp(r)
    normal = r >= np.ldexp(1.0, 1 - bias)
    e2 = np.where(normal, ex2 - 1, 1 - bias)
    mant = np.ldexp(r, Mb - e2)                      # integer: 2^Mb + m, or m
    m_field = np.where(normal, mant - (1 << Mb), mant).astype(np.int64)
    e_field = np.where(normal, e2 + bias, 0).astype(np.int64)
    code = (neg.astype(np.int64) << 7) | (e_field << Mb) | m_field
    return code.astype(np.uint8)


def mx_quantize(X, fmt: str):
    """Block-scale a float64 [R, K] matrix (K a multiple of 32): returns
    (codes [R, K] uint8, scale exponents [R, K/32] uint8), value =
    fp8(code) * 2^(scale - 127)."""
    X = np.asarray(X, dtype=np.float64)
    R, K = X.shape
    if K % SCALE_BLOCK:
        raise ValueError("K must be a multiple of 32")
    emax = _FP8[fmt][2]
    blocks = X.reshape(R, K // SCALE_BLOCK, SCALE_BLOCK)
    amax = np.abs(blocks).max(axis=2)
    _, ex = np.frexp(amax)
    s = np.where(amax > 0, ex - 1 - emax, 0)
    s = np.clip(s, -127, 127)
    codes = encode_fp8(np.ldexp(blocks, -s[:, :, None]), fmt).reshape(R, K)
    return codes, (s + 127).astype(np.uint8)


def make_fp8_inputs(w: Workload | str):
    """(A, B, a_scale, b_scale) of an FP8 workload: codes A [M, K] and
    B [N, K]; scale exponents [M, K/32] and [N, K/32], or None when the
    workload is unscaled. A is drawn first, then B."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    if w.kind != "fp8" or w.b_layout != "nk":
        raise ValueError("an FP8 workload with B stored N x K")
    rng = np.random.default_rng(w.seed)
    xa = rng.standard_normal((w.M, w.K)) * w.sigma_a
    xb = rng.standard_normal((w.N, w.K)) * w.sigma_b
    fa, fb = w.fp8
    if not w.scaled:
        return encode_fp8(xa, fa), encode_fp8(xb, fb), None, None
    A, sa = mx_quantize(xa, fa)
    B, sb = mx_quantize(xb, fb)
    return A, B, sa, sb


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


def make_integer_inputs(w: Workload | str, lo: int = -3, hi: int = 3):
    """(A, B) with the workload's shapes, storage types and layouts, but
    i.i.d. integers in [lo, hi] from a PCG64 generator seeded with (seed, 2)
    (A drawn first). With |values| <= 3 every partial sum of a product with
    K <= 8192 is an integer of magnitude at most 9K < 2^24, exact in fp32
    under any summation order, so any correct kernel returns the exact
    product bit for bit."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    if w.kind not in ("f32", "bf16"):
        raise ValueError(w.kind)
    rng = np.random.default_rng((w.seed, 2))
    A = small_int_matrix(rng, (w.K, w.M) if w.a_layout == "km" else (w.M, w.K), lo, hi,
                         kind=w.kind)
    B = small_int_matrix(rng, (w.N, w.K) if w.b_layout == "nk" else (w.K, w.N), lo, hi,
                         kind=w.kind)
    return A, B


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


@dataclasses.dataclass(frozen=True)
class AttnWorkload:
    """One attention forward: softmax(Q K^T / sqrt(d)) V per (batch, head),
    Q, K, V and O [batch, heads, seq, head_dim] in bf16."""

    name: str
    batch: int
    heads: int
    seq: int
    head_dim: int
    causal: bool
    seed: int

    @property
    def scale(self) -> float:
        return self.head_dim ** -0.5

    @property
    def flops(self) -> float:
        """2 * 2 * d per (query, visible key) pair: Q K^T and P V."""
        pairs = self.seq * (self.seq + 1) // 2 if self.causal else self.seq * self.seq
        return 4.0 * self.batch * self.heads * self.head_dim * pairs


ATTN_WORKLOADS = {
    w.name: w
    for w in (
        AttnWorkload("attn_fwd", 4, 32, 4096, 128, False, 8),
        AttnWorkload("attn_fwd_causal", 4, 32, 4096, 128, True, 9),
    )
}


def make_attention_inputs(w: AttnWorkload | str):
    """(Q, K, V) as bf16 bits, each [batch, heads, seq, head_dim]."""
    if isinstance(w, str):
        w = ATTN_WORKLOADS[w]
    rng = np.random.default_rng(w.seed)
    shape = (w.batch, w.heads, w.seq, w.head_dim)
    return tuple(normal_bf16(rng, shape, 1.0) for _ in range(3))
