"""CPU oracle for the tiled dense matrix product (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. It shares no code with the HIP library
and never imports it.

What it computes, and the passage each function follows:

* ``gemm`` / ``gemm_block`` -- the product itself, C[i,j] = sum_k A[i,k]B[k,j],
  accumulated in fp64 by a plain C triple loop (``oracle.c``). Definition:
  "09 计算受限还是访存受限" (compute- vs memory-bound), section on counting a
  matrix multiply (each output is a sum of N products, N multiplies and N
  adds); CS336 Lecture 5 GPU notes, §4.2, naive snippet. Row-major layout:
  CS336 Lecture 5 GPU notes, §4.1 (warning on row-major storage).
* ``roofline`` -- FLOPs = 2MNK and the ideal byte count (each matrix crosses
  HBM once: read A and B, write C); intensity = FLOPs / bytes. Same section
  of the compute- vs memory-bound lesson (2N^3, 12N^2 bytes, N/6), and
  CS336 Lecture 5 GPU notes, §2.1 (bf16 N = 8192 example).
* ``attainable`` -- the roofline bound P = min(peak, bandwidth * intensity)
  and the ridge point peak / bandwidth: CS336 Lecture 5 GPU notes, §2.2.
* ``parity`` -- the error metrics the tests report: the normalized max error
  max|C - R| / (max|A| max|B| K) and the relative Frobenius error.
* ``freivalds`` -- a full-coverage probabilistic check of a product
  (C x against A (B x) for a random +-1 vector x), used where the full
  product is too large for the triple loop.
* ``gelu``, ``epilogue`` -- the elementwise work a fused epilogue applies to
  the product before it is written: + bias[j], GELU(t) = t * Phi(t), +
  residual[i, j], in that order (CS336 Lecture 5 GPU notes, §4.3, operator
  fusion; LLM course ch. 15, the GELU-then-residual-add example). The pages
  name GELU without a formula; this is its exact (erf) form.
* ``gemm_nt`` / ``gemm_nt_tiles`` -- the product with B stored N x K (a
  linear layer's weight): C[i,j] = sum_k A[i,k] B[j,k], i.e. A times the
  transpose of the stored matrix (CS336 Lecture 5 GPU notes, review question
  5: op(A) in BLAS terms; §4.1: a transposed view is another memory layout).
  The stored matrix is transposed into K x N order and handed to ``gemm``.
* ``gemm_tn`` / ``gemm_tn_tiles`` -- the product with A stored K x M, the
  transpose of the M x K operand: C[i,j] = sum_k At[k,i] B[k,j], i.e. the
  pages' own example of a transposed operand, x = A.T @ B (CS336 Lecture 5
  GPU notes, review question 5; §4.1: a transposed view is a different
  memory layout, not a copy). The stored matrix is transposed into M x K
  order and handed to ``gemm``.
* ``fp8_decode``, ``e8m0_decode``, ``gemm_fp8`` / ``gemm_fp8_tiles`` -- the
  FP8 product. The two 8-bit formats are laid out as the table of
  floating-point formats in CS336 Lecture 5 GPU notes, §3.1 gives them:
  E4M3 = 1 sign, 4 exponent, 3 mantissa bits, range +-448; E5M2 = 1, 5, 2,
  range +-57,344. The pages give no exponent bias or special codes; the
  reading taken is the one those two ranges fix: an IEEE-style layout with
  bias 2^(e-1) - 1 (7 and 15) and subnormals, where E5M2 keeps IEEE's
  all-ones exponent for infinities and NaNs (largest finite 1.75 * 2^15 =
  57344) and E4M3 gives it back to finite values except the one code
  S.1111.111, its NaN (largest finite 1.75 * 2^8 = 448, no infinities).
  The fine-grained per-tile scaling the same section says FP8 needs is
  taken as block scaling along K: one power-of-two scale 2^(e-127), stored
  as an 8-bit exponent e (e = 255: NaN), per 32 consecutive k of each row
  of A and of each row of the N x K operand B; every element of a block is
  multiplied by its block's scale. The product is then
  C[i,j] = sum_k (sa[i,k/32] A[i,k]) (sb[j,k/32] B[j,k]), every term exact
  in fp64 and summed in fp64 by the C loop.
* ``attention`` / ``attention_rows`` -- the attention the pages' FlashAttention
  section computes exactly (CS336 Lecture 5 GPU notes, §6.2; GPU/attention
  notes, "why attention is memory-bound" and "online softmax"): per head,
  S = Q K^T * scale (scale 1/sqrt(d) there), P = the row softmax of S with
  its row maximum subtracted, O = P V, and the per-row logsumexp
  lse = m + log(l) that the backward pass keeps instead of P. Optionally
  causal (key j > query i masked out; the pages' sketch leaves the mask
  out). Written as the definition, in fp64 with NumPy matrix products, not
  as the blocked online recurrence the kernel uses.
* ``round_to_bf16`` -- bf16 bits of fp64 values that fp32 holds exactly,
  rounded to nearest with ties to even (CS336 Lecture 5 GPU notes, §3.1 on
  bf16 as the upper half of an fp32 word).

Every function is pinned by tests in ``tests/test_oracle.py`` against values
the pages print, closed forms (identity, permutation, all-ones, rank-1),
integer inputs and brute force on tiny shapes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

# gcc flags: no FMA contraction so the arithmetic is exactly the C text.
CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-std=c11"]


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc. Returns the path."""
    if force or not os.path.exists(_LIB_PATH) or (
        os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
    ):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *CFLAGS, _SRC, "-o", tmp], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB_PATH)
            i64 = ctypes.c_int64
            for name in ("oracle_gemm_f32", "oracle_gemm_bf16", "oracle_gemm_f64"):
                fn = getattr(lib, name)
                fn.restype = ctypes.c_int
                fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                               i64, i64, i64, i64, i64, i64, i64, ctypes.c_int]
            lib.oracle_max_threads.restype = ctypes.c_int
            _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _check_operands(A: np.ndarray, B: np.ndarray):
    if A.ndim != 2 or B.ndim != 2:
        raise ValueError("A and B must be 2-D")
    if A.dtype != B.dtype or A.dtype not in (np.float32, np.uint16):
        raise TypeError("A and B must both be float32, or both uint16 bf16 bits")
    if A.shape[1] != B.shape[0]:
        raise ValueError(f"inner dimensions differ: {A.shape} @ {B.shape}")


def gemm_block(A: np.ndarray, B: np.ndarray, rows: tuple[int, int], cols: tuple[int, int],
               threads: int | None = None) -> np.ndarray:
    """fp64 block R[i0:i1, j0:j1] of A @ B.

    A[M,K], B[K,N] are row-major float32 arrays, or uint16 arrays of bf16 bits
    (widened exactly inside the C code).
    """
    _check_operands(A, B)
    A = np.ascontiguousarray(A)
    B = np.ascontiguousarray(B)
    M, K = A.shape
    N = B.shape[1]
    i0, i1 = rows
    j0, j1 = cols
    R = np.empty((max(i1 - i0, 0), max(j1 - j0, 0)), dtype=np.float64)
    lib = _load()
    fn = lib.oracle_gemm_f32 if A.dtype == np.float32 else lib.oracle_gemm_bf16
    rc = fn(A.ctypes.data, B.ctypes.data, R.ctypes.data, M, N, K, i0, i1, j0, j1,
            int(threads or default_threads()))
    if rc != 0:
        raise ValueError(f"oracle rejected block rows={rows} cols={cols} for {A.shape}@{B.shape}")
    return R


def gemm(A: np.ndarray, B: np.ndarray, threads: int | None = None) -> np.ndarray:
    """Full fp64 product A @ B (see ``gemm_block``)."""
    _check_operands(A, B)
    return gemm_block(A, B, (0, A.shape[0]), (0, B.shape[1]), threads)


def gemm_tiles(A: np.ndarray, B: np.ndarray, tiles, tile: int = 32,
               threads: int | None = None) -> list[np.ndarray]:
    """fp64 tiles of A @ B at the given (row0, col0) corners."""
    M, N = A.shape[0], B.shape[1]
    return [gemm_block(A, B, (r, min(r + tile, M)), (c, min(c + tile, N)), threads)
            for r, c in tiles]


def gemm_nt(A: np.ndarray, Bt: np.ndarray, threads: int | None = None) -> np.ndarray:
    """fp64 A @ Bt.T for Bt[N, K] (C[i,j] = sum_k A[i,k] Bt[j,k])."""
    return gemm(A, np.ascontiguousarray(np.asarray(Bt).T), threads)


def gemm_nt_tiles(A: np.ndarray, Bt: np.ndarray, tiles, tile: int = 32,
                  threads: int | None = None) -> list[np.ndarray]:
    """fp64 tiles of A @ Bt.T at the given (row0, col0) corners."""
    out = []
    for r, c in tiles:
        c1 = min(c + tile, Bt.shape[0])
        B = np.ascontiguousarray(np.asarray(Bt)[c:c1].T)
        out.append(gemm_block(A, B, (r, min(r + tile, A.shape[0])), (0, c1 - c), threads))
    return out


def gemm_tn(At: np.ndarray, B: np.ndarray, threads: int | None = None) -> np.ndarray:
    """fp64 At.T @ B for At[K, M] (A stored transposed, K x M) and B[K, N]:
    C[i,j] = sum_k At[k,i] B[k,j]."""
    return gemm(np.ascontiguousarray(np.asarray(At).T), B, threads)


def gemm_tn_tiles(At: np.ndarray, B: np.ndarray, tiles, tile: int = 32,
                  threads: int | None = None) -> list[np.ndarray]:
    """fp64 tiles of At.T @ B at the given (row0, col0) corners."""
    out = []
    for r, c in tiles:
        r1 = min(r + tile, At.shape[1])
        A = np.ascontiguousarray(np.asarray(At)[:, r:r1].T)
        out.append(gemm_block(A, B, (0, r1 - r), (c, min(c + tile, B.shape[1])), threads))
    return out


def widen(X: np.ndarray) -> np.ndarray:
    """Exact fp64 value of a float32 array or of an array of bf16 bits."""
    if X.dtype == np.uint16:
        return (X.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return X.astype(np.float64)


# ---------------------------------------------------------------------------
# Cost model
# ---------------------------------------------------------------------------

def roofline(M: int, N: int, K: int, in_bytes: int, out_bytes: int):
    """(flops, bytes, intensity) of one product with every matrix crossing HBM once.

    flops = 2*M*N*K (a multiply-add counts as two floating-point operations);
    bytes = (M*K + K*N) * in_bytes + M*N * out_bytes (read A and B, write C).
    """
    flops = 2 * M * N * K
    nbytes = (M * K + K * N) * in_bytes + M * N * out_bytes
    return flops, nbytes, (flops / nbytes if nbytes else 0.0)


def attainable(peak: float, bandwidth: float, intensity: float) -> float:
    """Roofline: attainable rate = min(peak, bandwidth * intensity)."""
    return min(peak, bandwidth * intensity)


def ridge(peak: float, bandwidth: float) -> float:
    """Intensity at which the bandwidth slope meets the compute roof."""
    return peak / bandwidth


# ---------------------------------------------------------------------------
# Checks
# ---------------------------------------------------------------------------

def parity(C: np.ndarray, R: np.ndarray, max_a: float, max_b: float, K: int) -> dict:
    """Error metrics of a computed product C against the fp64 oracle R.

    ``norm_max_err`` = max|C - R| / (max|A| * max|B| * K) (0 when that
    denominator is 0 and C == R); ``rel_fro`` = ||C - R||_F / ||R||_F.
    """
    C64 = np.asarray(C, dtype=np.float64)
    R64 = np.asarray(R, dtype=np.float64)
    if C64.shape != R64.shape:
        raise ValueError(f"shape mismatch {C64.shape} vs {R64.shape}")
    diff = np.abs(C64 - R64)
    max_abs = float(diff.max()) if diff.size else 0.0
    denom = float(max_a) * float(max_b) * float(K)
    if denom > 0:
        norm = max_abs / denom
    else:
        norm = 0.0 if max_abs == 0.0 else float("inf")
    rn = float(np.linalg.norm(R64)) if R64.size else 0.0
    dn = float(np.linalg.norm(C64 - R64)) if R64.size else 0.0
    rel = dn / rn if rn > 0 else (0.0 if dn == 0.0 else float("inf"))
    return {"norm_max_err": norm, "rel_fro": rel, "max_abs_err": max_abs}


def freivalds(A: np.ndarray, B: np.ndarray, C: np.ndarray, x: np.ndarray) -> dict:
    """Compare C @ x with A @ (B @ x) in fp64 for a +-1 vector x.

    Returns the largest row residual, the residual's 2-norm, the scale
    sum_j |C[i,j]| (max over rows) and ||C||_F, from which a caller forms a
    tolerance. For random +-1 x, E||(C - R) x||^2 = ||C - R||_F^2 (R the exact
    product). Cost O(MK + KN + MN).
    """
    A64 = widen(np.asarray(A))
    B64 = widen(np.asarray(B))
    C64 = np.asarray(C, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    lhs = C64 @ x
    rhs = A64 @ (B64 @ x)
    res = np.abs(lhs - rhs)
    return {
        "max_residual": float(res.max()) if res.size else 0.0,
        "residual_norm": float(np.linalg.norm(res)),
        "max_row_abs_sum": float(np.abs(C64).sum(axis=1).max()) if C64.size else 0.0,
        "c_fro": float(np.linalg.norm(C64)),
    }


# ---------------------------------------------------------------------------
# Fused epilogue (elementwise work on the product before it is stored)
# ---------------------------------------------------------------------------

def gelu(x) -> np.ndarray:
    """GELU(x) = x * Phi(x) = x/2 * (1 + erf(x / sqrt(2))) in fp64, Phi the
    standard normal CDF (the exact form, not the tanh approximation)."""
    from scipy.special import erf
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def epilogue(R: np.ndarray, bias: np.ndarray | None = None,
             residual: np.ndarray | None = None, use_gelu: bool = False) -> np.ndarray:
    """fp64 epilogue of a product R[M, N]: R + bias[j] (bias broadcast along
    the rows), then GELU, then + residual[i, j]. bias and residual are
    float32 arrays or bf16 bits, widened exactly."""
    T = np.array(R, dtype=np.float64)
    if bias is not None:
        T = T + widen(np.asarray(bias))[None, :]
    if use_gelu:
        T = gelu(T)
    if residual is not None:
        T = T + widen(np.asarray(residual))
    return T


def round_to_bf16(x) -> np.ndarray:
    """bf16 bits nearest to each value (ties to even). The values must be
    exactly representable in fp32 (checked), so this is the rounding of the
    fp32 word's lower 16 bits."""
    x = np.asarray(x, dtype=np.float64)
    f = x.astype(np.float32)
    if not np.array_equal(f.astype(np.float64), x, equal_nan=True):
        raise ValueError("round_to_bf16 takes values that fp32 holds exactly")
    u = f.view(np.uint32).astype(np.uint64)
    upper, lower = u >> 16, u & 0xFFFF
    up = (lower > 0x8000) | ((lower == 0x8000) & ((upper & 1) == 1))
    return (upper + up.astype(np.uint64)).astype(np.uint16)



# ---------------------------------------------------------------------------
# FP8 operands with block scales
# ---------------------------------------------------------------------------

FP8_FORMATS = {"e4m3": (4, 3), "e5m2": (5, 2)}  # (exponent bits, mantissa bits)
SCALE_BLOCK = 32  # k per block scale


def fp8_decode(codes, fmt: str) -> np.ndarray:
    """Exact fp64 value of each FP8 code (uint8) in format "e4m3" or "e5m2".

    Fields sign | exponent | mantissa; exponent bias 2^(E-1) - 1. Exponent 0
    holds the subnormals m/2^M * 2^(1-bias); otherwise (1 + m/2^M) *
    2^(e-bias). E5M2's all-ones exponent is infinity (m = 0) or NaN; E4M3's
    all-ones exponent is finite except S.1111.111 (NaN)."""
    if fmt not in FP8_FORMATS:
        raise ValueError(f"unknown FP8 format {fmt!r}")
    E, Mb = FP8_FORMATS[fmt]
    bias = (1 << (E - 1)) - 1
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> Mb) & ((1 << E) - 1)
    m = (c & ((1 << Mb) - 1)).astype(np.float64)
    frac = m / float(1 << Mb)
    mag = np.where(e == 0, frac * 2.0 ** (1 - bias), (1.0 + frac) * np.exp2((e - bias).astype(np.float64)))
    top = (1 << E) - 1
    if fmt == "e5m2":
        mag = np.where((e == top) & (m == 0), np.inf, mag)
        mag = np.where((e == top) & (m != 0), np.nan, mag)
    else:
        mag = np.where((e == top) & (m == (1 << Mb) - 1), np.nan, mag)
    return sign * mag


def e8m0_decode(codes) -> np.ndarray:
    """Exact fp64 value 2^(e-127) of each 8-bit scale exponent; 255 is NaN."""
    e = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    return np.where(e == 255, np.nan, np.exp2((e - 127).astype(np.float64)))


def fp8_scaled(codes, fmt: str, scales=None) -> np.ndarray:
    """fp64 values of a row-major [R, K] FP8 operand, each element times the
    scale of its 32-k block (scales: [R, K/32] exponents, or None for 1)."""
    X = fp8_decode(codes, fmt)
    if scales is None:
        return X
    R, K = X.shape
    if K % SCALE_BLOCK:
        raise ValueError("a block-scaled operand needs K a multiple of 32")
    S = e8m0_decode(scales)
    if S.shape != (R, K // SCALE_BLOCK):
        raise ValueError(f"scales {S.shape} do not match operand {X.shape}")
    return X * np.repeat(S, SCALE_BLOCK, axis=1)


def gemm_f64_nt_block(a: np.ndarray, b: np.ndarray, rows, cols,
                      threads: int | None = None) -> np.ndarray:
    """fp64 block of a @ b.T for fp64 a[M, K], b[N, K] (the C loop)."""
    a = np.ascontiguousarray(a, dtype=np.float64)
    bt = np.ascontiguousarray(np.asarray(b, dtype=np.float64)[cols[0]:cols[1]].T)
    M, K = a.shape
    if bt.shape[0] != K:
        raise ValueError(f"inner dimensions differ: {a.shape} vs {np.asarray(b).shape}")
    i0, i1 = rows
    R = np.empty((max(i1 - i0, 0), bt.shape[1]), dtype=np.float64)
    rc = _load().oracle_gemm_f64(a.ctypes.data, bt.ctypes.data, R.ctypes.data, M, bt.shape[1], K,
                                 i0, i1, 0, bt.shape[1], int(threads or default_threads()))
    if rc != 0:
        raise ValueError(f"oracle rejected block rows={rows} cols={cols}")
    return R


def gemm_fp8(A, a_fmt: str, B, b_fmt: str, a_scale=None, b_scale=None,
             threads: int | None = None) -> np.ndarray:
    """fp64 C[i,j] = sum_k (sa[i,k/32] A[i,k]) (sb[j,k/32] B[j,k]) for FP8 codes
    A[M, K] and B[N, K] (B stored N x K), block scales optional."""
    a = fp8_scaled(A, a_fmt, a_scale)
    b = fp8_scaled(B, b_fmt, b_scale)
    return gemm_f64_nt_block(a, b, (0, a.shape[0]), (0, b.shape[0]), threads)


def gemm_fp8_tiles(A, a_fmt: str, B, b_fmt: str, tiles, a_scale=None, b_scale=None,
                   tile: int = 32, threads: int | None = None) -> list[np.ndarray]:
    """fp64 tiles of the FP8 product at the given (row0, col0) corners."""
    out = []
    for r, c in tiles:
        r1, c1 = min(r + tile, A.shape[0]), min(c + tile, B.shape[0])
        a = fp8_scaled(A[r:r1], a_fmt, None if a_scale is None else a_scale[r:r1])
        b = fp8_scaled(B[c:c1], b_fmt, None if b_scale is None else b_scale[c:c1])
        out.append(gemm_f64_nt_block(a, b, (0, r1 - r), (0, c1 - c), threads))
    return out


# ---------------------------------------------------------------------------
# Attention (the FlashAttention forward's result)
# ---------------------------------------------------------------------------

def attention_rows(Q, K, V, rows, scale: float, causal: bool = False):
    """fp64 (O[rows], lse[rows]) of one head: Q [n_q, d], K and V [n_kv, d]
    (float arrays or bf16 bits), `rows` the query indices wanted."""
    q = widen(np.asarray(Q))[np.asarray(rows)]
    k = widen(np.asarray(K))
    v = widen(np.asarray(V))
    S = (q @ k.T) * float(scale)
    if causal:
        keys = np.arange(k.shape[0])[None, :]
        S = np.where(keys > np.asarray(rows)[:, None], -np.inf, S)
    m = S.max(axis=1, keepdims=True)
    P = np.exp(S - m)
    l = P.sum(axis=1, keepdims=True)
    O = (P @ v) / l
    return O, (m + np.log(l))[:, 0]


def attention(Q, K, V, scale: float, causal: bool = False):
    """fp64 (O, lse) for Q [..., n_q, d], K and V [..., n_kv, d] (leading
    batch/head dimensions alike): every head separately."""
    Q = np.asarray(Q)
    K = np.asarray(K)
    V = np.asarray(V)
    lead = Q.shape[:-2]
    n_q, d = Q.shape[-2:]
    Qf = Q.reshape(-1, n_q, d)
    Kf = K.reshape(-1, K.shape[-2], d)
    Vf = V.reshape(-1, V.shape[-2], d)
    O = np.empty((Qf.shape[0], n_q, d))
    L = np.empty((Qf.shape[0], n_q))
    for h in range(Qf.shape[0]):
        O[h], L[h] = attention_rows(Qf[h], Kf[h], Vf[h], np.arange(n_q), scale, causal)
    return O.reshape(*lead, n_q, d), L.reshape(*lead, n_q)
