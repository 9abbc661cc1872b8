"""Fused epilogue of the bf16 product on every path (needs an MI355X).

gemm_bf16_epilogue finishes each output in the kernel that computes it:
t = sum_k A[i,k] B[k,j]; t += bias[j]; t = GELU(t); t += residual[i,j];
stored as fp32 or bf16 (nearest, ties to even). The oracle applies the same
steps in fp64 to its fp64 product. Checks:
  * small-integer operands, no GELU: every value is exact in fp32, so fp32
    outputs must equal the oracle and bf16 outputs its nearest-even rounding
    bit for bit (sums above 256 include ties);
  * GELU alone on an identity product: within a few fp32 rounding errors;
  * random operands with every step on: within a bound built from the fp32
    summation error of the product (K * 2^-24 * sum_k |a_k b_k|), GELU's
    slope (< 1.13), fp32 rounding and, for bf16 outputs, half a bf16 unit;
    plus a relative Frobenius gate;
  * in-place residual, K = 0, and no epilogue terms (equal to the plain
    product bit for bit).
"""
import numpy as np
import pytest

import oracle
import tiled_dense_matrix_amd as tdm
from tiled_dense_matrix_amd import inputs

from helpers import log, run, to_device

torch = pytest.importorskip("torch")

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

P = tdm.Path
PATHS = [P.AUTO, P.EDGE, P.MFMA, P.SKINNY]


def paths_for(M, N, K):
    return [p for p in PATHS if tdm.tdm_path_supports(tdm.Kind.BF16_F32ACC, p, M, N, K)]


def as_out_type(X: np.ndarray, out_bf16: bool) -> np.ndarray:
    """fp32 values in the output's element type (bf16 bits, nearest even)."""
    X = np.asarray(X, np.float32)
    return inputs.fp32_to_bf16_bits(X) if out_bf16 else X


def epi(A, B, out_bf16, bias=None, residual=None, gelu=False, path=P.AUTO, D=None):
    D = tdm.tdm_gemm_bf16_epilogue_path(
        to_device(A), to_device(B), D, out_dtype=torch.bfloat16 if out_bf16 else torch.float32,
        bias=None if bias is None else to_device(bias),
        residual=None if residual is None else to_device(residual), gelu=gelu, path=path)
    torch.cuda.synchronize()
    return D


def host(D) -> np.ndarray:
    """D as float32 values, or as bf16 bits."""
    if D.dtype == torch.bfloat16:
        return D.view(torch.int16).cpu().numpy().view(np.uint16)
    return D.cpu().numpy()


def bound(K, S, T, E, out_bf16):
    """Largest admissible |D - E| per element: fp32 summation of the product
    (K * 2^-24 * sum_k |a_k b_k|) and of the bias through GELU's slope
    (< 1.13), GELU's own evaluation, the final fp32 rounding, and half a bf16
    unit for bf16 outputs. S = sum_k |a_k b_k|, T = the value GELU takes, E =
    the fp64 result."""
    return (1.13 * (K * 2.0 ** -24 * S + 2.0 ** -24 * np.abs(T)) + 3e-7 * np.maximum(1.0, np.abs(T))
            + 2.0 ** -23 * np.abs(E) + (2.0 ** -8 * np.abs(E) if out_bf16 else 0.0))


def small_ints(rng, shape, lo, hi):
    return rng.integers(lo, hi + 1, size=shape).astype(np.float32)


EXACT_SHAPES = [(16, 256, 64), (5, 7, 3), (130, 200, 136), (300, 520, 136), (16, 1024, 2048)]


def _exact_cases():
    for shape in EXACT_SHAPES:
        for p in paths_for(*shape):
            for out in ("bf16", "f32"):
                yield pytest.param(shape, p, out, id=f"{shape[0]}x{shape[1]}x{shape[2]}-{p.name}-{out}")


@pytest.mark.parametrize("shape,path,out", list(_exact_cases()))
def test_exact_bias_residual_and_rounding(shape, path, out):
    M, N, K = shape
    log(f"case epilogue exact {shape} path={path.name} out={out}")
    rng = np.random.default_rng(M * 3 + N * 5 + K)
    A = inputs.fp32_to_bf16_bits(small_ints(rng, (M, K), -2, 2))
    B = inputs.fp32_to_bf16_bits(small_ints(rng, (K, N), -2, 2))
    out_bf16 = out == "bf16"
    bias = as_out_type(small_ints(rng, (N,), -4, 4), out_bf16)
    res = as_out_type(small_ints(rng, (M, N), -4, 4), out_bf16)
    E = oracle.epilogue(oracle.gemm(A, B), bias, res)
    got = host(epi(A, B, out_bf16, bias, res, path=path))
    if out_bf16:
        assert np.array_equal(got, oracle.round_to_bf16(E)), path.name
    else:
        assert np.array_equal(got.astype(np.float64), E), path.name


@pytest.mark.parametrize("M", [16, 64])
def test_gelu_on_an_identity_product(M):
    K, N = 64, 512
    x = np.linspace(-6.0, 6.0, K * N).reshape(K, N).astype(np.float32)
    B = inputs.fp32_to_bf16_bits(x)
    A = inputs.fp32_to_bf16_bits(np.eye(M, K, dtype=np.float32))
    ref = oracle.gelu(oracle.widen(B)[:M])
    for p in paths_for(M, N, K):
        log(f"case epilogue gelu M={M} path={p.name}")
        got = host(epi(A, B, False, gelu=True, path=p)).astype(np.float64)
        tol = 3e-7 * np.maximum(1.0, np.abs(oracle.widen(B)[:M]))
        assert np.all(np.abs(got - ref) <= tol), (p.name, float(np.abs(got - ref).max()))


RANDOM_SHAPES = [(16, 1024, 2048), (130, 200, 136), (512, 768, 1024), (7, 40, 24)]


def _random_cases():
    for shape in RANDOM_SHAPES:
        for p in paths_for(*shape):
            for out in ("bf16", "f32"):
                yield pytest.param(shape, p, out, id=f"{shape[0]}x{shape[1]}x{shape[2]}-{p.name}-{out}")


@pytest.mark.parametrize("shape,path,out", list(_random_cases()))
def test_random_operands_every_step(shape, path, out):
    M, N, K = shape
    log(f"case epilogue random {shape} path={path.name} out={out}")
    rng = np.random.default_rng(M + 7 * N + 11 * K)
    A = inputs.normal_bf16(rng, (M, K), 1.0)
    B = inputs.normal_bf16(rng, (K, N), 0.02)
    out_bf16 = out == "bf16"
    bias = as_out_type(rng.standard_normal(N) * 0.5, out_bf16)
    res = as_out_type(rng.standard_normal((M, N)), out_bf16)
    R = oracle.gemm(A, B)
    E = oracle.epilogue(R, bias, res, use_gelu=True)
    T = oracle.epilogue(R, bias)  # the value GELU is applied to
    S = oracle.gemm(A & 0x7FFF, B & 0x7FFF)  # sum_k |a_k b_k|
    got = host(epi(A, B, out_bf16, bias, res, gelu=True, path=path))
    got = oracle.widen(got) if out_bf16 else got.astype(np.float64)
    tol = bound(K, S, T, E, out_bf16)
    err = np.abs(got - E)
    assert np.all(err <= tol), (path.name, float((err / tol).max()))
    rel = float(np.linalg.norm(got - E) / np.linalg.norm(E))
    assert rel <= (4e-3 if out_bf16 else 1e-5), (path.name, rel)


@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_in_place_residual(out):
    M, N, K = 256, 512, 256
    rng = np.random.default_rng(5)
    A = inputs.normal_bf16(rng, (M, K), 1.0)
    B = inputs.normal_bf16(rng, (K, N), 0.05)
    out_bf16 = out == "bf16"
    bias = as_out_type(rng.standard_normal(N), out_bf16)
    res = as_out_type(rng.standard_normal((M, N)), out_bf16)
    for p in paths_for(M, N, K):
        log(f"case epilogue in-place path={p.name} out={out}")
        ref = host(epi(A, B, out_bf16, bias, res, gelu=True, path=p))
        D = to_device(res)
        if out_bf16:
            D = D.view(torch.bfloat16)
        tdm.tdm_gemm_bf16_epilogue_path(to_device(A), to_device(B), D, bias=to_device(bias),
                                        residual=D, gelu=True, path=p)
        torch.cuda.synchronize()
        assert np.array_equal(host(D), ref), p.name


@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_k_zero_is_the_epilogue_of_zero(out):
    M, N = 33, 70
    rng = np.random.default_rng(6)
    out_bf16 = out == "bf16"
    bias = as_out_type(rng.standard_normal(N), out_bf16)
    res = as_out_type(rng.standard_normal((M, N)), out_bf16)
    A = np.zeros((M, 0), np.uint16)
    B = np.zeros((0, N), np.uint16)
    log(f"case epilogue K=0 out={out}")
    got = host(epi(A, B, out_bf16, bias, res, gelu=True))
    got = oracle.widen(got) if out_bf16 else got.astype(np.float64)
    E = oracle.epilogue(np.zeros((M, N)), bias, res, use_gelu=True)
    tol = 3e-7 * np.maximum(1.0, np.abs(E)) + (2.0 ** -8 * np.abs(E) if out_bf16 else 0.0)
    assert np.all(np.abs(got - E) <= tol)


@pytest.mark.parametrize("shape", [(16, 1024, 2048), (300, 520, 136), (512, 512, 512)])
def test_no_epilogue_terms_equal_the_plain_product(shape):
    M, N, K = shape
    rng = np.random.default_rng(8)
    A = inputs.normal_bf16(rng, (M, K), 1.0)
    B = inputs.normal_bf16(rng, (K, N), 1.0)
    for p in paths_for(M, N, K):
        if p == P.AUTO:
            continue
        log(f"case epilogue none {shape} path={p.name}")
        plain = run("bf16", to_device(A), to_device(B), p)
        torch.cuda.synchronize()
        assert np.array_equal(host(epi(A, B, False, path=p)), plain.cpu().numpy()), p.name


def test_full_size_mlp_gelu_workload():
    """The benchmark's fused workload (8192 x 14336 x 4096, + bias, GELU, bf16
    out) in the launch configuration bench.py times: 64 sampled 32 x 32
    tiles and the four corners against the oracle, one by one."""
    w = inputs.WORKLOADS["bf16_mlp_gelu"]
    log(f"case workload {w.name} {w.M}x{w.N}x{w.K}")
    A, B = inputs.make_inputs(w)
    bias = inputs.make_bias(w)
    got = oracle.widen(host(epi(A, B, True, bias, gelu=True)))
    tiles = sorted(set(inputs.sample_tiles(w.M, w.N)) |
                   {(0, 0), (0, w.N - 32), (w.M - 32, 0), (w.M - 32, w.N - 32)})
    R = oracle.gemm_tiles(A, B, tiles, 32)
    S = oracle.gemm_tiles(A & 0x7FFF, B & 0x7FFF, tiles, 32)
    worst = 0.0
    num = den = 0.0
    for (r, c), Rt, St in zip(tiles, R, S):
        b = bias[c:c + 32]
        E = oracle.epilogue(Rt, b, None, use_gelu=True)
        T = oracle.epilogue(Rt, b)
        err = np.abs(got[r:r + 32, c:c + 32] - E)
        worst = max(worst, float((err / bound(w.K, St, T, E, True)).max()))
        num += float((err ** 2).sum())
        den += float((E ** 2).sum())
    assert worst <= 1.0, worst
    rel = (num / den) ** 0.5
    assert rel <= 4e-3, rel
    log(f"  {w.name}: worst err/bound {worst:.3f}, rel_fro {rel:.3e}")

