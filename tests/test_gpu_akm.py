"""The product with A stored K x M, C = A^T op(B) for the stored matrix (needs
an MI355X).

The pages' own transposed-operand case, x = A.T @ B (CS336 Lecture 5 GPU
notes, review question 5; §4.1: a transpose is another memory layout). The
matrix-core kernel stages such an A k-major in LDS and reads its fragments
with transposing LDS reads; the edge kernel loads it with swapped indices.
Every case calls gemm_bf16_ex / tdm_gemm_bf16_ex_path through the C ABI and
compares with oracle.gemm_tn (or the oracle's product of the transposed
copies when B is N x K as well):
  * random bf16 inputs: normalized max error <= 4e-3 and relative Frobenius
    error <= 1e-5 over the whole output;
  * integers in {-3..3}: bit for bit (every partial sum exact in fp32);
  * the fused epilogue, determinism, small M (no streaming path for this
    layout) and the full 8192^3 workload over every element.
"""
import numpy as np
import pytest

import oracle
import tiled_dense_matrix_amd as tdm
from tiled_dense_matrix_amd import inputs

from helpers import TOL_BF16, TOL_FRO, log, max_abs, to_device

torch = pytest.importorskip("torch")

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

P = tdm.Path
L = tdm.Layout


def stored(rng, M, N, K, layout, maker):
    """A (K x M) and B (K x N, or N x K) drawn by maker(rng, shape)."""
    A = maker(rng, (K, M))
    B = maker(rng, (N, K) if layout & L.NK else (K, N))
    return A, B


def normal(sig):
    return lambda rng, shape: inputs.normal_bf16(rng, shape, sig)


def integers(rng, shape):
    return inputs.small_int_matrix(rng, shape, kind="bf16")


def reference(A, B, layout):
    if layout & L.NK:
        return oracle.gemm(np.ascontiguousarray(A.T), np.ascontiguousarray(B.T))
    return oracle.gemm_tn(A, B)


def product(A, B, layout, path=P.AUTO, **epi):
    D = tdm.tdm_gemm_bf16_ex_path(to_device(A), to_device(B), layout,
                                  out_dtype=epi.pop("out_dtype", torch.float32), path=path, **epi)
    torch.cuda.synchronize()
    if D.dtype == torch.bfloat16:
        return oracle.widen(D.view(torch.int16).cpu().numpy().view(np.uint16))
    return D.cpu().numpy()


SHAPES = [(8, 8, 8), (8, 40, 24), (64, 64, 64), (96, 200, 48), (264, 257, 136),
          (256, 264, 520), (520, 512, 72), (1000, 24, 4104), (16, 1024, 2048),
          (33, 65, 17), (5, 7, 3)]


def _cases():
    for layout in (L.KM_KN, L.KM_NK):
        for M, N, K in SHAPES:
            for p in (P.AUTO, P.EDGE, P.MFMA, P.SKINNY):
                if tdm.tdm_path_supports_ex(tdm.Kind.BF16_F32ACC, layout, p, M, N, K):
                    yield pytest.param(layout, (M, N, K), p,
                                       id=f"{layout.name}-{M}x{N}x{K}-{p.name}")


@pytest.mark.parametrize("layout,shape,path", list(_cases()))
def test_random_parity(layout, shape, path):
    M, N, K = shape
    log(f"case A K x M random {layout.name} {shape} path={path.name}")
    A, B = stored(np.random.default_rng(M + 3 * N + 7 * K + int(layout)), M, N, K, layout,
                  normal(1.0))
    C = product(A, B, layout, path)
    R = reference(A, B, layout)
    p = oracle.parity(C, R, max_abs(A), max_abs(B), K)
    assert p["norm_max_err"] <= TOL_BF16 and p["rel_fro"] <= TOL_FRO, p


@pytest.mark.parametrize("layout,shape,path", list(_cases()))
def test_integer_inputs_bit_exact(layout, shape, path):
    M, N, K = shape
    log(f"case A K x M integer {layout.name} {shape} path={path.name}")
    A, B = stored(np.random.default_rng(11 + M + N + K + int(layout)), M, N, K, layout, integers)
    assert np.array_equal(product(A, B, layout, path).astype(np.float64), reference(A, B, layout))


@pytest.mark.parametrize("layout", [L.KM_KN, L.KM_NK])
def test_large_tiles_with_partial_tiles(layout):
    """3600 x 3000 runs on 256 x 256 tiles with partial tiles in M and N and
    K = 200 (a partial K step)."""
    M, N, K = 3600, 3000, 200
    log(f"case A K x M large tiles {layout.name}")
    rng = np.random.default_rng(40 + int(layout))
    A, B = stored(rng, M, N, K, layout, integers)
    assert np.array_equal(product(A, B, layout, P.MFMA).astype(np.float64),
                          reference(A, B, layout))
    A, B = stored(rng, M, N, K, layout, normal(1.0))
    p = oracle.parity(product(A, B, layout, P.MFMA), reference(A, B, layout), max_abs(A),
                      max_abs(B), K)
    assert p["norm_max_err"] <= TOL_BF16 and p["rel_fro"] <= TOL_FRO, p


@pytest.mark.parametrize("path", [P.MFMA, P.EDGE])
def test_fused_epilogue_exact(path):
    """Integers with an integer bias and residual, bf16 output: the outputs
    are integers, rounded to bf16 exactly as the oracle rounds them."""
    M, N, K = 264, 136, 320
    rng = np.random.default_rng(51)
    A, B = stored(rng, M, N, K, L.KM_KN, integers)
    bias = inputs.small_int_matrix(rng, (N,), kind="bf16")
    res = inputs.small_int_matrix(rng, (M, N), -50, 50, kind="bf16")
    log(f"case A K x M epilogue path={path.name}")
    got = product(A, B, L.KM_KN, path, out_dtype=torch.bfloat16, bias=to_device(bias),
                  residual=to_device(res))
    want = oracle.widen(oracle.round_to_bf16(oracle.epilogue(oracle.gemm_tn(A, B), bias, res)))
    assert np.array_equal(got, want)


def test_run_to_run_bitwise_determinism():
    M, N, K = 1024, 1024, 1024
    log("case A K x M determinism")
    A, B = stored(np.random.default_rng(52), M, N, K, L.KM_KN, normal(1.0))
    Ad, Bd = to_device(A), to_device(B)
    for p in (P.MFMA, P.EDGE):
        ref = tdm.tdm_gemm_bf16_ex_path(Ad, Bd, L.KM_KN, out_dtype=torch.float32, path=p).clone()
        for _ in range(100):
            again = tdm.tdm_gemm_bf16_ex_path(Ad, Bd, L.KM_KN, out_dtype=torch.float32, path=p)
            assert torch.equal(again, ref), p.name


@pytest.mark.parametrize("kind", ["integer", "random"])
def test_full_size_workload_over_the_whole_output(kind):
    """bf16_8192_tn (8192^3, A stored K x M) through gemm_bf16_ex as bench.py
    runs it, every element against the oracle."""
    w = inputs.WORKLOADS["bf16_8192_tn"]
    log(f"case workload {w.name} {kind}")
    A, B = inputs.make_integer_inputs(w) if kind == "integer" else inputs.make_inputs(w)
    assert A.shape == (w.K, w.M)
    C = product(A, B, L.KM_KN)
    R = oracle.gemm_tn(A, B)
    if kind == "integer":
        assert np.array_equal(C.astype(np.float64), R)
    else:
        p = oracle.parity(C, R, max_abs(A), max_abs(B), w.K)
        assert p["norm_max_err"] <= TOL_BF16 and p["rel_fro"] <= TOL_FRO, p
        log(f"  {w.name}: {p}")
