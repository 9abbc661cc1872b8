"""Non-finite inputs on every path (needs an MI355X).

The product is defined element by element as a sum of products, so IEEE
special values travel through it: a NaN in A[i, k] makes row i of C NaN, an
infinity gives a signed infinity (or NaN where it meets a zero or an infinity
of the other sign). Every path must put NaN and +-Inf exactly where the fp64
oracle does, and match it within the parity bar everywhere else. Padding and
clamped loads in partial tiles must not leak special values into outputs that
the definition keeps finite.
"""
import numpy as np
import pytest

import oracle
import tiled_dense_matrix_amd as tdm
from tiled_dense_matrix_amd import inputs

from helpers import TOL_BF16, TOL_F32, log, run, to_device

torch = pytest.importorskip("torch")

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

P = tdm.Path
KIND = {"f32": tdm.Kind.F32, "bf16": tdm.Kind.BF16_F32ACC}
PATHS = [P.AUTO, P.EDGE, P.VALU, P.MFMA, P.SKINNY]
SHAPES = [("f32", (130, 200, 136)), ("f32", (300, 520, 96)), ("bf16", (130, 200, 136)),
          ("bf16", (300, 520, 96)), ("bf16", (16, 512, 1024))]


def planted_inputs(kind, M, N, K, seed):
    """Seeded inputs with NaN and +-Inf planted in A and B (and zeros next to
    them, for Inf * 0)."""
    rng = np.random.default_rng(seed)
    A = inputs.uniform_fp32(rng, (M, K))
    B = inputs.uniform_fp32(rng, (K, N))
    A[1, 3] = np.nan                  # row 1 of C: NaN
    A[M - 1, K - 1] = np.inf          # last row: +-Inf by the sign of B[K-1, j]
    B[K - 1, N // 2] = 0.0            # ... and NaN (Inf * 0) in one column
    B[K // 2, N - 1] = -np.inf        # last column: -+Inf by the sign of A[i, K/2]
    A[M // 2, K // 2] = 0.0           # ... and NaN (0 * Inf) in one row
    if kind == "bf16":
        return inputs.fp32_to_bf16_bits(A), inputs.fp32_to_bf16_bits(B)
    return A, B


def _cases():
    for kind, shape in SHAPES:
        for p in PATHS:
            if tdm.tdm_path_supports(KIND[kind], p, *shape):
                yield pytest.param(kind, shape, p, id=f"{kind}-{shape[0]}x{shape[1]}x{shape[2]}-{p.name}")


@pytest.mark.parametrize("kind,shape,path", list(_cases()))
def test_special_values_land_where_the_definition_puts_them(kind, shape, path):
    M, N, K = shape
    log(f"case special values {kind} {shape} path={path.name}")
    A, B = planted_inputs(kind, M, N, K, seed=M + N + K)
    C = run(kind, to_device(A), to_device(B), path)
    torch.cuda.synchronize()
    C = C.cpu().numpy().astype(np.float64)
    R = oracle.gemm(A, B)
    assert np.isnan(R).any() and np.isinf(R).any()  # the planting worked
    assert np.array_equal(np.isnan(C), np.isnan(R)), path.name
    assert np.array_equal(np.isposinf(C), np.isposinf(R)), path.name
    assert np.array_equal(np.isneginf(C), np.isneginf(R)), path.name
    fin = np.isfinite(R)
    Aw, Bw = oracle.widen(A), oracle.widen(B)
    ma = float(np.abs(Aw[np.isfinite(Aw)]).max())
    mb = float(np.abs(Bw[np.isfinite(Bw)]).max())
    err = float(np.abs(C[fin] - R[fin]).max()) / (ma * mb * K)
    assert err <= (TOL_F32 if kind == "f32" else TOL_BF16), (path.name, err)


L = tdm.Layout
LAYOUT_SHAPES = [("f32", (132, 200, 136)), ("f32", (300, 520, 96)), ("bf16", (136, 200, 136)),
                 ("bf16", (304, 520, 96)), ("bf16", (16, 512, 1024))]


def _layout_cases():
    for kind, shape in LAYOUT_SHAPES:
        for layout in (L.NK, L.KM_KN, L.KM_NK):
            for p in (P.AUTO, P.EDGE, P.MFMA, P.SKINNY):
                if tdm.tdm_path_supports_ex(KIND[kind], layout, p, *shape):
                    yield pytest.param(kind, shape, layout, p,
                                       id=f"{kind}-{layout.name}-{shape[0]}x{shape[1]}x{shape[2]}"
                                          f"-{p.name}")


@pytest.mark.parametrize("kind,shape,layout,path", list(_layout_cases()))
def test_special_values_with_a_transposed_operand(kind, shape, layout, path):
    """The same planted values in op(A) and op(B), stored transposed as the
    layout says (A K x M, B N x K): they must land where the definition
    applied to op(A) and op(B) puts them."""
    M, N, K = shape
    log(f"case special values {kind} {layout.name} {shape} path={path.name}")
    A, B = planted_inputs(kind, M, N, K, seed=M + 2 * N + K)
    As = np.ascontiguousarray(A.T) if layout & L.KM_KN else A
    Bs = np.ascontiguousarray(B.T) if layout & L.NK else B
    if kind == "f32":
        C = tdm.tdm_gemm_f32_ex_path(to_device(As), to_device(Bs), layout, path=path)
    else:
        C = tdm.tdm_gemm_bf16_ex_path(to_device(As), to_device(Bs), layout,
                                      out_dtype=torch.float32, path=path)
    torch.cuda.synchronize()
    C = C.cpu().numpy().astype(np.float64)
    R = oracle.gemm(A, B)
    assert np.isnan(R).any() and np.isinf(R).any()
    assert np.array_equal(np.isnan(C), np.isnan(R)), path.name
    assert np.array_equal(np.isposinf(C), np.isposinf(R)), path.name
    assert np.array_equal(np.isneginf(C), np.isneginf(R)), path.name
    fin = np.isfinite(R)
    Aw, Bw = oracle.widen(A), oracle.widen(B)
    ma = float(np.abs(Aw[np.isfinite(Aw)]).max())
    mb = float(np.abs(Bw[np.isfinite(Bw)]).max())
    err = float(np.abs(C[fin] - R[fin]).max()) / (ma * mb * K)
    assert err <= (TOL_F32 if kind == "f32" else TOL_BF16), (path.name, err)
