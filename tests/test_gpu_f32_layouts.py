"""The fp32 product with a transposed operand (needs an MI355X).

C = op(A) op(B) with B stored N x K (op(B) = B^T) and/or A stored K x M
(op(A) = A^T), through gemm_f32_ex / tdm_gemm_f32_ex_path (CS336 Lecture 5
GPU notes, review question 5 on x = A.T @ B and the §4.1 warning: a
transposed operand is another memory layout). The fp32 matrix-core kernel
stages an N x K B like A and a K x M A like B; the edge kernel loads either
with swapped indices. Every case is compared with the oracle's product of
the same stored matrices (oracle.gemm_nt, oracle.gemm_tn, or oracle.gemm of
both transposes):
  * uniform fp32 inputs: normalized max error <= 1e-5 and relative Frobenius
    error <= 1e-5 over the whole output;
  * integers in {-3..3}: bit for bit (every partial sum exact in fp32);
  * large tiles with partial tiles and a partial K step, determinism, and
    4096^3 in every layout over every element.
"""
import numpy as np
import pytest

import oracle
import tiled_dense_matrix_amd as tdm
from tiled_dense_matrix_amd import inputs

from helpers import TOL_F32, TOL_FRO, log, max_abs, to_device

torch = pytest.importorskip("torch")

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

P = tdm.Path
L = tdm.Layout
LAYOUTS = (L.NK, L.KM_KN, L.KM_NK)


def stored(rng, M, N, K, layout, maker):
    """A (K x M when A is transposed, else M x K) and B (N x K or K x N)."""
    A = maker(rng, (K, M) if layout & L.KM_KN else (M, K))
    B = maker(rng, (N, K) if layout & L.NK else (K, N))
    return A, B


def uniform(rng, shape):
    return inputs.uniform_fp32(rng, shape)


def integers(rng, shape):
    return inputs.small_int_matrix(rng, shape, kind="f32")


def reference(A, B, layout):
    """The oracle's product of op(A) and op(B)."""
    if layout == L.NK:
        return oracle.gemm_nt(A, B)
    if layout == L.KM_KN:
        return oracle.gemm_tn(A, B)
    if layout == L.KM_NK:
        return oracle.gemm(np.ascontiguousarray(A.T), np.ascontiguousarray(B.T))
    return oracle.gemm(A, B)


def product(A, B, layout, path=P.AUTO):
    C = tdm.tdm_gemm_f32_ex_path(to_device(A), to_device(B), layout, path=path)
    torch.cuda.synchronize()
    return C.cpu().numpy()


SHAPES = [(4, 4, 4), (8, 40, 24), (64, 64, 64), (96, 200, 48), (264, 260, 136),
          (256, 264, 520), (520, 512, 72), (1000, 24, 4104), (16, 1024, 2048),
          (33, 65, 17), (5, 7, 3), (128, 132, 36)]


def _cases():
    for layout in LAYOUTS:
        for M, N, K in SHAPES:
            for p in (P.AUTO, P.EDGE, P.MFMA):
                if tdm.tdm_path_supports_ex(tdm.Kind.F32, layout, p, M, N, K):
                    yield pytest.param(layout, (M, N, K), p,
                                       id=f"{layout.name}-{M}x{N}x{K}-{p.name}")


@pytest.mark.parametrize("layout,shape,path", list(_cases()))
def test_random_parity(layout, shape, path):
    M, N, K = shape
    log(f"case f32 layout random {layout.name} {shape} path={path.name}")
    A, B = stored(np.random.default_rng(M + 3 * N + 7 * K + int(layout)), M, N, K, layout, uniform)
    p = oracle.parity(product(A, B, layout, path), reference(A, B, layout), max_abs(A),
                      max_abs(B), K)
    assert p["norm_max_err"] <= TOL_F32 and p["rel_fro"] <= TOL_FRO, p


@pytest.mark.parametrize("layout,shape,path", list(_cases()))
def test_integer_inputs_bit_exact(layout, shape, path):
    M, N, K = shape
    log(f"case f32 layout integer {layout.name} {shape} path={path.name}")
    A, B = stored(np.random.default_rng(17 + M + N + K + int(layout)), M, N, K, layout, integers)
    assert np.array_equal(product(A, B, layout, path).astype(np.float64), reference(A, B, layout))


def test_layout_kn_through_the_new_entry_point_matches_gemm_f32():
    """TDM_LAYOUT_KN through gemm_f32_ex is gemm_f32, bit for bit, on every
    path that takes the shape."""
    M, N, K = 300, 264, 200
    rng = np.random.default_rng(90)
    A, B = uniform(rng, (M, K)), uniform(rng, (K, N))
    Ad, Bd = to_device(A), to_device(B)
    for p in (P.AUTO, P.EDGE, P.MFMA, P.VALU):
        if not tdm.tdm_path_supports_ex(tdm.Kind.F32, L.KN, p, M, N, K):
            continue
        log(f"case f32 layout KN vs gemm_f32 path={p.name}")
        got = tdm.tdm_gemm_f32_ex_path(Ad, Bd, L.KN, path=p)
        want = tdm.tdm_gemm_f32_path(Ad, Bd, path=p)
        torch.cuda.synchronize()
        assert torch.equal(got, want), p.name


@pytest.mark.parametrize("layout", LAYOUTS)
def test_large_tiles_with_partial_tiles(layout):
    """4000 x 3900 runs on 256 x 256 tiles (16 x 16 of them fill the CUs)
    with partial tiles in M and N (the sizes keep K x M and K x N rows
    multiples of 4) and K = 200 (a partial K step)."""
    M, N, K = 4000, 3900, 200
    log(f"case f32 layout large tiles {layout.name}")
    rng = np.random.default_rng(41 + int(layout))
    A, B = stored(rng, M, N, K, layout, integers)
    assert np.array_equal(product(A, B, layout, P.MFMA).astype(np.float64),
                          reference(A, B, layout))
    A, B = stored(rng, M, N, K, layout, uniform)
    p = oracle.parity(product(A, B, layout, P.MFMA), reference(A, B, layout), max_abs(A),
                      max_abs(B), K)
    assert p["norm_max_err"] <= TOL_F32 and p["rel_fro"] <= TOL_FRO, p


def test_run_to_run_bitwise_determinism():
    M, N, K = 1024, 1024, 1024
    log("case f32 layout determinism")
    for layout in LAYOUTS:
        A, B = stored(np.random.default_rng(53 + int(layout)), M, N, K, layout, uniform)
        Ad, Bd = to_device(A), to_device(B)
        for p in (P.MFMA, P.EDGE):
            ref = tdm.tdm_gemm_f32_ex_path(Ad, Bd, layout, path=p).clone()
            for _ in range(100):
                again = tdm.tdm_gemm_f32_ex_path(Ad, Bd, layout, path=p)
                assert torch.equal(again, ref), (layout.name, p.name)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("kind", ["integer", "uniform"])
def test_4096_cubed_over_the_whole_output(layout, kind):
    """The fp32 4096^3 product (the f32_4096 workload's size) in each
    transposed layout, through gemm_f32_ex on the path the library chooses
    (the matrix cores), every element against the oracle."""
    M = N = K = 4096
    log(f"case f32 layout 4096^3 {layout.name} {kind}")
    rng = np.random.default_rng(60 + int(layout) + (0 if kind == "integer" else 10))
    A, B = stored(rng, M, N, K, layout, integers if kind == "integer" else uniform)
    assert tdm.tdm_select_path_ex(tdm.Kind.F32, layout, M, N, K) == P.MFMA
    C = tdm.gemm_f32_ex(to_device(A), to_device(B), layout)
    torch.cuda.synchronize()
    C = C.cpu().numpy()
    R = reference(A, B, layout)
    if kind == "integer":
        assert np.array_equal(C.astype(np.float64), R)
    else:
        p = oracle.parity(C, R, max_abs(A), max_abs(B), K)
        assert p["norm_max_err"] <= TOL_F32 and p["rel_fro"] <= TOL_FRO, p
        log(f"  {layout.name}: {p}")
