"""B stored N x K (C = A @ B.T, a linear layer's weight) on every path (needs
an MI355X).

The oracle is gemm_nt (the stored matrix transposed into K x N order, then
the fp64 triple loop). Checks, as for the K x N layout: the parity bars on
random inputs, bit-exact integer inputs, the fused epilogue, run-to-run
determinism, and the full-size workloads on sampled tiles.
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

P, L = tdm.Path, tdm.Layout
PATHS = [P.AUTO, P.EDGE, P.MFMA, P.SKINNY]


def paths_for(M, N, K):
    return [p for p in PATHS
            if tdm.tdm_path_supports_ex(tdm.Kind.BF16_F32ACC, L.NK, p, M, N, K)]


def run_nk(A, Bt, path=P.AUTO, out_bf16=False, bias=None, residual=None, gelu=False):
    D = tdm.tdm_gemm_bf16_ex_path(
        to_device(A), to_device(Bt), L.NK, None,
        out_dtype=torch.bfloat16 if out_bf16 else torch.float32,
        bias=None if bias is None else to_device(bias),
        residual=None if residual is None else to_device(residual), gelu=gelu, path=path)
    torch.cuda.synchronize()
    if out_bf16:
        return D.view(torch.int16).cpu().numpy().view(np.uint16)
    return D.cpu().numpy()


# Shapes: ragged everywhere; for the small-M kernel (256 k per step, start
# staggered over the full steps) K below one step, K tails after several
# wrapped full steps, and N on both sides of its switch from one to two
# 16-row tiles per workgroup (8192).
SHAPES = [(1, 1, 8), (5, 7, 24), (16, 100, 1000), (3, 4096, 520), (16, 8192, 1024),
          (9, 9000, 256), (4, 8300, 2312), (2, 33, 4104), (130, 200, 136), (300, 520, 136),
          (512, 768, 1024), (17, 64, 4096)]


def _cases():
    for shape in SHAPES:
        for p in paths_for(*shape):
            yield pytest.param(shape, p, id=f"{shape[0]}x{shape[1]}x{shape[2]}-{p.name}")


@pytest.mark.parametrize("shape,path", list(_cases()))
def test_random_parity(shape, path):
    M, N, K = shape
    log(f"case nk random {shape} path={path.name}")
    rng = np.random.default_rng(M * 11 + N + 3 * K)
    A = inputs.normal_bf16(rng, (M, K), 1.0)
    Bt = inputs.normal_bf16(rng, (N, K), 1.0)
    C = run_nk(A, Bt, path)
    R = oracle.gemm_nt(A, Bt)
    p = oracle.parity(C, R, max_abs(A), max_abs(Bt), K)
    assert p["norm_max_err"] <= TOL_BF16 and p["rel_fro"] <= TOL_FRO, (path.name, p)


@pytest.mark.parametrize("shape,path", list(_cases()))
def test_integer_inputs_bit_exact(shape, path):
    M, N, K = shape
    log(f"case nk integer {shape} path={path.name}")
    rng = np.random.default_rng(M + N * 7 + K)
    A = inputs.small_int_matrix(rng, (M, K), kind="bf16")
    Bt = inputs.small_int_matrix(rng, (N, K), kind="bf16")
    assert np.array_equal(run_nk(A, Bt, path).astype(np.float64), oracle.gemm_nt(A, Bt))


@pytest.mark.parametrize("shape", [(16, 1024, 2048), (300, 520, 136), (7, 40, 24)])
def test_fused_epilogue(shape):
    M, N, K = shape
    rng = np.random.default_rng(M + N + K + 1)
    A = inputs.normal_bf16(rng, (M, K), 1.0)
    Bt = inputs.normal_bf16(rng, (N, K), 0.02)
    bias = inputs.fp32_to_bf16_bits((rng.standard_normal(N) * 0.5).astype(np.float32))
    res = inputs.fp32_to_bf16_bits(rng.standard_normal((M, N)).astype(np.float32))
    R = oracle.gemm_nt(A, Bt)
    E = oracle.epilogue(R, bias, res, use_gelu=True)
    T = oracle.epilogue(R, bias)
    S = oracle.gemm_nt(A & 0x7FFF, Bt & 0x7FFF)
    tol = (1.13 * (K * 2.0 ** -24 * S + 2.0 ** -24 * np.abs(T)) + 3e-7 * np.maximum(1.0, np.abs(T))
           + 2.0 ** -23 * np.abs(E) + 2.0 ** -8 * np.abs(E))
    for p in paths_for(M, N, K):
        log(f"case nk epilogue {shape} path={p.name}")
        got = oracle.widen(run_nk(A, Bt, p, True, bias, res, True))
        assert np.all(np.abs(got - E) <= tol), (p.name, float((np.abs(got - E) / tol).max()))


@pytest.mark.parametrize("shape", [(16, 8192, 4096), (1000, 1000, 1000)])
def test_run_to_run_bitwise_determinism(shape):
    M, N, K = shape
    rng = np.random.default_rng(4)
    A = to_device(inputs.normal_bf16(rng, (M, K), 1.0))
    Bt = to_device(inputs.normal_bf16(rng, (N, K), 1.0))
    for p in paths_for(M, N, K):
        log(f"case nk determinism {shape} path={p.name}")
        ref = tdm.tdm_gemm_bf16_ex_path(A, Bt, L.NK, out_dtype=torch.float32, path=p).clone()
        for _ in range(100):
            again = tdm.tdm_gemm_bf16_ex_path(A, Bt, L.NK, out_dtype=torch.float32, path=p)
            assert torch.equal(again, ref), p.name


def _tiles(M, N):
    tiles = set(inputs.sample_tiles(M, N)) | {(0, 0), (0, N - 32), (M - 32, 0), (M - 32, N - 32)}
    return sorted((min(r, max(M - 32, 0)), c) for r, c in tiles)


def test_full_size_skinny_nk():
    """16 x 8192 x 8192 with the weight stored N x K: the whole product."""
    w = inputs.WORKLOADS["bf16_skinny_nk"]
    log(f"case workload {w.name} {w.M}x{w.N}x{w.K}")
    assert tdm.tdm_select_path_ex(tdm.Kind.BF16_F32ACC, L.NK, w.M, w.N, w.K) == P.SKINNY
    A, Bt = inputs.make_inputs(w)
    C = run_nk(A, Bt)
    p = oracle.parity(C, oracle.gemm_nt(A, Bt), max_abs(A), max_abs(Bt), w.K)
    assert p["norm_max_err"] <= TOL_BF16 and p["rel_fro"] <= TOL_FRO, p
    log(f"  {w.name}: norm_max_err={p['norm_max_err']:.3e} rel_fro={p['rel_fro']:.3e}")


def test_full_size_linear_gelu():
    """8192 x 14336 x 4096, weight N x K, + bias, GELU, bf16 out: sampled tiles."""
    w = inputs.WORKLOADS["bf16_linear_gelu"]
    log(f"case workload {w.name} {w.M}x{w.N}x{w.K}")
    A, Bt = inputs.make_inputs(w)
    bias = inputs.make_bias(w)
    got = oracle.widen(run_nk(A, Bt, P.AUTO, True, bias, None, True))
    tiles = _tiles(w.M, w.N)
    R = oracle.gemm_nt_tiles(A, Bt, tiles)
    S = oracle.gemm_nt_tiles(A & 0x7FFF, Bt & 0x7FFF, tiles)
    worst = 0.0
    for (r, c), Rt, St in zip(tiles, R, S):
        b = bias[c:c + 32]
        E = oracle.epilogue(Rt, b, None, use_gelu=True)
        T = oracle.epilogue(Rt, b)
        tol = (1.13 * (w.K * 2.0 ** -24 * St + 2.0 ** -24 * np.abs(T))
               + 3e-7 * np.maximum(1.0, np.abs(T)) + 2.0 ** -23 * np.abs(E) + 2.0 ** -8 * np.abs(E))
        worst = max(worst, float((np.abs(got[r:r + 32, c:c + 32] - E) / tol).max()))
    assert worst <= 1.0, worst
    log(f"  {w.name}: worst err/bound {worst:.3f}")


@pytest.mark.parametrize("shape", [(4000, 3900, 200), (5000, 4600, 200), (5000, 4600, 4096)])
def test_large_tiles_in_one_round_and_in_several(shape):
    """256 x 256 tiles with B stored N x K: 4000 x 3900 fills exactly one
    round of the CUs, 5000 x 4600 two rounds; partial tiles in M and N, and
    a partial last K step (K = 200: the interleaved loop) or none (K = 4096:
    the ping-pong schedule)."""
    M, N, K = shape
    log(f"case nk large tiles {shape}")
    rng = np.random.default_rng(M + N + K + 7)
    A = inputs.small_int_matrix(rng, (M, K), kind="bf16")
    Bt = inputs.small_int_matrix(rng, (N, K), kind="bf16")
    if K <= 256:
        assert np.array_equal(run_nk(A, Bt, P.MFMA).astype(np.float64), oracle.gemm_nt(A, Bt))
    else:  # sampled tiles keep the oracle's share to seconds
        got = run_nk(A, Bt, P.MFMA)
        tiles = _tiles(M, N)
        for (r, c), Rt in zip(tiles, oracle.gemm_nt_tiles(A, Bt, tiles)):
            assert np.array_equal(got[r:r + 32, c:c + 32].astype(np.float64), Rt), (r, c)
    A = inputs.normal_bf16(rng, (M, K), 1.0)
    Bt = inputs.normal_bf16(rng, (N, K), 1.0)
    if K <= 256:
        p = oracle.parity(run_nk(A, Bt, P.MFMA), oracle.gemm_nt(A, Bt), max_abs(A), max_abs(Bt), K)
        assert p["norm_max_err"] <= TOL_BF16 and p["rel_fro"] <= TOL_FRO, p
