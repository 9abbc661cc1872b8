"""The allocation-free entry point gemm_bf16_ex_noalloc (needs an MI355X).

It runs gemm_bf16_ex's kernels with the small-M K x N partial sums in the
library's one static buffer per GPU. Two calls in a row through the C ABI,
the second smaller (so the buffer holds the first call's partial sums when
the second runs), each compared bit for bit with gemm_bf16_ex on the same
inputs and with the fp64 oracle to the bf16 bars.
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


def _case(rng, M, N, K, bias):
    A = inputs.normal_bf16(rng, (M, K), 1.0)
    B = inputs.normal_bf16(rng, (K, N), 0.02)
    b = inputs.normal_bf16(rng, (N,), 0.5) if bias else None
    return A, B, b


def test_two_calls_in_a_row_match_gemm_bf16_ex():
    rng = np.random.default_rng(2024)
    # the small-M path with K split over workgroups, then a smaller product
    # of the same path with the epilogue (bias, GELU, bf16 output)
    cases = [(16, 8192, 8192, False, torch.float32), (7, 1024, 3000, True, torch.bfloat16)]
    assert all(tdm.tdm_select_path(tdm.Kind.BF16_F32ACC, M, N, K) == tdm.Path.SKINNY
               for M, N, K, _, _ in cases)
    ins = [_case(rng, M, N, K, bias) for M, N, K, bias, _ in cases]
    dev = [(to_device(A), to_device(B), None if b is None else to_device(b)) for A, B, b in ins]
    outs = [torch.empty((M, N), dtype=dt, device="cuda") for M, N, _, _, dt in cases]
    torch.cuda.synchronize()
    for (M, N, K, bias, dt), (Ad, Bd, bd), D in zip(cases, dev, outs):
        log(f"case no-alloc {M}x{N}x{K} bias={bias} out={dt}")
        tdm.gemm_bf16_ex_noalloc(Ad, Bd, tdm.Layout.KN, D=D, bias=bd, gelu=bias)
    torch.cuda.synchronize()
    for (M, N, K, bias, dt), (A, B, b), (Ad, Bd, bd), D in zip(cases, ins, dev, outs):
        ref = tdm.gemm_bf16_ex(Ad, Bd, tdm.Layout.KN, out_dtype=dt, bias=bd, gelu=bias)
        torch.cuda.synchronize()
        assert torch.equal(D.view(torch.int16) if dt == torch.bfloat16 else D,
                           ref.view(torch.int16) if dt == torch.bfloat16 else ref)
        R = oracle.gemm(A, B)
        if bias:
            E = oracle.epilogue(R, b, None, use_gelu=True)
            got = oracle.widen(D.view(torch.int16).cpu().numpy().view(np.uint16))
            rel = float(np.linalg.norm(got - E) / np.linalg.norm(E))
            assert rel <= 2.0 ** -8, rel  # the bf16 output's rounding
        else:
            p = oracle.parity(D.cpu().numpy(), R, max_abs(A), max_abs(B), K)
            assert p["norm_max_err"] <= TOL_BF16 and p["rel_fro"] <= TOL_FRO, p
