"""Every workload shape, on the path its benchmark line times, against the
oracle over the whole output (needs an MI355X).

The definition is C[i,j] = sum_k A[i,k] B[k,j] ("09 计算受限还是访存受限",
counting a matrix multiply; CS336 Lecture 5 GPU notes, §4.2). Two input
kinds per shape:

  * integers in {-3..3} (inputs.make_integer_inputs): every partial sum is
    an integer of magnitude at most 9K <= 73,728 < 2^24, exact in fp32 under
    any summation order, so every element must equal the oracle's bit for
    bit -- including the tile edges, the last tile and every tile a sampled
    check would miss;
  * the workload's own seeded random inputs: the normalized max error
    max|C - R| / (max|A| max|B| K) within 1e-5 (fp32) or 4e-3 (bf16) and the
    relative Frobenius error within 1e-5, over every element.

The products run through the C ABI with the same entry point, path and
launch configuration (tile size, grid, stagger) that bench.py times for the
workload: the tile choice depends only on M and N, so one call here runs
exactly the kernel the benchmark runs.
"""
import numpy as np
import pytest

import oracle
import tiled_dense_matrix_amd as tdm
from tiled_dense_matrix_amd import inputs

from helpers import TOL_BF16, TOL_F32, TOL_FRO, log, max_abs, run, to_device

torch = pytest.importorskip("torch")

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

P = tdm.Path

# (workload, path) as bench.py runs them: the square fp32 4096 product on
# the vector-ALU kernel (its line's main measurement) and on the library's
# own choice; everything else on the library's own choice.
CASES = [
    ("f32_256", P.AUTO), ("f32_256", P.VALU),
    ("f32_4096", P.VALU), ("f32_4096", P.AUTO),
    ("bf16_4096", P.AUTO), ("bf16_8192", P.AUTO), ("bf16_mlp", P.AUTO),
    ("bf16_skinny", P.AUTO), ("bf16_skinny_nk", P.AUTO),
    # the linear layer's shape with B stored N x K, plain fp32 output
    ("bf16_linear_gelu", P.AUTO),
    # the fp32 4096^3 product with B stored N x K, and with A stored K x M
    ("f32_4096_nk", P.AUTO), ("f32_4096_tn", P.AUTO),
]


def _layout(w):
    return tdm.Layout((tdm.Layout.NK if w.b_layout == "nk" else 0)
                      | (tdm.Layout.KM_KN if w.a_layout == "km" else 0))


def _ids():
    return [f"{name}-{path.name}" for name, path in CASES]


def product(w, A, B, path):
    """The GPU product of (A, B) for workload w through the C ABI, fp32."""
    Ad, Bd = to_device(A), to_device(B)
    layout = _layout(w)
    if layout != tdm.Layout.KN and w.kind == "f32":
        C = tdm.tdm_gemm_f32_ex_path(Ad, Bd, layout, path=path)
    elif layout != tdm.Layout.KN:
        C = tdm.tdm_gemm_bf16_ex_path(Ad, Bd, layout, out_dtype=torch.float32, path=path)
    else:
        C = run(w.kind, Ad, Bd, path)
    torch.cuda.synchronize()
    out = C.cpu().numpy()
    del Ad, Bd, C
    torch.cuda.empty_cache()
    return out


def reference(w, A, B):
    """The oracle's fp64 product (A and B in their stored layouts)."""
    if w.a_layout == "km":
        return oracle.gemm_tn(A, B) if w.b_layout == "kn" else \
            oracle.gemm(np.ascontiguousarray(A.T), np.ascontiguousarray(B.T))
    return oracle.gemm_nt(A, B) if w.b_layout == "nk" else oracle.gemm(A, B)


def path_taken(w, path):
    kind = tdm.Kind.F32 if w.kind == "f32" else tdm.Kind.BF16_F32ACC
    return path if path != P.AUTO else tdm.tdm_select_path_ex(kind, _layout(w), w.M, w.N, w.K)


@pytest.mark.parametrize("name,path", CASES, ids=_ids())
def test_integer_inputs_bit_exact_over_the_whole_output(name, path):
    w = inputs.WORKLOADS[name]
    taken = tdm.path_name(path_taken(w, path))
    log(f"case config-shape integer {name} {w.M}x{w.N}x{w.K} b={w.b_layout} "
        f"path={path.name} ({taken})")
    A, B = inputs.make_integer_inputs(w)
    C = product(w, A, B, path)
    R = reference(w, A, B)
    assert float(np.abs(R).max()) <= 9 * w.K < 2 ** 24  # every partial sum exact in fp32
    bad = np.argwhere(C.astype(np.float64) != R)
    assert bad.size == 0, (name, taken, len(bad), bad[:5].tolist())
    log(f"  {name} ({taken}): all {w.M * w.N} elements bit-exact")


@pytest.mark.parametrize("name,path", CASES, ids=_ids())
def test_random_inputs_over_the_whole_output(name, path):
    w = inputs.WORKLOADS[name]
    taken = tdm.path_name(path_taken(w, path))
    log(f"case config-shape random {name} {w.M}x{w.N}x{w.K} b={w.b_layout} "
        f"path={path.name} ({taken})")
    A, B = inputs.make_inputs(w)
    C = product(w, A, B, path)
    R = reference(w, A, B)
    p = oracle.parity(C, R, max_abs(A), max_abs(B), w.K)
    tol = TOL_F32 if w.kind == "f32" else TOL_BF16
    assert p["norm_max_err"] <= tol, (name, taken, p)
    assert p["rel_fro"] <= TOL_FRO, (name, taken, p)
    log(f"  {name} ({taken}): norm_max_err={p['norm_max_err']:.3e} "
        f"rel_fro={p['rel_fro']:.3e} max_abs_err={p['max_abs_err']:.3e}")
