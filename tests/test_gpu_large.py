"""Near the size limit: matrices just below 2^31 elements (needs an MI355X).

The library indexes each matrix with 32-bit element counts (and the
matrix-core kernels' copies with 32-bit byte offsets per lane), so the largest
legal operands are where an overflow would show. Inputs are small integers, so
every partial sum is exact in fp32 and sampled tiles must match the oracle
bit for bit; the tiles include the last rows and columns, which sit at the
largest offsets.
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


def small_ints(rng, shape, kind):
    """Values in {-2..2} as fp32 or bf16 bits, without a float64 temporary."""
    values = np.array([-2, -1, 0, 1, 2], dtype=np.float32)
    if kind == "bf16":
        values = inputs.fp32_to_bf16_bits(values)
    return values[rng.integers(0, 5, size=shape, dtype=np.uint8)]


def corner_tiles(M, N, tile=32):
    rows = sorted({0, (M // 2) // tile * tile, max(M - tile, 0)})
    cols = sorted({0, max(N - tile, 0)})
    return [(r, c) for r in rows for c in cols]


@pytest.mark.parametrize("kind,shape,path", [
    ("bf16", (65536, 256, 32760), P.AUTO),    # M*K = 2^31 - 2^19: matrix cores
    ("f32", (65536, 128, 32764), P.AUTO),     # M*K = 2^31 - 2^18: fp32 matrix cores
    ("bf16", (16, 262136, 8184), P.AUTO),     # K*N just below 2^31: streaming path
    ("f32", (65536, 128, 32764), P.VALU),
    ("f32", (65536, 128, 32764), P.EDGE),
    ("bf16", (65536, 256, 32760), P.EDGE),
    # The fp32 matrix-core kernel copies with 32-bit byte offsets from the
    # tile's first row: 32 rows of B reach 31*N*4 bytes, just below 2^32 here,
    # and K just below 2^22 is the longest it takes.
    ("f32", (32, (1 << 25) - 4, 32), P.MFMA),
    ("f32", (32, (1 << 25) - 4, 32), P.VALU),
    ("f32", (256, 128, (1 << 22) - 4), P.MFMA),
])
def test_operands_just_below_two_to_the_31(kind, shape, path):
    M, N, K = shape
    log(f"case near-max {kind} {shape} path={path.name} "
        f"(selected {tdm.tdm_select_path(tdm.Kind.F32 if kind == 'f32' else tdm.Kind.BF16_F32ACC, M, N, K).name})")
    assert max(M * K, K * N, M * N) < 2 ** 31
    rng = np.random.default_rng(M + N + K)
    A = small_ints(rng, (M, K), kind)
    B = small_ints(rng, (K, N), kind)
    Ad, Bd = to_device(A), to_device(B)
    C = run(kind, Ad, Bd, path)
    torch.cuda.synchronize()
    del Ad, Bd
    tiles = corner_tiles(M, N)
    for (r, c), R in zip(tiles, oracle.gemm_tiles(A, B, tiles, 32)):
        got = C[r:r + R.shape[0], c:c + R.shape[1]].cpu().numpy().astype(np.float64)
        assert np.array_equal(got, R), (kind, shape, r, c)
