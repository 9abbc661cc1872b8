"""FP8 product with block scales (needs an MI355X).

gemm_fp8 computes C[i,j] = sum_k (sa[i,k/32] A[i,k]) (sb[j,k/32] B[j,k]) for
FP8 codes A [M, K], B [N, K] (E4M3 or E5M2 each) and optional power-of-two
block scales, in fp32, then the fused epilogue. The oracle decodes every code
and scale exactly and sums in fp64 (oracle.gemm_fp8).

The tolerance follows the arithmetic of the instruction, as measured on
gfx950 through the library (test_instruction_arithmetic_reading): the
products of each aligned group of 8 consecutive k are added on the grid
2^(E - 13), E the exponent of the group's largest product magnitude, each
cut toward zero (1 + 2^-13 is exact, 1 + 2^-14 gives 1; 256 + 2^-5 is exact,
256 + 2^-6 gives 256; 1 - 1.5 * 2^-13 gives 1 - 2^-13), before the group's
sum joins the fp32 accumulator; products in different groups do not cut
each other. The bound below takes the coarser groups of 64 k of one
instruction (its E_g is at least that of any group of 8 inside it, so it
covers the measured arithmetic). Per element the bound is then
  sum over groups g of 64 * 2^(E_g - 13)            (the cut products)
  + 2 * K * 2^-24 * sum_k |a_k b_k|                  (fp32 accumulation)
  + the output rounding,
and the normalized max error stays within the bf16 parity bar (the cut
alone is below 2^-13 of max|a| max|b| per term).

Checks:
  * the measured arithmetic itself, on crafted one-row operands;
  * random block-quantized operands, all four format pairs, with and without
    scales, against that bound and (outputs of 1024 elements or more) a
    relative Frobenius gate;
  * small-integer values with power-of-two scales: sums exact in fp32, so
    the output must equal the oracle bit for bit;
  * the fused epilogue (bias, GELU, residual, bf16 output);
  * scale rows that cannot be read as aligned words (K not a multiple of
    128, or a misaligned scale pointer) and the partial K step;
  * NaN / infinity codes and NaN scales where the oracle puts them;
  * run-to-run determinism and the full-size workload on sampled tiles.
"""
import numpy as np
import pytest

import oracle
import tiled_dense_matrix_amd as tdm
from tiled_dense_matrix_amd import inputs

from helpers import log, to_device

torch = pytest.importorskip("torch")

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

F = tdm.Fp8Format
NAME = {F.E4M3: "e4m3", F.E5M2: "e5m2"}


def dev8(X):
    return None if X is None else torch.from_numpy(np.ascontiguousarray(X)).cuda()


def run(A, fa, B, fb, sa=None, sb=None, out=torch.float32, bias=None, residual=None, gelu=False):
    D = tdm.gemm_fp8(dev8(A), dev8(B), fa, fb, dev8(sa), dev8(sb), out_dtype=out,
                     bias=None if bias is None else to_device(bias),
                     residual=None if residual is None else to_device(residual), gelu=gelu)
    torch.cuda.synchronize()
    if out == torch.bfloat16:
        return oracle.widen(D.view(torch.int16).cpu().numpy().view(np.uint16))
    return D.cpu().numpy().astype(np.float64)


def quantized(rng, rows, K, fmt, scaled, sigma=1.0):
    x = rng.standard_normal((rows, K)) * sigma
    if scaled:
        return inputs.mx_quantize(x, fmt)
    return inputs.encode_fp8(x, fmt), None


def abs_codes(X):
    return None if X is None else (X & 0x7F).astype(np.uint8)


def cut_bound(A, fa, B, fb, sa=None, sb=None):
    """sum over 64-k groups of 64 * 2^(E_g - 13) per output element, E_g the
    exponent of the group's largest |a_k b_k| (scaled values; NaN and
    infinite inputs count as 0)."""
    a = np.nan_to_num(oracle.fp8_scaled(A, fa, sa), nan=0.0, posinf=0.0, neginf=0.0)
    b = np.nan_to_num(oracle.fp8_scaled(B, fb, sb), nan=0.0, posinf=0.0, neginf=0.0)
    M, K = a.shape
    out = np.zeros((M, b.shape[0]))
    for r0 in range(0, M, 64):
        for g0 in range(0, K, 64):
            pa = np.abs(a[r0:r0 + 64, g0:g0 + 64])
            pb = np.abs(b[:, g0:g0 + 64])
            mx = (pa[:, None, :] * pb[None, :, :]).max(axis=2)
            e = np.floor(np.log2(np.where(mx > 0, mx, 1.0)))
            out[r0:r0 + 64] += np.where(mx > 0, 64.0 * np.exp2(e - 13), 0.0)
    return out


def bound(K, S, R, cut, out_bf16=False):
    """The instruction's product cut, fp32 accumulation (factor 2 of slack
    for the order the matrix cores add in), the output rounding."""
    return (cut + 2.0 * K * 2.0 ** -24 * S + 2.0 ** -23 * np.abs(R)
            + (2.0 ** -8 * np.abs(R) if out_bf16 else 0))


TOL_NORM = 4e-3  # normalized max error bar of the bf16 product
# Relative Frobenius gate, for outputs of at least 1024 elements. The
# elementwise bound above adds worst cases term by term; this gate asks that
# the errors stay small on the whole. A CPU emulation of the reading above
# (each 64-k group's products cut toward zero to multiples of 2^(E - 13),
# summed exactly) gives 2e-5 to 4.5e-5 on every random shape and format pair
# of this file; a single output (a few dozen terms) is not averaged and can
# reach a few 1e-4, so small outputs keep only the elementwise bound. 1.5e-4
# leaves a margin of three and still fails a product missing one 32-k block
# of 4096 (relative error about (32/4096)^(1/2) = 0.09) or one with a wrong
# scale on one block (about 0.1).
TOL_FRO_FP8 = 1.5e-4
FRO_MIN_OUTPUTS = 1024


def rel_fro(got, R):
    den = float(np.linalg.norm(R))
    return float(np.linalg.norm(got - R)) / den if den > 0 else float(np.linalg.norm(got))


def normalized_max_error(got, R, A, fa, B, fb, sa, sb, K):
    a = np.abs(oracle.fp8_scaled(A, fa, sa)).max()
    b = np.abs(oracle.fp8_scaled(B, fb, sb)).max()
    return float(np.abs(got - R).max() / (a * b * K))


SHAPES = [(1, 1, 32), (5, 7, 96), (64, 64, 128), (130, 200, 160), (300, 520, 256),
          (512, 768, 1024), (40, 1000, 4096)]
PAIRS = [(F.E4M3, F.E4M3), (F.E5M2, F.E5M2), (F.E4M3, F.E5M2), (F.E5M2, F.E4M3)]


def _cases():
    for shape in SHAPES:
        for fa, fb in PAIRS:
            for scaled in (True, False):
                if shape[0] * shape[1] * shape[2] > 1 << 28 and (fa, fb) != PAIRS[0]:
                    continue
                yield pytest.param(shape, fa, fb, scaled,
                                   id=f"{shape[0]}x{shape[1]}x{shape[2]}-{NAME[fa]}-{NAME[fb]}-"
                                      f"{'scaled' if scaled else 'plain'}")


@pytest.mark.parametrize("shape,fa,fb,scaled", list(_cases()))
def test_random_parity(shape, fa, fb, scaled):
    M, N, K = shape
    log(f"case fp8 random {shape} {NAME[fa]}x{NAME[fb]} scaled={scaled}")
    rng = np.random.default_rng(M * 7 + N + K + 100 * int(fa) + 10 * int(fb) + scaled)
    A, sa = quantized(rng, M, K, NAME[fa], scaled)
    B, sb = quantized(rng, N, K, NAME[fb], scaled, sigma=0.05)
    got = run(A, fa, B, fb, sa, sb)
    R = oracle.gemm_fp8(A, NAME[fa], B, NAME[fb], sa, sb)
    S = oracle.gemm_fp8(abs_codes(A), NAME[fa], abs_codes(B), NAME[fb], sa, sb)
    err = np.abs(got - R)
    tol = bound(K, S, R, cut_bound(A, NAME[fa], B, NAME[fb], sa, sb))
    assert np.all(err <= tol), float((err / np.maximum(tol, 1e-300)).max())
    assert normalized_max_error(got, R, A, NAME[fa], B, NAME[fb], sa, sb, K) <= TOL_NORM
    if M * N >= FRO_MIN_OUTPUTS:
        assert rel_fro(got, R) <= TOL_FRO_FP8, rel_fro(got, R)


def _one_row(K, vals_a, scales_a):
    """A 1 x K operand: code `c` at k, and one scale exponent per 32-k block
    (or None: no scales)."""
    A = np.zeros((1, K), np.uint8)
    for k, c in vals_a:
        A[0, k] = c
    return A, None if scales_a is None else np.array([scales_a], np.uint8)


# E5M2 codes of A: 1.0 = 0x3C, 2^-13 = 0x08, 2^-14 = 0x04, -1.5 * 2^-13 = 0x8A,
# 256 = 0x5C, 2^-5 = 0x28, 2^-6 = 0x24; E4M3 1.0 = 0x38.
CUT_CASES = [
    # (K, A format, [(k, code)], block scale exponents of A or None, D[0, 0])
    # k in one aligned group of 8: the smaller product lands on the grid of
    # the larger one, 2^(E - 13), cut toward zero
    (64, F.E5M2, [(0, 0x3C), (1, 0x08)], None, 1.0 + 2.0 ** -13),
    (64, F.E5M2, [(0, 0x3C), (1, 0x04)], None, 1.0),
    (64, F.E5M2, [(0, 0x3C), (7, 0x04)], None, 1.0),
    (64, F.E5M2, [(16, 0x3C), (20, 0x04)], None, 1.0),
    (64, F.E5M2, [(0, 0x3C), (1, 0x04), (2, 0x04)], None, 1.0),
    (64, F.E5M2, [(0, 0x3C), (1, 0x8A)], None, 1.0 - 2.0 ** -13),
    (64, F.E5M2, [(0, 0x5C), (1, 0x28)], None, 256.0 + 2.0 ** -5),
    (64, F.E5M2, [(0, 0x5C), (1, 0x24)], None, 256.0),
    (64, F.E4M3, [(0, 0x38), (1, 0x38)], [127, 127], 2.0),
    # products in different groups of 8 do not cut each other, within one
    # instruction (k < 64) or across two: they keep every bit
    (64, F.E5M2, [(0, 0x3C), (8, 0x04)], None, 1.0 + 2.0 ** -14),
    (64, F.E5M2, [(16, 0x3C), (24, 0x04)], None, 1.0 + 2.0 ** -14),
    (64, F.E5M2, [(0, 0x3C), (31, 0x04)], None, 1.0 + 2.0 ** -14),
    (64, F.E5M2, [(0, 0x3C), (32, 0x04)], None, 1.0 + 2.0 ** -14),
    (64, F.E5M2, [(0, 0x3C), (63, 0x04)], None, 1.0 + 2.0 ** -14),
    (128, F.E5M2, [(0, 0x3C), (64, 0x04)], None, 1.0 + 2.0 ** -14),
    (64, F.E5M2, [(0, 0x5C), (33, 0x24)], None, 256.0 + 2.0 ** -6),
    (64, F.E5M2, [(0, 0x3C), (1, 0x04), (2, 0x04), (33, 0x04), (34, 0x04)], None,
     1.0 + 2.0 ** -13),
    # with block scales, the scale multiplies after the cut of its group
    (64, F.E4M3, [(0, 0x38), (32, 0x38)], [127, 127 - 14], 1.0 + 2.0 ** -14),
    (64, F.E5M2, [(0, 0x3C), (1, 0x04)], [128, 128], 2.0),
]


@pytest.mark.parametrize("K,fa,vals,scales,want", CUT_CASES)
def test_instruction_arithmetic_reading(K, fa, vals, scales, want):
    """The arithmetic the elementwise bound rests on, measured through the
    library with B all ones (E4M3 1.0, scale 1), so D[0, 0] is the sum of
    A's (scaled) values: the products of each aligned group of 8 consecutive
    k are summed on the grid 2^(E - 13) of the largest of them, cut toward
    zero; products in different groups are not cut by each other. The
    bound's groups of 64 k (one instruction) contain eight such groups, and
    a group's E is at most the instruction's, so the bound holds."""
    log(f"case fp8 instruction reading K={K} {NAME[fa]} {vals} {scales}")
    A, sa = _one_row(K, vals, scales)
    B = np.full((1, K), 0x38, np.uint8)
    sb = None if scales is None else np.full((1, K // 32), 127, np.uint8)
    exact = float(oracle.gemm_fp8(A, NAME[fa], B, "e4m3", sa, sb)[0, 0])
    got = run(A, fa, B, F.E4M3, sa, sb)
    assert got[0, 0] == want, (got[0, 0], want, exact)


def _int_codes(rng, shape, fmt):
    """Codes of integers in [-4, 4], exact in both formats."""
    one = {"e4m3": 0x38, "e5m2": 0x3C}[fmt]
    step = {"e4m3": 8, "e5m2": 4}[fmt]  # code distance of one binade
    table = np.array([0, one, one + step, one + step + step // 2, one + 2 * step], np.int64)
    v = rng.integers(-4, 5, size=shape)
    codes = table[np.abs(v)] | np.where(v < 0, 0x80, 0)
    return codes.astype(np.uint8), v.astype(np.float64)


@pytest.mark.parametrize("shape", [(16, 256, 128), (130, 200, 160), (300, 520, 256), (7, 9, 32)])
def test_integer_values_with_power_of_two_scales_are_exact(shape):
    M, N, K = shape
    rng = np.random.default_rng(M + N + K)
    for fa, fb in PAIRS:
        log(f"case fp8 integer {shape} {NAME[fa]}x{NAME[fb]}")
        A, va = _int_codes(rng, (M, K), NAME[fa])
        B, vb = _int_codes(rng, (N, K), NAME[fb])
        assert np.array_equal(oracle.fp8_decode(A, NAME[fa]), va)  # the codes are the integers
        sa = rng.integers(125, 130, size=(M, K // 32)).astype(np.uint8)
        sb = rng.integers(125, 130, size=(N, K // 32)).astype(np.uint8)
        for s_a, s_b in ((None, None), (sa, sb)):
            got = run(A, fa, B, fb, s_a, s_b)
            assert np.array_equal(got, oracle.gemm_fp8(A, NAME[fa], B, NAME[fb], s_a, s_b))


@pytest.mark.parametrize("shape", [(300, 520, 256), (16, 1024, 2048), (7, 40, 96)])
def test_fused_epilogue(shape):
    M, N, K = shape
    rng = np.random.default_rng(M + 3 * N + K)
    A, sa = quantized(rng, M, K, "e4m3", True)
    B, sb = quantized(rng, N, K, "e4m3", True, sigma=0.02)
    bias = inputs.fp32_to_bf16_bits((rng.standard_normal(N) * 0.5).astype(np.float32))
    res = inputs.fp32_to_bf16_bits(rng.standard_normal((M, N)).astype(np.float32))
    log(f"case fp8 epilogue {shape}")
    got = run(A, F.E4M3, B, F.E4M3, sa, sb, torch.bfloat16, bias, res, True)
    R = oracle.gemm_fp8(A, "e4m3", B, "e4m3", sa, sb)
    E = oracle.epilogue(R, bias, res, use_gelu=True)
    T = oracle.epilogue(R, bias)
    S = oracle.gemm_fp8(abs_codes(A), "e4m3", abs_codes(B), "e4m3", sa, sb)
    cut = cut_bound(A, "e4m3", B, "e4m3", sa, sb)
    tol = (1.13 * (cut + 2.0 * K * 2.0 ** -24 * S + 2.0 ** -24 * np.abs(T))
           + 3e-7 * np.maximum(1.0, np.abs(T)) + 2.0 ** -23 * np.abs(E) + 2.0 ** -8 * np.abs(E))
    assert np.all(np.abs(got - E) <= tol), float((np.abs(got - E) / tol).max())


@pytest.mark.parametrize("shape", [(130, 200, 160), (64, 96, 4096 + 32)])
def test_scale_rows_read_byte_by_byte(shape):
    """K/32 not a multiple of 4 (scale rows not word-aligned) and scale
    tensors at an odd address: the register path for the scales."""
    M, N, K = shape
    rng = np.random.default_rng(M + N)
    A, sa = quantized(rng, M, K, "e4m3", True)
    B, sb = quantized(rng, N, K, "e5m2", True, sigma=0.05)
    R = oracle.gemm_fp8(A, "e4m3", B, "e5m2", sa, sb)
    S = oracle.gemm_fp8(abs_codes(A), "e4m3", abs_codes(B), "e5m2", sa, sb)
    log(f"case fp8 scale rows {shape}")
    ref = run(A, F.E4M3, B, F.E5M2, sa, sb)
    assert np.all(np.abs(ref - R) <= bound(K, S, R, cut_bound(A, "e4m3", B, "e5m2", sa, sb)))
    # the same scales one byte into their allocations
    nkb = K // 32
    ba = torch.zeros(M * nkb + 1, dtype=torch.uint8, device="cuda")
    bb = torch.zeros(N * nkb + 1, dtype=torch.uint8, device="cuda")
    ba[1:] = dev8(sa.reshape(-1))
    bb[1:] = dev8(sb.reshape(-1))
    D = tdm.gemm_fp8(dev8(A), dev8(B), F.E4M3, F.E5M2, ba[1:].view(M, nkb), bb[1:].view(N, nkb),
                     out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(D.cpu().numpy().astype(np.float64), ref)


def test_special_values():
    """NaN codes, E5M2 infinities (and infinity times zero) and a NaN scale
    land where the oracle puts them; other outputs stay finite and close."""
    M, N, K = 64, 96, 128
    rng = np.random.default_rng(9)
    A, sa = quantized(rng, M, K, "e4m3", True)
    B, sb = quantized(rng, N, K, "e5m2", True, sigma=0.05)
    A[3, 17] = 0x7F             # E4M3 NaN: row 3
    B[10, 5] = 0x7C             # E5M2 +inf: column 10 (signed by A[:, 5])
    A[20, 5] = 0x00             # ... times zero: NaN at (20, 10)
    B[40, 70] = 0xFC            # E5M2 -inf: column 40
    sa[50, 2] = 255             # NaN scale: row 50
    log("case fp8 special values")
    got = run(A, F.E4M3, B, F.E5M2, sa, sb)
    R = oracle.gemm_fp8(A, "e4m3", B, "e5m2", sa, sb)
    assert np.isnan(R).any() and np.isinf(R).any()
    assert np.array_equal(np.isnan(got), np.isnan(R))
    assert np.array_equal(np.isposinf(got), np.isposinf(R))
    assert np.array_equal(np.isneginf(got), np.isneginf(R))
    fin = np.isfinite(R)
    Af, Bf = A.copy(), B.copy()
    Af[3, 17] = 0; Bf[10, 5] = 0; Bf[40, 70] = 0
    sa_f = np.where(sa == 255, 127, sa).astype(np.uint8)
    S = oracle.gemm_fp8(abs_codes(Af), "e4m3", abs_codes(Bf), "e5m2", sa_f, sb)
    cut = cut_bound(Af, "e4m3", Bf, "e5m2", sa_f, sb)
    assert np.all(np.abs(got[fin] - R[fin]) <= bound(K, S, R, cut)[fin])


def test_large_tiles_with_a_partial_step_sampled():
    """4096 x 3072 runs on 256 x 256 tiles; K = 672 is five full steps and a
    partial one (taken first). 48 sampled tiles and the corners."""
    M, N, K = 4096, 3072, 672
    rng = np.random.default_rng(31)
    A, sa = quantized(rng, M, K, "e4m3", True)
    B, sb = quantized(rng, N, K, "e5m2", True, sigma=0.05)
    log(f"case fp8 large tiles {M}x{N}x{K}")
    got = run(A, F.E4M3, B, F.E5M2, sa, sb)
    tiles = sorted(set(inputs.sample_tiles(M, N, count=48)) |
                   {(0, 0), (0, N - 32), (M - 32, 0), (M - 32, N - 32)})
    R = oracle.gemm_fp8_tiles(A, "e4m3", B, "e5m2", tiles, sa, sb)
    S = oracle.gemm_fp8_tiles(abs_codes(A), "e4m3", abs_codes(B), "e5m2", tiles, sa, sb)
    for (r, c), Rt, St in zip(tiles, R, S):
        cut = cut_bound(A[r:r + 32], "e4m3", B[c:c + 32], "e5m2", sa[r:r + 32], sb[c:c + 32])
        assert np.all(np.abs(got[r:r + 32, c:c + 32] - Rt) <= bound(K, St, Rt, cut)), (r, c)


@pytest.mark.parametrize("shape", [(4096, 3072, 512), (16, 8192, 1024)])
def test_run_to_run_bitwise_determinism(shape):
    M, N, K = shape
    rng = np.random.default_rng(4)
    A, sa = quantized(rng, M, K, "e4m3", True)
    B, sb = quantized(rng, N, K, "e4m3", True)
    a, b, s_a, s_b = dev8(A), dev8(B), dev8(sa), dev8(sb)
    log(f"case fp8 determinism {shape}")
    ref = tdm.gemm_fp8(a, b, F.E4M3, F.E4M3, s_a, s_b, out_dtype=torch.float32).clone()
    for _ in range(100):
        again = tdm.gemm_fp8(a, b, F.E4M3, F.E4M3, s_a, s_b, out_dtype=torch.float32)
        assert torch.equal(again, ref)


def test_full_size_workload():
    """8192 x 14336 x 4096 E4M3 with block scales, bf16 output, as bench.py
    times it: 64 sampled 32 x 32 tiles and the four corners against the
    oracle, one by one."""
    w = inputs.WORKLOADS["fp8_mlp"]
    log(f"case workload {w.name} {w.M}x{w.N}x{w.K}")
    A, B, sa, sb = inputs.make_fp8_inputs(w)
    got = run(A, F.E4M3, B, F.E4M3, sa, sb, torch.bfloat16)
    tiles = sorted(set(inputs.sample_tiles(w.M, w.N)) |
                   {(0, 0), (0, w.N - 32), (w.M - 32, 0), (w.M - 32, w.N - 32)})
    R = oracle.gemm_fp8_tiles(A, "e4m3", B, "e4m3", tiles, sa, sb)
    S = oracle.gemm_fp8_tiles(abs_codes(A), "e4m3", abs_codes(B), "e4m3", tiles, sa, sb)
    worst = 0.0
    for (r, c), Rt, St in zip(tiles, R, S):
        err = np.abs(got[r:r + 32, c:c + 32] - Rt)
        cut = cut_bound(A[r:r + 32], "e4m3", B[c:c + 32], "e4m3", sa[r:r + 32], sb[c:c + 32])
        worst = max(worst, float((err / bound(w.K, St, Rt, cut, True)).max()))
    assert worst <= 1.0, worst
    got_t = np.concatenate([got[r:r + 32, c:c + 32].ravel() for r, c in tiles])
    ref_t = np.concatenate([Rt.ravel() for Rt in R])
    fro = rel_fro(got_t, ref_t)
    assert fro <= TOL_FRO_FP8 + 2.0 ** -8, fro  # + the bf16 output's rounding
    log(f"  {w.name}: worst err/bound {worst:.3f} rel_fro {fro:.3e}")


def test_full_size_shape_integer_values_bit_exact():
    """The workload's shape (8192 x 14336 x 4096, B stored N x K) with
    integer codes in [-4, 4] and block scales 2^-1..2^1: every product is a
    multiple of 2^-2 below 64 in magnitude, every partial sum below 2^18,
    exact in fp32 under any order and above the instruction's cut (2^-7 at
    most), so the output equals the oracle bit for bit. Compared on the 64
    sampled tiles, the four corners and the first and last 32 rows."""
    w = inputs.WORKLOADS["fp8_mlp"]
    log(f"case fp8 integer full shape {w.M}x{w.N}x{w.K}")
    rng = np.random.default_rng((w.seed, 2))
    A, _ = _int_codes(rng, (w.M, w.K), "e4m3")
    B, _ = _int_codes(rng, (w.N, w.K), "e4m3")
    sa = rng.integers(126, 129, size=(w.M, w.K // 32)).astype(np.uint8)
    sb = rng.integers(126, 129, size=(w.N, w.K // 32)).astype(np.uint8)
    got = run(A, F.E4M3, B, F.E4M3, sa, sb)
    tiles = sorted(set(inputs.sample_tiles(w.M, w.N)) |
                   {(0, 0), (0, w.N - 32), (w.M - 32, 0), (w.M - 32, w.N - 32)})
    for (r, c), Rt in zip(tiles, oracle.gemm_fp8_tiles(A, "e4m3", B, "e4m3", tiles, sa, sb)):
        assert np.array_equal(got[r:r + 32, c:c + 32], Rt), (r, c)
    for r0 in (0, w.M - 32):
        rows = oracle.gemm_fp8(A[r0:r0 + 32], "e4m3", B, "e4m3", sa[r0:r0 + 32], sb)
        assert np.array_equal(got[r0:r0 + 32], rows), r0
