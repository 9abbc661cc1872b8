"""Pins of the CPU oracle against facts fixed outside the oracle itself.

The oracle computes C[i,j] = sum_k A[i,k] B[k,j] in fp64 ("09 计算受限还是访存受限",
section on counting a matrix multiply; CS336 Lecture 5 GPU notes, §4.2). It is
pinned here by:

* closed forms that hold exactly in fp64: identity and permutation operands,
  all-ones (every element equals K), rank-1 integer outer products;
* integer inputs, whose exact product is known from integer arithmetic;
* brute force on tiny shapes against an exactly rounded sum (math.fsum),
  within the fp64 summation bound;
* NumPy's fp64 matmul as an independent library routine;
* the bf16 bit patterns of known values;
* the worked numbers the pages print for the cost model and the roofline
  (tests/golden/pages_worked_numbers.json).

The last test plants plausible mistakes in small pure-Python copies of the
oracle (a dropped term, a sign error, a transposed operand, swapped indices,
a wrong bf16 widening, shifted block offsets) and checks that the pins catch
every one of them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from tiled_dense_matrix_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_worked_numbers.json")
U = 2.0 ** -53

TINY = [1, 2, 3, 5, 7, 8, 16, 17, 31, 33]


def _f32(rng, shape):
    return inputs.uniform_fp32(rng, shape)


def _as_kind(X64, kind):
    """Store exact small values as fp32 or as bf16 bits."""
    X32 = np.asarray(X64, dtype=np.float32)
    return X32 if kind == "f32" else inputs.fp32_to_bf16_bits(X32)


# ---------------------------------------------------------------------------
# Pin suites: each takes a product function f(A, B) -> fp64 array and raises
# AssertionError when f disagrees with the fact it checks.
# ---------------------------------------------------------------------------

def pin_identity(f, kind="f32", shapes=((5, 7, 3), (16, 4, 9), (1, 8, 1))):
    rng = np.random.default_rng(11)
    for M, N, K in shapes:
        B = _as_kind(rng.integers(-50, 50, size=(M, N)), kind)  # K == M for A = I
        R = f(_as_kind(np.eye(M), kind), B)
        assert np.array_equal(R, oracle.widen(B)), "I @ B != B"
        A = _as_kind(rng.integers(-50, 50, size=(M, K)), kind)
        R = f(A, _as_kind(np.eye(K), kind))
        assert np.array_equal(R, oracle.widen(A)), "A @ I != A"


def pin_permutation(f, kind="f32"):
    rng = np.random.default_rng(12)
    for M, N in ((6, 9), (17, 3)):
        perm = rng.permutation(M)
        P = np.zeros((M, M))
        P[np.arange(M), perm] = 1.0  # (P @ B)[i] = B[perm[i]]
        Bv = rng.integers(-100, 100, size=(M, N))
        R = f(_as_kind(P, kind), _as_kind(Bv, kind))
        assert np.array_equal(R, Bv[perm].astype(np.float64)), "P @ B != rows of B permuted"
        Av = rng.integers(-100, 100, size=(N, M))
        R = f(_as_kind(Av, kind), _as_kind(P, kind))  # (A @ P)[:, perm[i]] = A[:, i]
        expect = np.empty_like(Av)
        expect[:, perm] = Av
        assert np.array_equal(R, expect.astype(np.float64)), "A @ P != columns of A permuted"


def pin_all_ones(f, kind="f32", shapes=((3, 4, 5), (1, 1, 1), (7, 2, 129), (2, 3, 1000))):
    for M, N, K in shapes:
        R = f(_as_kind(np.ones((M, K)), kind), _as_kind(np.ones((K, N)), kind))
        assert R.shape == (M, N)
        assert np.all(R == K), "all-ones product is not K everywhere"


def pin_rank1(f, kind="f32"):
    rng = np.random.default_rng(13)
    for M, N, K in ((4, 6, 5), (9, 3, 12)):
        u, s = rng.integers(-4, 5, size=M), rng.integers(-4, 5, size=K)
        t, v = rng.integers(-4, 5, size=K), rng.integers(-4, 5, size=N)
        A, B = np.outer(u, s), np.outer(t, v)
        R = f(_as_kind(A, kind), _as_kind(B, kind))
        expect = float(np.dot(s, t)) * np.outer(u, v).astype(np.float64)
        assert np.array_equal(R, expect), "rank-1 closed form violated"


def pin_integers(f, kind="f32"):
    rng = np.random.default_rng(14)
    for M, N, K in ((5, 6, 7), (16, 17, 31), (3, 2, 257)):
        A = rng.integers(-3, 4, size=(M, K))
        B = rng.integers(-3, 4, size=(K, N))
        R = f(_as_kind(A, kind), _as_kind(B, kind))
        assert np.array_equal(R, (A.astype(np.int64) @ B.astype(np.int64)).astype(np.float64)), \
            "integer product differs from exact integer arithmetic"


def pin_brute_force(f, sizes=TINY, count=40):
    """Random fp32 inputs on tiny shapes vs an exactly rounded sum (math.fsum)."""
    rng = np.random.default_rng(15)
    for _ in range(count):
        M, N, K = (int(rng.choice(sizes)) for _ in range(3))
        A = _f32(rng, (M, K))
        B = _f32(rng, (K, N))
        R = f(A, B)
        assert R.shape == (M, N)
        A64, B64 = A.astype(np.float64), B.astype(np.float64)
        for i in range(M):
            for j in range(N):
                terms = [A64[i, k] * B64[k, j] for k in range(K)]  # exact in fp64
                exact = math.fsum(terms)
                bound = (K + 1) * U * math.fsum(abs(x) for x in terms)
                assert abs(R[i, j] - exact) <= bound, (M, N, K, i, j)


def pin_bf16_values(f):
    """Known bf16 bit patterns through a 1x1x1 product with 1.0."""
    cases = {
        0x3F80: 1.0, 0xBF80: -1.0, 0xC040: -3.0, 0x3F81: 1.0 + 2.0 ** -7,
        0x4049: 3.140625, 0x0001: 2.0 ** -133, 0x7F7F: (2.0 - 2.0 ** -7) * 2.0 ** 127,
        0x0000: 0.0, 0x3C00: 2.0 ** -7,
    }
    one = np.array([[0x3F80]], dtype=np.uint16)
    for bits, value in cases.items():
        R = f(np.array([[bits]], dtype=np.uint16), one)
        assert R[0, 0] == value, hex(bits)


ALL_PINS = [pin_identity, pin_permutation, pin_all_ones, pin_rank1, pin_integers]


# ---------------------------------------------------------------------------
# The real oracle passes every pin.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kind", ["f32", "bf16"])
@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_closed_forms(pin, kind):
    pin(oracle.gemm, kind)


def test_brute_force_fsum():
    pin_brute_force(oracle.gemm)


def test_bf16_widening():
    pin_bf16_values(oracle.gemm)


def test_matches_numpy_fp64():
    rng = np.random.default_rng(16)
    for M, N, K in ((64, 48, 200), (33, 65, 129), (128, 96, 1024)):
        A, B = _f32(rng, (M, K)), _f32(rng, (K, N))
        R = oracle.gemm(A, B)
        ref = A.astype(np.float64) @ B.astype(np.float64)
        scale = np.abs(A.astype(np.float64)) @ np.abs(B.astype(np.float64))
        assert np.all(np.abs(R - ref) <= 2 * (K + 1) * U * scale)


def test_bf16_matches_numpy_fp64():
    rng = np.random.default_rng(17)
    A = inputs.normal_bf16(rng, (40, 300), 1.0)
    B = inputs.normal_bf16(rng, (300, 50), 0.02)
    R = oracle.gemm(A, B)
    A64, B64 = oracle.widen(A), oracle.widen(B)
    scale = np.abs(A64) @ np.abs(B64)
    assert np.all(np.abs(R - A64 @ B64) <= 2 * 301 * U * scale)


def test_blocks_equal_full_product():
    rng = np.random.default_rng(18)
    A, B = _f32(rng, (70, 90)), _f32(rng, (90, 110))
    full = oracle.gemm(A, B)
    for (i0, i1), (j0, j1) in (((0, 70), (0, 110)), ((3, 40), (17, 18)), ((69, 70), (0, 32)),
                               ((32, 64), (96, 110))):
        assert np.array_equal(oracle.gemm_block(A, B, (i0, i1), (j0, j1)), full[i0:i1, j0:j1])
    tiles = [(0, 0), (32, 64), (64, 96)]
    for (r, c), T in zip(tiles, oracle.gemm_tiles(A, B, tiles)):
        assert np.array_equal(T, full[r:r + 32, c:c + 32])


def test_thread_count_does_not_change_bits():
    rng = np.random.default_rng(19)
    A, B = _f32(rng, (97, 300)), _f32(rng, (300, 61))
    assert np.array_equal(oracle.gemm(A, B, threads=1), oracle.gemm(A, B, threads=8))


def test_empty_shapes():
    z = np.zeros((0, 5), np.float32)
    assert oracle.gemm(z, np.zeros((5, 3), np.float32)).shape == (0, 3)
    R = oracle.gemm(np.zeros((4, 0), np.float32), np.zeros((0, 6), np.float32))
    assert R.shape == (4, 6) and np.all(R == 0.0)  # empty sum


def test_rejects_bad_operands():
    with pytest.raises(ValueError):
        oracle.gemm(np.zeros((2, 3), np.float32), np.zeros((4, 2), np.float32))
    with pytest.raises(TypeError):
        oracle.gemm(np.zeros((2, 3), np.float64), np.zeros((3, 2), np.float64))
    with pytest.raises(ValueError):
        oracle.gemm_block(np.zeros((2, 3), np.float32), np.zeros((3, 2), np.float32), (0, 3), (0, 2))


# ---------------------------------------------------------------------------
# Cost model and roofline against the pages' printed numbers.
# ---------------------------------------------------------------------------

def _golden():
    with open(GOLDEN) as fh:
        return json.load(fh)


def _close(got, want, rel):
    return abs(got - want) <= rel * abs(want)


def test_roofline_cost_matches_pages():
    for e in _golden()["matmul_cost"]:
        flops, nbytes, ai = oracle.roofline(e["M"], e["N"], e["K"], e["in_bytes"], e["out_bytes"])
        if "flops" in e:
            assert _close(flops, e["flops"], e["flops_rel_tol"]), e["cite"]
        if "bytes" in e:
            assert _close(nbytes, e["bytes"], e["bytes_rel_tol"]), e["cite"]
        assert _close(ai, e["intensity"], e["intensity_rel_tol"]), e["cite"]


def test_square_fp32_intensity_is_n_over_6():
    for n in (1, 6, 256, 4096, 12345):
        assert math.isclose(oracle.roofline(n, n, n, 4, 4)[2], n / 6)


def test_ridge_and_attainable_match_pages():
    g = _golden()
    for e in g["roofline"]:
        assert _close(oracle.ridge(e["peak"], e["bandwidth"]), e["ridge"], e["ridge_rel_tol"]), e["cite"]
    for e in g["attainable"]:
        got = oracle.attainable(e["peak"], e["bandwidth"], e["flops"] / e["bytes"])
        assert _close(got, e["attained"], e["rel_tol"]), e["cite"]


def test_times_and_classification_match_pages():
    g = _golden()
    for e in g["times"]:
        if "M" in e:
            flops, nbytes, ai = oracle.roofline(e["M"], e["N"], e["K"], e["in_bytes"], e["out_bytes"])
            assert _close(flops / e["peak"], e["compute_s"], e["compute_rel_tol"]), e["cite"]
            assert _close(nbytes / e["bandwidth"], e["data_s"], e["data_rel_tol"]), e["cite"]
            bound = "compute" if ai > oracle.ridge(e["peak"], e["bandwidth"]) else "memory"
            assert bound == e["bound"], e["cite"]
        else:
            assert _close(e["bytes"] / e["bandwidth"], e["data_s"], e["data_rel_tol"]), e["cite"]
    for e in g["classification"]:
        ai = oracle.roofline(e["M"], e["N"], e["K"], e["in_bytes"], e["out_bytes"])[2]
        bound = "compute" if ai > oracle.ridge(e["peak"], e["bandwidth"]) else "memory"
        assert bound == e["bound"], e["cite"]


# ---------------------------------------------------------------------------
# Error metrics and Freivalds check.
# ---------------------------------------------------------------------------

def test_parity_metric_hand_values():
    R = np.arange(12, dtype=np.float64).reshape(3, 4)
    p = oracle.parity(R.copy(), R, 2.0, 3.0, 5)
    assert p["norm_max_err"] == 0.0 and p["rel_fro"] == 0.0
    C = R.copy()
    C[1, 2] += 0.3
    p = oracle.parity(C, R, 2.0, 3.0, 5)
    assert math.isclose(p["norm_max_err"], 0.3 / 30.0)
    assert math.isclose(p["rel_fro"], 0.3 / math.sqrt(float((R ** 2).sum())))
    assert oracle.parity(np.zeros_like(R), R, 2.0, 3.0, 5)["rel_fro"] == 1.0
    # A zero denominator demands an exact zero result.
    assert oracle.parity(np.zeros((2, 2)), np.zeros((2, 2)), 0.0, 1.0, 4)["norm_max_err"] == 0.0
    assert oracle.parity(np.ones((2, 2)), np.zeros((2, 2)), 0.0, 1.0, 4)["norm_max_err"] == math.inf


def test_freivalds_detects_a_corrupted_element():
    rng = np.random.default_rng(20)
    A, B = _f32(rng, (50, 70)), _f32(rng, (70, 40))
    R = oracle.gemm(A, B)
    x = inputs.pm_one_vector(rng, 40)
    good = oracle.freivalds(A, B, R, x)
    assert good["max_residual"] <= 1e-12 * good["max_row_abs_sum"]
    bad = R.copy()
    bad[7, 11] += 0.5
    assert math.isclose(oracle.freivalds(A, B, bad, x)["max_residual"], 0.5, rel_tol=1e-9)


# ---------------------------------------------------------------------------
# Planted mistakes: small pure-Python oracles with one plausible bug each.
# Every one must fail at least one pin.
# ---------------------------------------------------------------------------

def _py_oracle(bug=None):
    def widen(X):
        if X.dtype == np.uint16:
            shift = 15 if bug == "bf16_shift" else 16
            return ((X.astype(np.uint64) << shift) & 0xFFFFFFFF).astype(np.uint32).view(np.float32) \
                .astype(np.float64)
        return X.astype(np.float64)

    def f(A, B):
        A64, B64 = widen(A), widen(B)
        M, K = A64.shape
        N = B64.shape[1]
        R = np.zeros((M, N))
        for i in range(M):
            for j in range(N):
                s = 0.0
                kmax = K - 1 if bug == "drop_last_term" else K
                for k in range(kmax):
                    if bug == "transpose_b":
                        b = B64[j, k] if j < B64.shape[0] and k < B64.shape[1] else 0.0
                    else:
                        b = B64[k, j]
                    if bug == "swap_a_index":
                        a = A64[k, i] if k < M and i < K else 0.0
                    else:
                        a = A64[i, k]
                    term = a * b
                    if bug == "sign_last" and k == K - 1:
                        term = -term
                    s += term
                R[i, j] = s
        if bug == "first_row_zero":
            R[0, :] = 0.0
        return R
    return f


BUGS = ["drop_last_term", "transpose_b", "swap_a_index", "sign_last", "bf16_shift",
        "first_row_zero"]


def _run_pins(f):
    failures = 0
    small = [1, 2, 3, 5]
    for pin in ALL_PINS:
        for kind in ("f32", "bf16"):
            try:
                pin(f, kind)
            except (AssertionError, IndexError, ValueError):
                failures += 1
    for pin in (lambda g: pin_brute_force(g, sizes=small, count=8), pin_bf16_values):
        try:
            pin(f)
        except (AssertionError, IndexError, ValueError):
            failures += 1
    return failures


def test_correct_python_copy_passes_pins():
    assert _run_pins(_py_oracle()) == 0


@pytest.mark.parametrize("bug", BUGS)
def test_planted_mistake_is_caught(bug):
    assert _run_pins(_py_oracle(bug)) > 0, bug


def test_block_offset_mistake_is_caught():
    rng = np.random.default_rng(21)
    A, B = _f32(rng, (40, 50)), _f32(rng, (50, 60))
    full = oracle.gemm(A, B)
    shifted = oracle.gemm_block(A, B, (1, 33), (0, 32))  # a block taken one row off
    assert not np.array_equal(shifted, full[0:32, 0:32])


def test_special_values_follow_ieee_products_and_sums():
    """Closed forms from IEEE arithmetic: Inf * finite is a signed Inf,
    Inf * 0 and Inf + (-Inf) are NaN, and NaN is sticky. Checked on fp32
    inputs and on the same values as bf16 bits."""
    inf, nan = math.inf, math.nan
    A = np.array([[inf, 1.0], [nan, 0.0], [1.0, -inf]], np.float32)
    B = np.array([[1.0, 0.0, inf], [-1.0, 2.0, 1.0]], np.float32)
    for a, b in ((A, B), (inputs.fp32_to_bf16_bits(A), inputs.fp32_to_bf16_bits(B))):
        R = oracle.gemm(a, b)
        assert R[0, 0] == inf                  # inf*1 + 1*(-1)
        assert math.isnan(R[0, 1])             # inf*0 + 1*2
        assert R[0, 2] == inf                  # inf*inf + 1*1
        assert np.isnan(R[1]).all()            # NaN row
        assert R[2, 0] == inf                  # 1*1 + (-inf)*(-1)
        assert R[2, 1] == -inf                 # 1*0 + (-inf)*2
        assert math.isnan(R[2, 2])             # 1*inf + (-inf)*1


# ---------------------------------------------------------------------------
# Fused epilogue: GELU, bias, residual, bf16 rounding.
# ---------------------------------------------------------------------------

def test_gelu_matches_the_normal_cdf_table():
    """GELU(x) = x Phi(x): Phi(1) = 0.8413447460685429 and Phi(2) =
    0.9772498680518208 (standard normal table). The tanh approximation
    (0.84119 at 1), x*sigmoid(1.702x), a missing 1/2 or erf(x/2) all miss."""
    assert oracle.gelu(0.0) == 0.0
    assert abs(oracle.gelu(1.0) - 0.8413447460685429) < 1e-15
    assert abs(oracle.gelu(-1.0) + (1.0 - 0.8413447460685429)) < 1e-15
    assert abs(oracle.gelu(2.0) - 2 * 0.9772498680518208) < 1e-15
    x = np.linspace(-8.0, 8.0, 161)
    assert np.allclose(oracle.gelu(x) - oracle.gelu(-x), x, rtol=0, atol=1e-14)  # Phi(x)+Phi(-x) = 1
    assert abs(oracle.gelu(20.0) - 20.0) < 1e-12 and abs(oracle.gelu(-20.0)) < 1e-12


def test_epilogue_order_and_broadcast():
    """bias before GELU, residual after: 1 + 1 -> GELU(2) = 2 Phi(2), + 3.
    Residual before GELU would give ~5, bias after GELU 4.84."""
    R = np.array([[1.0]])
    got = oracle.epilogue(R, np.array([1.0], np.float32), np.array([[3.0]], np.float32), True)
    assert abs(got[0, 0] - (2 * 0.9772498680518208 + 3.0)) < 1e-14
    # bias is per column, residual per element; bf16 bits are widened exactly
    bias = inputs.fp32_to_bf16_bits(np.array([1.0, 2.0, 3.0], np.float32))
    res = inputs.fp32_to_bf16_bits(np.array([[0.5, 0.0, 0.0], [0.0, 0.0, -0.25]], np.float32))
    got = oracle.epilogue(np.zeros((2, 3)), bias, res)
    assert np.array_equal(got, [[1.5, 2.0, 3.0], [1.0, 2.0, 2.75]])
    assert np.array_equal(oracle.epilogue(np.ones((2, 2))), np.ones((2, 2)))


def test_round_to_bf16_ties_to_even():
    """bf16 keeps 8 significant bits: on [256, 512) neighbours are 2 apart,
    on [1, 2) 2^-7 apart. Halfway cases go to the even neighbour."""
    got = oracle.round_to_bf16([257.0, 259.0, 1 + 2 ** -8, 1 + 3 * 2 ** -9, 1 + 2 ** -7,
                                -257.0, 0.0, 256.0])
    assert [int(v) for v in got] == [0x4380, 0x4382, 0x3F80, 0x3F81, 0x3F81, 0xC380, 0x0000,
                                     0x4380]
    with pytest.raises(ValueError):
        oracle.round_to_bf16([0.1])  # not an fp32 value


# ---------------------------------------------------------------------------
# B stored N x K (a linear layer's weight): C = A B^T.
# ---------------------------------------------------------------------------

def test_gemm_nt_hand_values_and_shape():
    """C[i,j] = sum_k A[i,k] Bt[j,k] worked by hand for a 2x3 A and 4x3 Bt;
    reading Bt as K x N would not even have matching shapes."""
    A = np.array([[1, 2, 3], [4, 5, 6]], np.float32)
    Bt = np.array([[1, 0, -1], [2, 1, 0], [0, 0, 1], [1, 1, 1]], np.float32)
    C = oracle.gemm_nt(A, Bt)
    assert C.shape == (2, 4)
    assert np.array_equal(C, [[-2, 4, 3, 6], [-2, 13, 6, 15]])
    for a, b in ((A, Bt), (inputs.fp32_to_bf16_bits(A), inputs.fp32_to_bf16_bits(Bt))):
        assert np.array_equal(oracle.gemm_nt(a, b), C)


def test_gemm_nt_of_a_matrix_with_itself_is_its_gram_matrix():
    """A A^T is symmetric with the squared row norms on the diagonal (exact
    for small integers); the tile helper agrees with the full product."""
    rng = np.random.default_rng(12)
    A = rng.integers(-3, 4, size=(37, 53)).astype(np.float32)
    G = oracle.gemm_nt(A, A)
    assert np.array_equal(G, G.T)
    assert np.array_equal(np.diag(G), (A.astype(np.float64) ** 2).sum(axis=1))
    Bt = rng.integers(-3, 4, size=(70, 53)).astype(np.float32)
    full = oracle.gemm_nt(A, Bt)
    tiles = [(0, 0), (32, 32), (5, 64)]
    for (r, c), T in zip(tiles, oracle.gemm_nt_tiles(A, Bt, tiles, 32)):
        assert np.array_equal(T, full[r:r + 32, c:c + 32])


def test_gemm_tn_hand_values_and_shape():
    """C[i,j] = sum_k At[k,i] B[k,j] worked by hand for a 3x2 At (K = 3,
    M = 2) and a 3x4 B; reading At as M x K would not even have matching
    shapes, and on a square operand it gives other values (next test)."""
    At = np.array([[1, 2], [3, 4], [5, 6]], np.float32)
    B = np.array([[1, 0, 2, -1], [0, 1, 0, 1], [1, 1, -1, 0]], np.float32)
    C = oracle.gemm_tn(At, B)
    assert C.shape == (2, 4)
    # row 0 of A is column 0 of At: (1, 3, 5); row 1 is (2, 4, 6)
    assert np.array_equal(C, [[6, 8, -3, 2], [8, 10, -2, 2]])
    for a, b in ((At, B), (inputs.fp32_to_bf16_bits(At), inputs.fp32_to_bf16_bits(B))):
        assert np.array_equal(oracle.gemm_tn(a, b), C)


def test_gemm_tn_of_a_matrix_with_itself_is_its_gram_matrix():
    """A^T A (A stored K x M here, so gemm_tn(X, X) = X^T X) is symmetric with
    the squared column norms of X on the diagonal, exact for small integers;
    the tile helper agrees with the full product."""
    rng = np.random.default_rng(13)
    X = rng.integers(-3, 4, size=(53, 37)).astype(np.float32)
    G = oracle.gemm_tn(X, X)
    assert G.shape == (37, 37)
    assert np.array_equal(G, G.T)
    assert np.array_equal(np.diag(G), (X.astype(np.float64) ** 2).sum(axis=0))
    B = rng.integers(-3, 4, size=(53, 70)).astype(np.float32)
    full = oracle.gemm_tn(X, B)
    tiles = [(0, 0), (32, 32), (5, 64)]
    for (r, c), T in zip(tiles, oracle.gemm_tn_tiles(X, B, tiles, 32)):
        assert np.array_equal(T, full[r:r + 32, c:c + 32])


def test_gemm_tn_planted_orientation_mistake_is_caught():
    """A copy that multiplies the stored K x M matrix as if it were M x K
    (the mistake the pages warn about: a transpose is another layout) fails
    both gemm_tn pins on square operands, where the shapes do not give it
    away."""
    def wrong_tn(At, B):
        return oracle.gemm(At, B)

    rng = np.random.default_rng(14)
    X = rng.integers(-3, 4, size=(16, 16)).astype(np.float32)
    B = rng.integers(-3, 4, size=(16, 16)).astype(np.float32)
    G = wrong_tn(X, X)
    gram_ok = np.array_equal(G, G.T) and np.array_equal(
        np.diag(G), (X.astype(np.float64) ** 2).sum(axis=0))
    assert not gram_ok
    assert not np.array_equal(wrong_tn(X, B), oracle.gemm_tn(X, B))


# ---------------------------------------------------------------------------
# FP8 operands with block scales
# ---------------------------------------------------------------------------

FP8_GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_fp8_formats.json")
ALL_CODES = np.arange(256, dtype=np.uint8)


def _fp8_formats():
    with open(FP8_GOLDEN) as fh:
        return json.load(fh)["formats"]


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_largest_value_is_the_pages_range(fmt):
    """The largest finite magnitude is the range the pages' format table
    prints (448, 57344), reached by the positive and the negative code."""
    g = {f["name"]: f for f in _fp8_formats()}[fmt]
    assert g["sign_bits"] + g["exponent_bits"] + g["mantissa_bits"] == g["total_bits"] == 8
    v = oracle.fp8_decode(ALL_CODES, fmt)
    fin = v[np.isfinite(v)]
    assert fin.max() == g["max_finite"] and fin.min() == -g["max_finite"]


@pytest.mark.parametrize("fmt,torch_dtype", [("e4m3", "float8_e4m3fn"), ("e5m2", "float8_e5m2")])
def test_fp8_decode_of_every_code_matches_torch(fmt, torch_dtype):
    """All 256 codes against PyTorch's own float8 types (an independent
    library decode): equal values, NaN and infinities at the same codes."""
    torch = pytest.importorskip("torch")
    ref = torch.from_numpy(ALL_CODES.copy()).view(getattr(torch, torch_dtype)).to(torch.float64).numpy()
    got = oracle.fp8_decode(ALL_CODES, fmt)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))  # -0.0 at 0x80


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_value_ladder(fmt):
    """Structure the field widths fix: positive codes increase strictly; the
    spacing is constant across the subnormals and the first binade (no gap
    or overlap at the boundary) and doubles from binade to binade; the sign
    bit only negates; E4M3 has exactly two NaN codes and no infinity, E5M2
    two infinities and six NaNs."""
    E, Mb = oracle.FP8_FORMATS[fmt]
    v = oracle.fp8_decode(ALL_CODES, fmt)
    pos = v[:128]
    fin = pos[np.isfinite(pos)]
    assert np.all(np.diff(fin) > 0)
    step0 = fin[1] - fin[0]
    per = 1 << Mb
    assert np.all(np.diff(fin[:2 * per + 1]) == step0)  # subnormals + first binade
    for b in range(1, (len(fin) - 1) // per - 1):
        seg = np.diff(fin[per * b: per * (b + 1) + 1])
        assert np.all(seg == step0 * 2.0 ** (b - 1)), b
    neg = v[128:]
    assert np.array_equal(np.isnan(neg), np.isnan(pos))
    okv = ~np.isnan(pos)
    assert np.array_equal(neg[okv], -pos[okv])
    if fmt == "e4m3":
        assert np.isnan(v).sum() == 2 and not np.isinf(v).any()
        assert step0 == 2.0 ** -9
    else:
        assert np.isnan(v).sum() == 6 and np.isinf(v).sum() == 2
        assert step0 == 2.0 ** -16
    assert oracle.fp8_decode(np.array([(7 if fmt == "e4m3" else 15) << Mb], np.uint8), fmt)[0] == 1.0


def test_e8m0_scale_exponents():
    v = oracle.e8m0_decode(ALL_CODES)
    assert v[127] == 1.0 and v[128] == 2.0 and v[0] == 2.0 ** -127 and v[254] == 2.0 ** 127
    assert np.isnan(v[255]) and not np.isnan(v[:255]).any()
    assert np.array_equal(v[1:255], 2.0 * v[:254])


def test_gemm_fp8_hand_values():
    """2 x 2 by hand: A = [[1, 2], [-0.5, 448]], B (N x K) = [[1, 1], [4, -2]]
    in E4M3: C = [[3, 0], [447.5, -898]]."""
    enc = {1.0: 0x38, 2.0: 0x40, -0.5: 0xB0, 448.0: 0x7E, 4.0: 0x48, -2.0: 0xC0}
    A = np.array([[enc[1.0], enc[2.0]], [enc[-0.5], enc[448.0]]], np.uint8)
    B = np.array([[enc[1.0], enc[1.0]], [enc[4.0], enc[-2.0]]], np.uint8)
    assert np.array_equal(oracle.gemm_fp8(A, "e4m3", B, "e4m3"), [[3.0, 0.0], [447.5, -898.0]])


def test_gemm_fp8_all_ones_with_block_scales_has_a_closed_form():
    """A and B all 1.0: C[i,j] = 32 * sum_b 2^(sa[i,b]-127) 2^(sb[j,b]-127).
    Scales differ per row and per block, and M != N, so swapped scale axes or
    rows would not pass."""
    rng = np.random.default_rng(21)
    M, N, K = 3, 5, 96
    A = np.full((M, K), 0x38, np.uint8)
    B = np.full((N, K), 0x3C, np.uint8)  # 1.0 in E5M2
    sa = rng.integers(120, 135, size=(M, K // 32)).astype(np.uint8)
    sb = rng.integers(120, 135, size=(N, K // 32)).astype(np.uint8)
    C = oracle.gemm_fp8(A, "e4m3", B, "e5m2", sa, sb)
    want = 32.0 * (2.0 ** (sa.astype(np.int64) - 127)) @ (2.0 ** (sb.astype(np.int64) - 127)).T
    assert np.array_equal(C, want)


def test_gemm_fp8_equals_the_fp32_product_of_independently_decoded_operands():
    """Random codes and scales: the operands rebuilt through PyTorch's float8
    decode and np.ldexp, as fp32 (exact for these scales), through the fp32
    oracle path with B transposed to K x N. Rows, columns, blocks and the
    transpose all differ in size."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(22)
    M, N, K = 7, 9, 128
    A = rng.integers(0, 256, size=(M, K), dtype=np.uint8)
    B = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    A[(A & 0x7F) == 0x7F] = 0x11  # no NaN codes in this test
    B[(B & 0x7C) == 0x7C] = 0x22  # no infinities or NaNs
    sa = rng.integers(118, 137, size=(M, K // 32)).astype(np.uint8)
    sb = rng.integers(118, 137, size=(N, K // 32)).astype(np.uint8)

    def rebuild(codes, dt, s):
        x = torch.from_numpy(codes.copy()).view(dt).to(torch.float64).numpy()
        return np.ldexp(x, np.repeat(s.astype(np.int64) - 127, 32, axis=1)).astype(np.float32)

    a32 = rebuild(A, torch.float8_e4m3fn, sa)
    b32 = rebuild(B, torch.float8_e5m2, sb)
    ref = oracle.gemm(a32, np.ascontiguousarray(b32.T))
    assert np.array_equal(oracle.gemm_fp8(A, "e4m3", B, "e5m2", sa, sb), ref)
    tiles = oracle.gemm_fp8_tiles(A, "e4m3", B, "e5m2", [(0, 0), (3, 4)], sa, sb, tile=4)
    assert np.array_equal(tiles[0], ref[0:4, 0:4]) and np.array_equal(tiles[1], ref[3:7, 4:8])


def test_gemm_fp8_special_values():
    """A NaN code or a NaN scale (255) makes its row NaN; E5M2 infinity times
    a positive value is +inf, times zero NaN."""
    M, N, K = 2, 2, 32
    A = np.full((M, K), 0x38, np.uint8)
    B = np.full((N, K), 0x3C, np.uint8)
    C = oracle.gemm_fp8(A, "e4m3", B, "e5m2")
    assert np.array_equal(C, np.full((2, 2), 32.0))
    A2 = A.copy()
    A2[0, 5] = 0x7F  # E4M3 NaN
    C = oracle.gemm_fp8(A2, "e4m3", B, "e5m2")
    assert np.isnan(C[0]).all() and np.array_equal(C[1], [32.0, 32.0])
    B2 = B.copy()
    B2[1, 3] = 0x7C  # E5M2 +inf
    C = oracle.gemm_fp8(A, "e4m3", B2, "e5m2")
    assert np.isposinf(C[:, 1]).all() and np.array_equal(C[:, 0], [32.0, 32.0])
    A3 = A.copy()
    A3[1, 3] = 0x00  # zero meets the infinity
    C = oracle.gemm_fp8(A3, "e4m3", B2, "e5m2")
    assert np.isnan(C[1, 1]) and np.isposinf(C[0, 1])
    sa = np.full((M, 1), 127, np.uint8)
    sb = np.full((N, 1), 127, np.uint8)
    sa[1, 0] = 255
    C = oracle.gemm_fp8(A, "e4m3", B, "e5m2", sa, sb)
    assert np.isnan(C[1]).all() and np.array_equal(C[0], [32.0, 32.0])


# Planted mistakes in the FP8 decode and block scaling: each must fail at
# least one of the FP8 pins above.
_FP8_PINS = [
    lambda: [test_fp8_largest_value_is_the_pages_range(f) for f in ("e4m3", "e5m2")],
    lambda: [test_fp8_decode_of_every_code_matches_torch(f, t)
             for f, t in (("e4m3", "float8_e4m3fn"), ("e5m2", "float8_e5m2"))],
    lambda: [test_fp8_value_ladder(f) for f in ("e4m3", "e5m2")],
    test_e8m0_scale_exponents,
    test_gemm_fp8_hand_values,
    test_gemm_fp8_all_ones_with_block_scales_has_a_closed_form,
    test_gemm_fp8_equals_the_fp32_product_of_independently_decoded_operands,
    test_gemm_fp8_special_values,
]


def _fp8_mutant(bug):
    good_decode, good_e8m0, good_scaled = oracle.fp8_decode, oracle.e8m0_decode, oracle.fp8_scaled

    def decode(codes, fmt):
        E, Mb = oracle.FP8_FORMATS[fmt]
        bias = (1 << (E - 1)) - 1 + (1 if bug == "bias_off_by_one" else 0)
        c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
        sign = 1.0 if bug == "sign_ignored" else np.where(c & 0x80, -1.0, 1.0)
        e = (c >> Mb) & ((1 << E) - 1)
        frac = (c & ((1 << Mb) - 1)) / float(1 << Mb)
        sub_exp = -bias if bug == "subnormal_exponent" else 1 - bias
        mag = np.where(e == 0, frac * 2.0 ** sub_exp, (1.0 + frac) * np.exp2((e - bias).astype(float)))
        top = (1 << E) - 1
        if fmt == "e5m2" or bug == "e4m3_ieee_specials":
            mag = np.where((e == top) & (frac == 0), np.inf, mag)
            mag = np.where((e == top) & (frac != 0), np.nan, mag)
        else:
            mag = np.where((e == top) & (frac == 1 - 1 / (1 << Mb)), np.nan, mag)
        return sign * mag

    def e8m0(codes):
        v = good_e8m0(codes)
        return v / 2.0 if bug == "scale_bias" else v

    def scaled(codes, fmt, scales=None):
        if scales is None or bug != "scale_blocks_tiled":
            return good_scaled(codes, fmt, scales)
        X = oracle.fp8_decode(codes, fmt)
        return X * np.tile(oracle.e8m0_decode(scales), (1, 32))

    patches = {}
    if bug in ("bias_off_by_one", "sign_ignored", "subnormal_exponent", "e4m3_ieee_specials"):
        patches["fp8_decode"] = decode
    if bug == "scale_bias":
        patches["e8m0_decode"] = e8m0
    if bug == "scale_blocks_tiled":
        patches["fp8_scaled"] = scaled
    return patches


FP8_BUGS = ["bias_off_by_one", "sign_ignored", "subnormal_exponent", "e4m3_ieee_specials",
            "scale_bias", "scale_blocks_tiled"]


@pytest.mark.parametrize("bug", FP8_BUGS)
def test_planted_fp8_mistake_is_caught(bug, monkeypatch):
    for name, fn in _fp8_mutant(bug).items():
        monkeypatch.setattr(oracle, name, fn)
    failures = 0
    for pin in _FP8_PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            failures += 1
    assert failures > 0, bug


# ---------------------------------------------------------------------------
# Attention: O = softmax(Q K^T * scale) V per head, and the row logsumexp.
# ---------------------------------------------------------------------------

def _sdpa(Q, K, V, scale, causal):
    torch = pytest.importorskip("torch")
    t = lambda X: torch.tensor(oracle.widen(np.asarray(X)))  # noqa: E731
    return torch.nn.functional.scaled_dot_product_attention(
        t(Q), t(K), t(V), is_causal=causal, scale=scale).numpy()


@pytest.mark.parametrize("shape,causal", [((2, 3, 17, 23, 16), False), ((1, 2, 40, 40, 64), True),
                                          ((1, 1, 1, 9, 8), False), ((2, 2, 33, 33, 128), True)])
def test_attention_matches_torch_sdpa_in_fp64(shape, causal):
    """PyTorch's own scaled_dot_product_attention on the CPU in fp64 (an
    independent library routine), with and without the causal mask."""
    B, H, nq, nk, d = shape
    rng = np.random.default_rng(nq * 31 + d)
    Q = rng.standard_normal((B, H, nq, d))
    K = rng.standard_normal((B, H, nk, d))
    V = rng.standard_normal((B, H, nk, d))
    O, _ = oracle.attention(Q, K, V, d ** -0.5, causal)
    assert np.abs(O - _sdpa(Q, K, V, d ** -0.5, causal)).max() < 1e-13


def test_attention_closed_forms():
    """Equal keys: every weight is 1/n, O = the mean of V's rows and lse =
    s + log n. One key: O = that value row, lse = its score. Causal row 0
    sees key 0 only."""
    rng = np.random.default_rng(5)
    d, n = 8, 6
    Q = rng.standard_normal((4, d))
    k = rng.standard_normal(d)
    K = np.tile(k, (n, 1))
    V = rng.standard_normal((n, d))
    O, L = oracle.attention(Q, K, V, 0.5)
    assert np.allclose(O, V.mean(axis=0)[None, :], rtol=0, atol=1e-15)
    assert np.allclose(L, 0.5 * (Q @ k) + np.log(n), rtol=0, atol=1e-14)
    O1, L1 = oracle.attention(Q, K[:1], V[:1], 0.5)
    assert np.array_equal(O1, np.tile(V[0], (4, 1))) and np.allclose(L1, 0.5 * (Q @ k), atol=1e-15)
    Kr = rng.standard_normal((4, d))
    Oc, Lc = oracle.attention(Q, Kr, V[:4], 0.3, causal=True)
    assert np.array_equal(Oc[0], V[0]) and abs(Lc[0] - 0.3 * Q[0] @ Kr[0]) < 1e-15


def test_attention_brute_force_and_logsumexp():
    """A 3 x 5 head by explicit loops with math.exp and math.fsum; lse
    against scipy's logsumexp."""
    from scipy.special import logsumexp
    rng = np.random.default_rng(6)
    Q, K, V = rng.standard_normal((3, 4)), rng.standard_normal((5, 4)), rng.standard_normal((5, 4))
    sc = 0.7
    O, L = oracle.attention(Q, K, V, sc)
    for i in range(3):
        s = [sc * math.fsum(Q[i, t] * K[j, t] for t in range(4)) for j in range(5)]
        w = [math.exp(x) for x in s]
        tot = math.fsum(w)
        for c in range(4):
            assert abs(O[i, c] - math.fsum(w[j] * V[j, c] for j in range(5)) / tot) < 1e-14
        assert abs(L[i] - logsumexp(s)) < 1e-14


def test_attention_is_stable_for_large_scores_and_takes_bf16():
    """Scores near 1000 (exp would overflow without the row maximum taken
    out) stay finite and agree with torch; bf16 bits are widened exactly."""
    rng = np.random.default_rng(7)
    Q = rng.standard_normal((5, 16)) * 30.0
    K = rng.standard_normal((9, 16)) * 30.0
    V = rng.standard_normal((9, 16))
    O, L = oracle.attention(Q, K, V, 0.25)
    assert np.isfinite(O).all() and np.isfinite(L).all() and np.abs(L).max() > 100
    assert np.abs(O - _sdpa(Q[None], K[None], V[None], 0.25, False)[0]).max() < 1e-12
    Qb, Kb, Vb = (inputs.fp32_to_bf16_bits(X.astype(np.float32)) for X in (Q, K, V))
    Ob, _ = oracle.attention(Qb, Kb, Vb, 0.25)
    Ow, _ = oracle.attention(oracle.widen(Qb), oracle.widen(Kb), oracle.widen(Vb), 0.25)
    assert np.array_equal(Ob, Ow)
    rows = [0, 3, 4]
    Or, Lr = oracle.attention_rows(Q, K, V, rows, 0.25)
    assert np.allclose(Or, O[rows], atol=1e-15) and np.allclose(Lr, L[rows], atol=1e-13)


def _attention_mutant(bug):
    def f(Q, K, V, scale, causal=False):
        q, k, v = (oracle.widen(np.asarray(X)) for X in (Q, K, V))
        S = q @ k.T * (1.0 if bug == "no_scale" else scale)
        if causal:
            keys = np.arange(k.shape[0])[None, :]
            rows = np.arange(q.shape[0])[:, None]
            S = np.where(keys >= rows if bug == "mask_diagonal" else keys > rows, -np.inf, S)
        axis = 0 if bug == "softmax_axis" else 1
        m = 0.0 if bug == "no_max" else S.max(axis=axis, keepdims=True)
        P = np.exp(S - m)
        l = P.sum(axis=axis, keepdims=True)
        vv = v.T if bug == "v_transposed" else v
        O = (P @ vv) / l
        lse = (np.log(l) if bug == "lse_without_m" else m + np.log(l))
        return O, np.broadcast_to(lse, (q.shape[0], 1))[:, 0]
    return f


@pytest.mark.parametrize("bug", ["no_scale", "mask_diagonal", "softmax_axis", "no_max",
                                 "v_transposed", "lse_without_m"])
def test_planted_attention_mistake_is_caught(bug):
    """Each plausible mistake disagrees with torch (or the closed forms) on
    one of these square heads; the correct copy agrees."""
    rng = np.random.default_rng(8)
    caught = False
    for causal, big in ((False, 1.0), (True, 1.0), (False, 40.0)):
        n, d = 12, 12
        Q = rng.standard_normal((n, d)) * big
        K = rng.standard_normal((n, d)) * big
        V = rng.standard_normal((n, d))
        from scipy.special import logsumexp
        S = Q @ K.T * d ** -0.5
        if causal:
            S = np.where(np.arange(n)[None, :] > np.arange(n)[:, None], -np.inf, S)
        ref_O = _sdpa(Q[None], K[None], V[None], d ** -0.5, causal)[0]
        ref_L = logsumexp(S, axis=1)
        with np.errstate(all="ignore"):
            for f, expect_ok in ((_attention_mutant(None), True), (_attention_mutant(bug), False)):
                try:
                    O, L = f(Q, K, V, d ** -0.5, causal)
                    ok = np.allclose(O, ref_O, atol=1e-10) and np.allclose(L, ref_L, atol=1e-9)
                except ValueError:  # a mistake that breaks the shapes is caught too
                    ok = False
                if expect_ok:
                    assert ok
                elif not ok:
                    caught = True
    assert caught, bug
