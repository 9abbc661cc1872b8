"""Attention forward (FlashAttention scheme) against the fp64 oracle (needs an
MI355X).

attention_fwd computes O = softmax(Q K^T * scale) V per (batch, head) from
bf16 Q, K, V with fp32 accumulation, rounding the probabilities to bf16
before they multiply V, and stores O in bf16 and the row logsumexp in fp32.
The oracle is the definition in fp64 (oracle.attention).

Bound per output element, with W = sum_j P_ij |V_jd| (the oracle's weights
applied to |V|):
  2^-8 W      the probabilities rounded to bf16 (2^-9 relative each) and
              the normalizer summed from the unrounded ones (2^-9);
  2^-9 |O|    the bf16 output;
  (2^-12 + 2 e) W, e = head_dim * 2^-24 * |scale| * max_j sum_t |q_t k_jt|:
              each score is an fp32 sum of head_dim exact products, off by
              at most e (times log2 e, which the base-2 exponent turns back
              into a relative error of e in p), once in O's numerator and
              once in its normalizer; 2^-12 for the hardware exp2.
lse: the fp32 score error bound (head_dim * 2^-24 * scale * sum_t |q_t k_t|
at the row's largest) plus 2^-20 (1 + |lse|) for exp2, log2 and the sums.
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


def run(Q, K, V, causal, scale=None):
    O, L = tdm.attention_fwd(to_device(Q).view(torch.bfloat16), to_device(K).view(torch.bfloat16),
                             to_device(V).view(torch.bfloat16), causal=causal, scale=scale,
                             return_lse=True)
    torch.cuda.synchronize()
    return oracle.widen(O.view(torch.int16).cpu().numpy().view(np.uint16)), L.cpu().numpy()


def check(Q, K, V, causal, scale, got_O, got_L, heads=None, rows=None):
    """Compare (sampled) heads and rows with the oracle."""
    Qf = Q.reshape(-1, *Q.shape[-2:]); Kf = K.reshape(-1, *K.shape[-2:]); Vf = V.reshape(-1, *V.shape[-2:])
    gO = got_O.reshape(-1, *got_O.shape[-2:]); gL = got_L.reshape(-1, got_L.shape[-1])
    heads = range(Qf.shape[0]) if heads is None else heads
    worst = 0.0
    for h in heads:
        r = np.arange(Qf.shape[1]) if rows is None else np.asarray(rows)
        O, L = oracle.attention_rows(Qf[h], Kf[h], Vf[h], r, scale, causal)
        W, _ = oracle.attention_rows(Qf[h], Kf[h], np.abs(oracle.widen(Vf[h])), r, scale, causal)
        qa, ka = np.abs(oracle.widen(Qf[h][r])), np.abs(oracle.widen(Kf[h]))
        smax = (qa @ ka.T).max(axis=1) * abs(scale)
        e = (Qf.shape[-1] * 2.0 ** -24 * smax)[:, None]
        tol = 2.0 ** -8 * W + 2.0 ** -9 * np.abs(O) + (2.0 ** -12 + 2 * e) * W + 1e-30
        err = np.abs(gO[h][r] - O)
        worst = max(worst, float((err / tol).max()))
        assert np.all(err <= tol), (h, float((err / tol).max()))
        tol_l = Qf.shape[-1] * 2.0 ** -24 * smax + 2.0 ** -20 * (1 + np.abs(L))
        assert np.all(np.abs(gL[h][r] - L) <= tol_l), (h, float((np.abs(gL[h][r] - L) / tol_l).max()))
    return worst


SHAPES = [  # batch, heads, n_q, n_kv, head_dim, causal
    (1, 1, 1, 1, 64, False), (1, 2, 37, 53, 64, False), (2, 3, 128, 128, 128, True),
    (1, 2, 300, 300, 128, True), (1, 1, 129, 65, 128, False), (1, 2, 1000, 777, 64, False),
    (2, 2, 256, 256, 64, True), (1, 1, 64, 4096, 128, False), (1, 1, 200, 1, 128, False),
    # a second 256-query workgroup holding one query; causal diagonals that
    # cross the waves of several workgroups
    (1, 2, 257, 700, 128, False), (1, 1, 520, 520, 64, True), (1, 1, 513, 513, 128, True),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"{b}x{h}x{q}x{k}x{d}{'c' if c else ''}"
                                               for b, h, q, k, d, c in SHAPES])
def test_random_parity(shape):
    B, H, nq, nk, d, causal = shape
    log(f"case attention {shape}")
    rng = np.random.default_rng(nq * 13 + nk + d)
    Q = inputs.normal_bf16(rng, (B, H, nq, d), 1.0)
    K = inputs.normal_bf16(rng, (B, H, nk, d), 1.0)
    V = inputs.normal_bf16(rng, (B, H, nk, d), 1.0)
    O, L = run(Q, K, V, causal)
    worst = check(Q, K, V, causal, d ** -0.5, O, L)
    log(f"  worst err/bound {worst:.3f}")


def test_one_key_returns_its_value_row_exactly():
    """n_kv = 1: every weight is exactly 1, so O is V's row bit for bit and
    lse is the scaled score."""
    rng = np.random.default_rng(2)
    Q = inputs.normal_bf16(rng, (1, 3, 70, 128), 1.0)
    K = inputs.normal_bf16(rng, (1, 3, 1, 128), 1.0)
    V = inputs.normal_bf16(rng, (1, 3, 1, 128), 1.0)
    O, L = run(Q, K, V, False)
    assert np.array_equal(O, np.broadcast_to(oracle.widen(V), O.shape))
    ref = np.einsum("bhqd,bhkd->bhq", oracle.widen(Q), oracle.widen(K)) * 128 ** -0.5
    assert np.allclose(L, ref, rtol=0, atol=1e-4)


def test_equal_keys_average_the_values_and_scale_is_taken_as_given():
    """All keys equal: the weights are uniform whatever the scale (here a
    negative one), O = the mean of V."""
    rng = np.random.default_rng(3)
    Q = inputs.normal_bf16(rng, (1, 1, 96, 64), 1.0)
    k = inputs.normal_bf16(rng, (1, 1, 1, 64), 1.0)
    K = np.broadcast_to(k, (1, 1, 200, 64)).copy()
    V = inputs.normal_bf16(rng, (1, 1, 200, 64), 1.0)
    O, L = run(Q, K, V, False, scale=-0.3)
    mean = oracle.widen(V)[0, 0].mean(axis=0)
    assert np.all(np.abs(O[0, 0] - mean) <= 2.0 ** -8 * np.abs(mean) + 1e-4)
    check(Q, K, V, False, -0.3, O, L)


def test_large_scores_stay_finite():
    """Scores in the hundreds: the running maximum keeps exp in range."""
    rng = np.random.default_rng(4)
    Q = inputs.normal_bf16(rng, (1, 2, 130, 64), 8.0)
    K = inputs.normal_bf16(rng, (1, 2, 190, 64), 8.0)
    V = inputs.normal_bf16(rng, (1, 2, 190, 64), 1.0)
    O, L = run(Q, K, V, False)
    assert np.isfinite(O).all() and np.isfinite(L).all() and np.abs(L).max() > 100
    check(Q, K, V, False, 64 ** -0.5, O, L)


@pytest.mark.parametrize("causal", [False, True])
def test_rising_scores_move_the_maximum_in_many_blocks(causal):
    """Keys that grow along the sequence make later blocks' scores pass the
    running maximum again and again, so most blocks redo their
    probabilities from the new maximum and rescale O and l."""
    rng = np.random.default_rng(6)
    n, d = 900, 128
    Q = inputs.normal_bf16(rng, (1, 2, n, d), 1.0)
    grow = (0.25 + np.arange(n) / 60.0).reshape(1, 1, n, 1)
    K = inputs.fp32_to_bf16_bits(
        (inputs.bf16_bits_to_fp32(inputs.normal_bf16(rng, (1, 2, n, d), 1.0)) * grow).astype(np.float32))
    V = inputs.normal_bf16(rng, (1, 2, n, d), 1.0)
    O, L = run(Q, K, V, causal)
    assert np.isfinite(O).all() and np.isfinite(L).all()
    check(Q, K, V, causal, d ** -0.5, O, L)


@pytest.mark.parametrize("causal", [False, True])
def test_run_to_run_bitwise_determinism(causal):
    rng = np.random.default_rng(5)
    Q, K, V = (to_device(inputs.normal_bf16(rng, (2, 4, 1024, 128), 1.0)).view(torch.bfloat16)
               for _ in range(3))
    log(f"case attention determinism causal={causal}")
    ref = tdm.attention_fwd(Q, K, V, causal=causal).clone()
    for _ in range(100):
        assert torch.equal(tdm.attention_fwd(Q, K, V, causal=causal), ref)


@pytest.mark.parametrize("name", ["attn_fwd", "attn_fwd_causal"])
def test_full_size_workload(name):
    """4 x 32 heads, sequence 4096, head_dim 128, as bench.py runs it: 48
    sampled query rows (first and last included) on 6 sampled heads."""
    w = inputs.ATTN_WORKLOADS[name]
    log(f"case workload {name}")
    Q, K, V = inputs.make_attention_inputs(w)
    O, L = run(Q, K, V, w.causal)
    rng = np.random.default_rng(11)
    heads = sorted(set(rng.choice(w.batch * w.heads, 6, replace=False).tolist()) | {0})
    rows = sorted(set(rng.choice(w.seq, 46, replace=False).tolist()) | {0, w.seq - 1})
    worst = check(Q, K, V, w.causal, w.scale, O, L, heads, rows)
    log(f"  {name}: worst err/bound {worst:.3f}")


def test_zero_scale_with_the_causal_mask_averages_the_visible_values():
    """scale = 0: every visible key weighs the same, so row i is the mean of
    V[0..i] (masked keys must not turn into NaN on the way)."""
    rng = np.random.default_rng(12)
    n = 150
    Q = inputs.normal_bf16(rng, (1, 1, n, 64), 1.0)
    K = inputs.normal_bf16(rng, (1, 1, n, 64), 1.0)
    V = inputs.normal_bf16(rng, (1, 1, n, 64), 1.0)
    O, L = run(Q, K, V, True, scale=0.0)
    v = oracle.widen(V)[0, 0]
    mean = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
    assert np.isfinite(O).all()
    assert np.all(np.abs(O[0, 0] - mean) <= 2.0 ** -8 * np.abs(mean) + 2.0 ** -9 * np.abs(v).max())
    assert np.allclose(L[0, 0], np.log(np.arange(1, n + 1)), atol=1e-5)


@pytest.mark.parametrize("d", [64, 128])
def test_infinite_value_in_the_last_key_row_of_a_ragged_block(d):
    """n_kv = 100 leaves 28 padded rows in the second 64-key block, which
    hold copies of key row 99. With +Inf in one element of V[99] every query
    sees that key with a nonzero probability, so O is +Inf in that column
    and finite elsewhere, as the fp64 definition gives; a padded copy of the
    row taken with probability 0 must not turn it into NaN."""
    rng = np.random.default_rng(90 + d)
    Q, K, V = (inputs.normal_bf16(rng, (1, 1, n, d), 1.0) for n in (40, 100, 100))
    col = 5
    V[0, 0, 99, col] = 0x7F80  # bf16 +Inf
    log(f"case attention Inf in V row n_kv-1, d={d}")
    scale = d ** -0.5
    got_O, _ = run(Q, K, V, False, scale)
    R, _ = oracle.attention(Q, K, V, scale)
    assert np.all(np.isposinf(R[0, 0, :, col])) and np.all(np.isfinite(np.delete(R, col, axis=-1)))
    assert np.array_equal(np.isposinf(got_O), np.isposinf(R))
    assert not np.isnan(got_O).any()
    # the other columns: the bound of the module docstring, computed with
    # V's infinite element set to 0 (it does not reach them)
    fin = np.delete(np.arange(d), col)
    V2 = V.copy()
    V2[0, 0, 99, col] = 0
    r = np.arange(40)
    O_ref, _ = oracle.attention_rows(Q[0, 0], K[0, 0], V2[0, 0], r, scale)
    W, _ = oracle.attention_rows(Q[0, 0], K[0, 0], np.abs(oracle.widen(V2[0, 0])), r, scale)
    smax = (np.abs(oracle.widen(Q[0, 0])) @ np.abs(oracle.widen(K[0, 0])).T).max(axis=1) * scale
    e = (d * 2.0 ** -24 * smax)[:, None]
    tol = 2.0 ** -8 * W + 2.0 ** -9 * np.abs(O_ref) + (2.0 ** -12 + 2 * e) * W + 1e-30
    assert np.all(np.abs(got_O[0, 0][:, fin] - O_ref[:, fin]) <= tol[:, fin])
