"""Checks of the seeded input generator (shared by the oracle's and the GPU's tests)."""
import dataclasses
import json
import os

import numpy as np
import pytest
import torch

from tiled_dense_matrix_amd import inputs

DIGESTS = os.path.join(os.path.dirname(__file__), "golden", "input_digests.json")


def _golden_digests():
    with open(DIGESTS) as fh:
        return json.load(fh)


def _digest_module():
    import importlib.util
    path = os.path.join(os.path.dirname(__file__), "golden", "make_input_digests.py")
    spec = importlib.util.spec_from_file_location("make_input_digests", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_every_workload_has_a_digest():
    assert sorted(_golden_digests()) == sorted(_digest_module().names())


@pytest.mark.parametrize("name", sorted(_golden_digests()))
def test_digests_are_stable(name):
    """Every array of every workload (operands, block scales, bias, Q/K/V)
    hashes to the committed value: the recipe is pinned at full size."""
    assert _digest_module().workload_digests(name) == _golden_digests()[name], name


def test_workload_shapes_and_types():
    w = inputs.WORKLOADS
    assert (w["f32_4096"].M, w["f32_4096"].N, w["f32_4096"].K) == (4096, 4096, 4096)
    assert (w["bf16_mlp"].M, w["bf16_mlp"].N, w["bf16_mlp"].K) == (8192, 14336, 4096)
    assert (w["bf16_skinny"].M, w["bf16_skinny"].N, w["bf16_skinny"].K) == (16, 8192, 8192)
    A, B = inputs.make_inputs("f32_256")
    assert A.dtype == np.float32 and A.shape == (256, 256) and B.shape == (256, 256)
    A, B = inputs.make_inputs("bf16_skinny")
    assert A.dtype == np.uint16 and A.shape == (16, 8192) and B.shape == (8192, 8192)


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100_000).astype(np.float32),
        (rng.standard_normal(1000) * 1e-38).astype(np.float32),  # subnormal range
        np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 0.0, -0.0,
                  3.4e38, -3.4e38], dtype=np.float32),  # exact ties and extremes
    ])
    mine = inputs.fp32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)


def test_bf16_ties_go_to_even():
    # 1 + 2^-8 lies halfway between bf16 1.0 (even) and 1 + 2^-7 (odd).
    assert inputs.fp32_to_bf16_bits(np.array([1.0 + 2.0 ** -8], np.float32))[0] == 0x3F80
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even).
    assert inputs.fp32_to_bf16_bits(np.array([1.0 + 3 * 2.0 ** -8], np.float32))[0] == 0x3F82
    assert inputs.bf16_bits_to_fp32(np.array([0x3F82], np.uint16))[0] == 1.0 + 2.0 ** -6


def test_distributions():
    A, B = inputs.make_inputs("f32_256")
    assert A.min() >= -1.0 and A.max() < 1.0
    assert abs(float(A.mean())) < 0.01 and abs(float(A.var()) - 1.0 / 3.0) < 0.01
    A, B = inputs.make_inputs("bf16_skinny")
    a = inputs.bf16_bits_to_fp32(A).astype(np.float64)
    b = inputs.bf16_bits_to_fp32(B[:512]).astype(np.float64)
    assert abs(a.std() - 1.0) < 0.01
    assert abs(b.std() - 0.02) < 0.0005


def test_seeds_and_draw_order():
    A1, B1 = inputs.make_inputs(inputs.Workload("x", "f32", 8, 9, 10, 5, "uniform"))
    A2, B2 = inputs.make_inputs(inputs.Workload("x", "f32", 8, 9, 10, 5, "uniform"))
    A3, _ = inputs.make_inputs(inputs.Workload("x", "f32", 8, 9, 10, 6, "uniform"))
    assert np.array_equal(A1, A2) and np.array_equal(B1, B2)
    assert not np.array_equal(A1, A3)
    # A is drawn first from the seed's stream, then B.
    rng = np.random.default_rng(5)
    assert np.array_equal(A1, rng.uniform(-1.0, 1.0, (8, 10)).astype(np.float32))
    assert np.array_equal(B1, rng.uniform(-1.0, 1.0, (10, 9)).astype(np.float32))


def test_sample_tiles():
    t = inputs.sample_tiles(8192, 14336)
    assert len(t) == 64 and len(set(t)) == 64
    assert all(r % 32 == 0 and c % 32 == 0 and 0 <= r < 8192 and 0 <= c < 14336 for r, c in t)
    assert t == inputs.sample_tiles(8192, 14336)
    assert len(inputs.sample_tiles(64, 64)) == 4


def test_small_int_and_pm_one():
    rng = np.random.default_rng(1)
    X = inputs.small_int_matrix(rng, (50, 60), kind="bf16")
    v = inputs.bf16_bits_to_fp32(X)
    assert set(np.unique(v).tolist()) <= set(range(-3, 4))
    x = inputs.pm_one_vector(rng, 1000)
    assert set(np.unique(x).tolist()) == {-1.0, 1.0}


def test_epilogue_workload_shares_the_mlp_operands_and_draws_its_bias_apart():
    w = inputs.WORKLOADS["bf16_mlp_gelu"]
    m = inputs.WORKLOADS["bf16_mlp"]
    assert (w.M, w.N, w.K, w.seed, w.sigma_a, w.sigma_b) == (m.M, m.N, m.K, m.seed, m.sigma_a, m.sigma_b)
    assert w.has_epilogue and not m.has_epilogue and w.gelu and w.out == "bf16"
    b = inputs.make_bias(w)
    assert b.dtype == np.uint16 and b.shape == (w.N,)
    assert np.array_equal(b, inputs.make_bias("bf16_mlp_gelu"))  # seeded
    x = inputs.bf16_bits_to_fp32(b).astype(np.float64)
    assert abs(x.std() - 0.02) < 0.002 and abs(x.mean()) < 0.002


def test_fp8_encoding_matches_torch_round_to_nearest_even():
    """encode_fp8 against PyTorch's float8 conversion on values spread over
    both formats' ranges (subnormals, ties, saturation excluded by clipping)."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal(200_000) * np.array([1e-3, 0.05, 1.0, 30.0, 3e3])[rng.integers(0, 5, 200_000)]
    for fmt, dt, top in (("e4m3", torch.float8_e4m3fn, 448.0), ("e5m2", torch.float8_e5m2, 57344.0)):
        xc = np.clip(x, -top, top)
        ref = torch.from_numpy(xc).to(dt).view(torch.uint8).numpy()
        assert np.array_equal(inputs.encode_fp8(xc, fmt), ref), fmt
        # beyond the range: saturates to the largest finite code
        big = inputs.encode_fp8(np.array([1e6, -1e6]), fmt)
        assert np.array_equal(big, torch.tensor([top, -top], dtype=torch.float64).to(dt).view(torch.uint8).numpy())


def test_mx_block_scales_follow_the_recipe():
    """Per 32-k block: scale exponent floor(log2 max|x|) - emax + 127; the
    block's values divided by 2^(scale-127) round to the stored codes (the
    block maximum can land above the largest finite value, 1.75 * 2^emax, and
    saturates there)."""
    rng = np.random.default_rng(4)
    X = rng.standard_normal((6, 128)) * np.exp2(rng.integers(-6, 6, size=(6, 1)))
    X[5, 32:64] = 0.0
    for fmt, dt, emax, top in (("e4m3", torch.float8_e4m3fn, 8, 448.0),
                               ("e5m2", torch.float8_e5m2, 15, 57344.0)):
        codes, s = inputs.mx_quantize(X, fmt)
        assert codes.shape == X.shape and s.shape == (6, 4) and s.dtype == np.uint8
        blocks = np.abs(X).reshape(6, 4, 32).max(axis=2)
        want = np.where(blocks > 0, np.floor(np.log2(np.where(blocks > 0, blocks, 1.0))) - emax, 0) + 127
        assert np.array_equal(s, want.astype(np.uint8))
        scale = np.repeat(np.exp2(s.astype(np.float64) - 127), 32, axis=1)
        ref = torch.from_numpy(np.clip(X / scale, -top, top)).to(dt).view(torch.uint8).numpy()
        assert np.array_equal(codes, ref), fmt


def test_fp8_workload():
    w = inputs.WORKLOADS["fp8_mlp"]
    assert (w.kind, w.M, w.N, w.K, w.b_layout, w.scaled, w.out) == ("fp8", 8192, 14336, 4096, "nk", True, "bf16")
    small = inputs.Workload("t", "fp8", 40, 24, 96, 11, "normal", b_layout="nk", scaled=True)
    A, B, sa, sb = inputs.make_fp8_inputs(small)
    assert A.shape == (40, 96) and B.shape == (24, 96) and sa.shape == (40, 3) and sb.shape == (24, 3)
    assert A.dtype == B.dtype == sa.dtype == sb.dtype == np.uint8
    A2, B2, sa2, sb2 = inputs.make_fp8_inputs(small)  # seeded: the same draws again
    assert np.array_equal(A, A2) and np.array_equal(sb, sb2)
    plain = dataclasses.replace(small, scaled=False)
    A3, B3, sa3, sb3 = inputs.make_fp8_inputs(plain)
    assert sa3 is None and sb3 is None and A3.shape == (40, 96)
    with pytest.raises(ValueError):
        inputs.make_inputs("fp8_mlp")


def test_attention_workloads():
    w = inputs.ATTN_WORKLOADS["attn_fwd"]
    assert (w.batch, w.heads, w.seq, w.head_dim, w.causal) == (4, 32, 4096, 128, False)
    assert w.flops == 4.0 * 4 * 32 * 128 * 4096 * 4096
    c = inputs.ATTN_WORKLOADS["attn_fwd_causal"]
    assert c.causal and c.flops == 4.0 * 4 * 32 * 128 * (4096 * 4097 // 2)
    small = inputs.AttnWorkload("t", 1, 2, 50, 64, True, 3)
    Q, K, V = inputs.make_attention_inputs(small)
    assert Q.shape == K.shape == V.shape == (1, 2, 50, 64) and Q.dtype == np.uint16
    Q2, _, V2 = inputs.make_attention_inputs(small)
    assert np.array_equal(Q, Q2) and np.array_equal(V, V2) and not np.array_equal(Q, K)
