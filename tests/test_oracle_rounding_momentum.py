"""Pins of the oracle's rounding helpers and momentum against library routines
and exact special cases (no GPU)."""

import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- rounding --
def test_bf16_rounding_matches_torch_on_float32_values(rng):
    # torch's float32 -> bfloat16 cast is round-to-nearest-even; on float32
    # inputs a direct fp64 rounding must agree with it exactly.
    x = (rng.standard_normal(200_000) * 10.0 ** rng.integers(-30, 30, 200_000)).astype(np.float32)
    x = np.concatenate([x, np.float32([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38, 1e-40, -1e-40])])
    assert x.dtype == np.float32  # torch rounds float64 -> bf16 through float32 (twice)
    ours = oracle.round_to_bf16(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(ours, ref)


def test_bf16_rounding_is_direct_not_double():
    # x just above the midpoint between two bf16 neighbours, by less than a
    # float32 half-ulp: rounding through float32 would land on the midpoint and
    # tie to even (down); the single rounding must go up.
    lo = 1.0 + 2.0 ** -7 * 2  # even-significand bf16 (1.0000010b)
    mid = lo + 2.0 ** -8
    x = mid + 2.0 ** -30
    assert oracle.round_to_bf16(np.array([x]))[0] == lo + 2.0 ** -7
    assert oracle.round_to_bf16(np.array([mid]))[0] == lo  # exact tie -> even
    # ties to even in the other parity
    odd = 1.0 + 2.0 ** -7
    assert oracle.round_to_bf16(np.array([odd + 2.0 ** -8]))[0] == odd + 2.0 ** -7


def test_bf16_special_values():
    big = np.ldexp(255.0 / 128.0, 127)
    vals = np.array([np.inf, -np.inf, np.nan, big, big + 2.0 ** 119, big + 2.0 ** 118,
                     2.0 ** -133, 2.0 ** -135])
    r = oracle.round_to_bf16(vals)
    assert r[0] == np.inf and r[1] == -np.inf and np.isnan(r[2])
    assert r[3] == big
    assert r[4] == np.inf  # half a quantum past the largest finite bf16 ties away to inf
    assert r[5] == big
    assert r[6] == 2.0 ** -133  # smallest subnormal
    assert r[7] == 0.0  # below half the smallest subnormal


def test_bf16_bits_roundtrip(rng):
    x = oracle.round_to_bf16(rng.standard_normal(1000))
    np.testing.assert_array_equal(oracle.bf16_from_bits(oracle.bf16_bits(x)), x)
    t = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)
    np.testing.assert_array_equal(t.view(torch.int16).numpy().view(np.uint16), oracle.bf16_bits(x))


# ---------------------------------------------------------------- momentum --
def test_momentum_equals_float32_multiply_then_add(rng):
    M = (rng.standard_normal(1_000_000) * 1e-3).astype(np.float32)
    G = (rng.standard_normal(1_000_000) * 1e-3).astype(np.float32)
    ours = oracle.momentum_update(M, G, 0.95)
    # NumPy float32 ops are IEEE single, round-to-nearest-even, one op at a time.
    ref = (np.float32(0.95) * M) + G
    np.testing.assert_array_equal(ours, ref)


def test_momentum_is_not_fused(rng):
    # With a fused multiply-add the result differs on a large fraction of
    # elements; the oracle must match the two-rounding form, not the fused one.
    M = (rng.standard_normal(100_000) * 1e-3).astype(np.float32)
    G = (rng.standard_normal(100_000) * 1e-3).astype(np.float32)
    ours = oracle.momentum_update(M, G, 0.95)
    fused = oracle.round_to_f32(np.float64(np.float32(0.95)) * M.astype(np.float64) + G.astype(np.float64))
    assert np.mean(ours != fused) > 0.05


def test_momentum_special_cases(rng):
    M = (rng.standard_normal(10_000)).astype(np.float32)
    G = (rng.standard_normal(10_000)).astype(np.float32)
    np.testing.assert_array_equal(oracle.momentum_update(M, G, 0.0), G)  # mu = 0 -> M = G
    np.testing.assert_array_equal(oracle.momentum_update(np.zeros_like(M), G, 0.95), G)  # M_0 = 0
    np.testing.assert_array_equal(oracle.momentum_update(M, np.zeros_like(G), 0.95), np.float32(0.95) * M)
    # mu is the float32 nearest 0.95
    assert np.float32(0.95) == np.float32(0.949999988079071)


def test_page_constants_golden():
    with open(os.path.join(GOLDEN, "page_constants.json")) as f:
        g = json.load(f)
    assert oracle.MU == g["momentum_mu"]["value"]
    assert oracle.WEIGHT_DECAY == g["weight_decay_lambda"]["value"]
    assert oracle.TAU == g["tau"]["value"]
    assert oracle.ALPHA == g["alpha"]["value"]
    assert oracle.RMS_MATCH == g["rms_match_factor"]["value"]
    e = g["mla_scale_exponents"]["value"]
    # The oracle's MLA split with alpha = 0.5: q^C x gamma^alpha, k^C x gamma^(1-alpha), q^R x gamma.
    assert oracle.ALPHA == e["q_C"] and 1.0 - oracle.ALPHA == e["k_C"] and e["q_R"] == 1.0 and e["k_R"] == 0.0
    s = g["model_shapes"]["value"]
    assert oracle.muon_scale(s["expert_hidden"], s["hidden"]) == pytest.approx(np.sqrt(7168) * 0.2)
