"""Pins of the fp64 attention-forward oracle (no GPU).

The definition (softmax(Q K^T / sqrt(d)) V per head, with the per-head max
logit of the same logits, "Kimi K2 内部机制": S_max is computed in the forward)
is pinned against a pure-Python loop, the separately pinned max-logit
function, and closed forms of the softmax.
"""

import math

import numpy as np
import pytest
from scipy.special import logsumexp

import oracle


def _inputs(rng, B, H, Sq, Sk, dc, dr, dv, scale=1.0):
    Q = rng.standard_normal((B, H, Sq, dc + dr)) * scale
    Kc = rng.standard_normal((B, H, Sk, dc)) * scale
    Kr = rng.standard_normal((B, Sk, dr)) * scale if dr else None
    V = rng.standard_normal((B, H, Sk, dv))
    return Q, Kc, Kr, V


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dr", [0, 2])
def test_attention_equals_bruteforce(rng, causal, dr):
    Q, Kc, Kr, V = _inputs(rng, 2, 2, 5, 7, 4, dr, 3)
    O, lse, smax = oracle.attention_forward(Q, Kc, Kr, V, causal)
    O2, smax2 = oracle.attention_forward_bruteforce(Q, Kc, Kr, V, causal)
    np.testing.assert_allclose(O, O2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(smax, smax2, rtol=1e-13)


def test_max_logit_is_the_unmasked_max_logit(rng):
    Q, Kc, Kr, V = _inputs(rng, 2, 3, 9, 11, 6, 2, 4, scale=3.0)
    _, _, smax = oracle.attention_forward(Q, Kc, Kr, V)
    np.testing.assert_allclose(smax, oracle.max_logit(Q, Kc, Kr), rtol=1e-13)


def test_causal_max_logit_only_sees_visible_keys(rng):
    B, H, S, d = 1, 1, 6, 4
    Q = rng.standard_normal((B, H, S, d))
    Kc = rng.standard_normal((B, H, S, d))
    Kc[0, 0, -1] = 50.0 * Q[0, 0, 0]  # the largest logit pairs query 0 with the last key
    V = rng.standard_normal((B, H, S, 2))
    _, _, full = oracle.attention_forward(Q, Kc, None, V)
    _, _, causal = oracle.attention_forward(Q, Kc, None, V, causal=True)
    # query 0 cannot see the last key under the mask; the last query can
    logits = Q[0, 0] @ Kc[0, 0].T / math.sqrt(d)
    visible = np.tril(np.ones((S, S), dtype=bool))
    assert full[0] == pytest.approx(logits.max(), rel=1e-14)
    assert causal[0] == pytest.approx(logits[visible].max(), rel=1e-14)
    assert causal[0] < full[0]


def test_softmax_closed_forms(rng):
    B, H, S, d, dv = 1, 2, 5, 4, 3
    V = rng.standard_normal((B, H, S, dv))
    Kc = rng.standard_normal((B, H, S, d))
    # Q = 0: every visible key has the same weight: O = mean of V (causal:
    # prefix means), lse = log(number of visible keys), smax = 0
    Q = np.zeros((B, H, S, d))
    O, lse, smax = oracle.attention_forward(Q, Kc, None, V)
    np.testing.assert_allclose(O[0, :, :], np.broadcast_to(V[0].mean(axis=1, keepdims=True), O[0].shape), atol=1e-15)
    np.testing.assert_allclose(lse, math.log(S), rtol=1e-15)
    assert np.all(smax == 0.0)
    O, lse, _ = oracle.attention_forward(Q, Kc, None, V, causal=True)
    for i in range(S):
        np.testing.assert_allclose(O[0, :, i], V[0, :, :i + 1].mean(axis=1), atol=1e-15)
        np.testing.assert_allclose(lse[0, :, i], math.log(i + 1), rtol=1e-15)
    # causal, square: query 0 sees only key 0
    Q = rng.standard_normal((B, H, S, d))
    O, _, _ = oracle.attention_forward(Q, Kc, None, V, causal=True)
    np.testing.assert_allclose(O[0, :, 0], V[0, :, 0], rtol=1e-15)
    # rows of weights sum to one: V = 1 gives O = 1
    O, _, _ = oracle.attention_forward(Q, Kc, None, np.ones_like(V))
    np.testing.assert_allclose(O, 1.0, rtol=1e-14)


def test_lse_is_logsumexp_and_large_logits_stay_finite(rng):
    Q, Kc, Kr, V = _inputs(rng, 1, 2, 4, 6, 4, 2, 3, scale=30.0)  # logits in the thousands
    O, lse, smax = oracle.attention_forward(Q, Kc, Kr, V)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(lse))
    for h in range(2):
        k = np.concatenate([Kc[0, h], Kr[0]], 1)
        logits = Q[0, h] @ k.T / math.sqrt(6)
        np.testing.assert_allclose(lse[0, h], logsumexp(logits, axis=1), rtol=1e-14)
        assert smax[h] == pytest.approx(logits.max(), rel=1e-14)


def test_causal_with_fewer_queries_than_keys(rng):
    # Sq < Sk: the queries are the last Sq positions; the last query sees all keys
    Q, Kc, Kr, V = _inputs(rng, 1, 1, 3, 7, 4, 0, 2)
    O, _, _ = oracle.attention_forward(Q, Kc, Kr, V, causal=True)
    Of, _, _ = oracle.attention_forward(Q[:, :, -1:], Kc, Kr, V)
    np.testing.assert_allclose(O[:, :, -1:], Of, rtol=1e-14)
    O2, _ = oracle.attention_forward_bruteforce(Q, Kc, Kr, V, causal=True)
    np.testing.assert_allclose(O, O2, rtol=1e-12, atol=1e-12)
