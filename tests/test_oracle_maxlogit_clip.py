"""Pins of the oracle's per-head max logit and QK-Clip (no GPU)."""

import math

import numpy as np
import pytest

import oracle


def _int_inputs(rng, B, H, S, dc, dr):
    Q = rng.integers(-6, 7, (B, H, S, dc + dr)).astype(np.float64)
    Kc = rng.integers(-6, 7, (B, H, S, dc)).astype(np.float64)
    Kr = rng.integers(-6, 7, (B, S, dr)).astype(np.float64) if dr else None
    return Q, Kc, Kr


@pytest.mark.parametrize("dr", [0, 2])
def test_max_logit_equals_bruteforce_bitwise(rng, dr):
    # Integer inputs make every fp64 dot product exact, so the blocked oracle
    # and the pure-Python triple loop must agree bit for bit.
    Q, Kc, Kr = _int_inputs(rng, 2, 3, 8, 4, dr)
    got = oracle.max_logit(Q, Kc, Kr, block=3)
    ref = oracle.max_logit_bruteforce(Q, Kc, Kr)
    np.testing.assert_array_equal(got, ref)


def test_max_logit_uses_shared_rotary_key(rng):
    # Changing only Kr must change the result (it is part of every head's key);
    # dropping it (MHA form) must give the nope-only logits.
    Q, Kc, Kr = _int_inputs(rng, 1, 2, 6, 4, 2)
    full = oracle.max_logit(Q, Kc, Kr)
    Kr2 = Kr.copy()
    Kr2[0, 0] += 50.0
    assert np.all(oracle.max_logit(Q, Kc, Kr2) != full)
    nope = oracle.max_logit(Q[..., :4], Kc, None) * math.sqrt(4) / math.sqrt(6)
    manual = max(float((Q[0, h, :, :4] @ Kc[0, h].T).max()) for h in range(1)) / math.sqrt(6)
    assert nope[0] == pytest.approx(manual, rel=1e-15)


def test_max_logit_closed_form():
    # Q_i = c e_{i}, K_j = c e_{j+1}: the only non-zero logits are c^2 (i = j+1),
    # so S = c^2 / sqrt(d).  With all keys negated every logit is <= 0 and the
    # signed max is 0, not c^2 (no absolute value in the definition).
    d, S, c = 16, 8, 3.0
    Q = np.zeros((1, 1, S, d))
    K = np.zeros((1, 1, S, d))
    for i in range(S):
        Q[0, 0, i, i] = c
        K[0, 0, i, i + 1] = c
    assert oracle.max_logit(Q, K)[0] == c * c / math.sqrt(d)
    assert oracle.max_logit(Q, -K)[0] == 0.0
    Kneg = -np.ones((1, 1, S, d))
    Qpos = np.ones((1, 1, S, d))
    assert oracle.max_logit(Qpos, Kneg)[0] == -d / math.sqrt(d)


def test_max_logit_over_batch_is_max_of_parts(rng):
    Q, Kc, Kr = _int_inputs(rng, 3, 2, 5, 4, 2)
    whole = oracle.max_logit(Q, Kc, Kr)
    parts = np.max([oracle.max_logit(Q[b:b + 1], Kc[b:b + 1], Kr[b:b + 1]) for b in range(3)], axis=0)
    np.testing.assert_array_equal(whole, parts)


def test_max_logit_nan_handling(rng):
    Q, Kc, Kr = _int_inputs(rng, 1, 2, 4, 4, 0)
    clean = oracle.max_logit(Q, Kc, None)
    Qn = Q.copy()
    Qn[0, 0, 1, 2] = np.nan  # one NaN row of logits in head 0 is ignored
    got = oracle.max_logit(Qn, Kc, None)
    assert got[1] == clean[1]
    assert got[0] == oracle.max_logit_bruteforce(Qn, Kc, None)[0]
    Qn[0, 1] = np.nan  # every logit of head 1 is NaN -> -inf
    assert oracle.max_logit(Qn, Kc, None)[1] == -np.inf


# ------------------------------------------------------------------ clip ----
def _mla_weights(rng, H, dc, dr, d_in):
    Wq = rng.standard_normal((H * (dc + dr), d_in))
    Wkc = rng.standard_normal((H * dc, d_in))
    Wkr = rng.standard_normal((dr, d_in))
    return Wq, Wkc, Wkr


def _mla_qk(X, Wq, Wkc, Wkr, H):
    Q = oracle.project_heads(X, Wq, H)
    Kc = oracle.project_heads(X, Wkc, H)
    Kr = oracle.project_heads(X, Wkr, 1)[:, 0]
    return Q, Kc, Kr


def test_clip_brings_clipped_heads_to_tau_mla(rng):
    # S recomputed on the clipped weights (same X, same weights S was measured
    # on) equals tau for clipped heads: every logit of a clipped head is scaled
    # by exactly gamma (sqrt(gamma) sqrt(gamma) on the nope part, gamma x 1 on
    # the rotary part).  Unclipped heads and the shared rotary key are unchanged.
    H, dc, dr, d_in = 4, 8, 4, 16
    X = rng.standard_normal((2, 10, d_in))
    Wq, Wkc, Wkr = _mla_weights(rng, H, dc, dr, d_in)
    Wq[: dc + dr] *= 20.0  # head 0 far over tau
    Wkc[:dc] *= 20.0
    Q, Kc, Kr = _mla_qk(X, Wq, Wkc, Wkr, H)
    S = oracle.max_logit(Q, Kc, Kr)
    tau = float(np.sort(S)[-2]) * 1.5  # only head 0 above tau
    Wq2, Wkc2, gamma, clipped = oracle.qk_clip(S, Wq, Wkc, dc + dr, dc, dc, tau=tau, w_dtype="f64")
    assert list(clipped) == [1, 0, 0, 0]
    Q2, Kc2, Kr2 = _mla_qk(X, Wq2, Wkc2, Wkr, H)
    S2 = oracle.max_logit(Q2, Kc2, Kr2)
    assert S2[0] == pytest.approx(tau, rel=1e-12)
    np.testing.assert_array_equal(S2[1:], S[1:])
    np.testing.assert_array_equal(Wq2[dc + dr:], Wq[dc + dr:])
    np.testing.assert_array_equal(Wkc2[dc:], Wkc[dc:])
    # every logit of head 0 scales by gamma
    full = Q[0, 0] @ np.concatenate([Kc[0, 0], Kr[0]], 1).T
    full2 = Q2[0, 0] @ np.concatenate([Kc2[0, 0], Kr2[0]], 1).T
    np.testing.assert_allclose(full2, gamma[0] * full, rtol=1e-12, atol=1e-12)


def test_clip_exact_when_gamma_is_power_of_four(rng):
    # gamma = 1/4: sqrt(gamma) = 1/2 and gamma are exact, so the clipped weights
    # and the recomputed max are exact in fp64.
    H, dc, dr, d_in = 2, 4, 4, 8
    Wq = rng.integers(-8, 9, (H * (dc + dr), d_in)).astype(np.float64)
    Wkc = rng.integers(-8, 9, (H * dc, d_in)).astype(np.float64)
    smax = np.array([400.0, 50.0])
    Wq2, Wkc2, gamma, clipped = oracle.qk_clip(smax, Wq, Wkc, dc + dr, dc, dc, tau=100.0, w_dtype="f64")
    assert gamma[0] == 0.25 and list(clipped) == [1, 0]
    np.testing.assert_array_equal(Wq2[:dc], Wq[:dc] * 0.5)
    np.testing.assert_array_equal(Wq2[dc:dc + dr], Wq[dc:dc + dr] * 0.25)
    np.testing.assert_array_equal(Wkc2[:dc], Wkc[:dc] * 0.5)
    np.testing.assert_array_equal(Wq2[dc + dr:], Wq[dc + dr:])


def test_clip_mha_general_alpha(rng):
    # MHA: W_q^h x gamma^alpha, W_k^h x gamma^(1-alpha); the logits of head h
    # scale by gamma for any alpha.
    H, dh, d_in = 3, 4, 12
    X = rng.standard_normal((1, 6, d_in))
    Wq = rng.standard_normal((H * dh, d_in))
    Wk = rng.standard_normal((H * dh, d_in))
    smax = np.array([250.0, 80.0, 1000.0])
    for alpha in (0.5, 0.3, 1.0):
        Wq2, Wk2, gamma, clipped = oracle.qk_clip(smax, Wq, Wk, dh, dh, dh, tau=100.0, alpha=alpha,
                                                  w_dtype="f64")
        assert list(clipped) == [1, 0, 1]
        for h in range(H):
            L = oracle.project_heads(X, Wq, H)[0, h] @ oracle.project_heads(X, Wk, H)[0, h].T
            L2 = oracle.project_heads(X, Wq2, H)[0, h] @ oracle.project_heads(X, Wk2, H)[0, h].T
            np.testing.assert_allclose(L2, gamma[h] * L, rtol=1e-12, atol=1e-12)
        np.testing.assert_array_equal(Wq2[dh:2 * dh], Wq[dh:2 * dh])


def test_clip_tie_nan_and_unclipped_bitwise(rng):
    Wq = oracle.round_to_bf16(rng.standard_normal((4 * 6, 8)) * 0.02)
    Wk = oracle.round_to_bf16(rng.standard_normal((4 * 4, 8)) * 0.02)
    smax = np.array([100.0, np.nan, -5.0, 100.0000001])
    Wq2, Wk2, gamma, clipped = oracle.qk_clip(smax, Wq, Wk, 6, 4, 4, tau=100.0)
    assert list(clipped) == [0, -1, 0, 1]  # tie at tau is not clipped; NaN flagged
    np.testing.assert_array_equal(Wq2[:18], Wq[:18])
    np.testing.assert_array_equal(Wk2[:12], Wk[:12])
    assert gamma[3] == 100.0 / 100.0000001


def test_clip_rounds_once_to_bf16(rng):
    Wq = oracle.round_to_bf16(rng.standard_normal((6, 32)) * 0.02)
    Wk = oracle.round_to_bf16(rng.standard_normal((4, 32)) * 0.02)
    smax = np.array([523.25])
    Wq2, Wk2, gamma, _ = oracle.qk_clip(smax, Wq, Wk, 6, 4, 4, tau=100.0)
    g = 100.0 / 523.25
    np.testing.assert_array_equal(Wq2[:4], oracle.round_to_bf16(Wq[:4] * math.sqrt(g)))
    np.testing.assert_array_equal(Wq2[4:], oracle.round_to_bf16(Wq[4:] * g))
    np.testing.assert_array_equal(Wk2, oracle.round_to_bf16(Wk * math.sqrt(g)))


def test_full_step_composition(rng):
    # One step = momentum, NS x scale, decoupled-decay update for every matrix,
    # then QK-Clip on the updated attention weights (Algorithm 1 order).
    H, dh, d_in = 2, 4, 8
    W = {n: oracle.round_to_bf16(rng.standard_normal((H * dh, d_in)) * 0.1) for n in ("q", "k", "v")}
    G = {n: (rng.standard_normal((H * dh, d_in)) * 1e-3).astype(np.float32) for n in W}
    att = dict(q="q", k="k", q_rows_per_head=dh, q_c_rows=dh, k_rows_per_head=dh)
    smax = np.array([300.0, 10.0])
    new_w, new_m, gamma, clipped = oracle.muonclip_step(W, G, {}, smax, att, lr=0.02)
    for n in W:
        np.testing.assert_array_equal(new_m[n], G[n])  # M_0 = 0 -> M_1 = G
    Wv = oracle.apply_update(W["v"], oracle.muon_orthogonalised_update(G["v"].astype(np.float64)), 0.02)
    np.testing.assert_array_equal(new_w["v"], Wv)
    Wq1 = oracle.apply_update(W["q"], oracle.muon_orthogonalised_update(G["q"].astype(np.float64)), 0.02)
    np.testing.assert_array_equal(new_w["q"][:dh], oracle.round_to_bf16(Wq1[:dh] * math.sqrt(1 / 3)))
    np.testing.assert_array_equal(new_w["q"][dh:], Wq1[dh:])
    assert list(clipped) == [1, 0]


def test_full_step_clips_every_layer_with_its_own_max_logits(rng):
    # Two attention layers (Algorithm 1 clips every head of every attention
    # layer).  With eta = 0 the Muon part leaves W bit-unchanged, so the clip
    # acts on the weights S was measured on: recomputed per layer, every
    # clipped head's max logit is tau again and the other heads' rows are
    # untouched.  Layer 0 has head 1 hot, layer 1 head 0: reading the wrong
    # layer's row of S, or clipping only one layer, fails.
    H, dh, d_in, tau = 3, 4, 8, 5.0
    X = rng.standard_normal((2, 6, d_in))
    W, att, S = {}, [], []
    for layer, hot in ((0, 1), (1, 0)):
        Wq = rng.standard_normal((H * dh, d_in)) * 0.3
        Wk = rng.standard_normal((H * dh, d_in)) * 0.3
        Wq[hot * dh:(hot + 1) * dh] *= 6.0
        Wk[hot * dh:(hot + 1) * dh] *= 6.0
        W[f"q{layer}"], W[f"k{layer}"] = Wq, Wk
        att.append(dict(q=f"q{layer}", k=f"k{layer}", q_rows_per_head=dh, q_c_rows=dh, k_rows_per_head=dh))
        S.append(oracle.max_logit(oracle.project_heads(X, Wq, H), oracle.project_heads(X, Wk, H)))
    S = np.stack(S)
    assert S[0, 1] > tau and S[1, 0] > tau and S[0, 0] < tau and S[1, 1] < tau
    G = {n: np.zeros(w.shape, dtype=np.float32) for n, w in W.items()}
    new_w, _, gamma, clipped = oracle.muonclip_step(W, G, {}, S, att, lr=0.0, tau=tau, w_dtype="f64")
    assert gamma.shape == clipped.shape == (2, H)
    np.testing.assert_array_equal(clipped, (S > tau).astype(np.int32))
    for layer in range(2):
        Wq2, Wk2 = new_w[f"q{layer}"], new_w[f"k{layer}"]
        S2 = oracle.max_logit(oracle.project_heads(X, Wq2, H), oracle.project_heads(X, Wk2, H))
        for h in range(H):
            rows = slice(h * dh, (h + 1) * dh)
            if S[layer, h] > tau:
                assert S2[h] == pytest.approx(tau, rel=1e-12)
            else:
                np.testing.assert_array_equal(Wq2[rows], W[f"q{layer}"][rows])
                np.testing.assert_array_equal(Wk2[rows], W[f"k{layer}"][rows])


def test_full_step_stacked_matrices_are_separate_matrices(rng):
    # A stack [count, rows, cols] is count independent Muon matrices.
    W = {"e": oracle.round_to_bf16(rng.standard_normal((3, 8, 16)) * 0.1),
         "q": oracle.round_to_bf16(rng.standard_normal((8, 16)) * 0.1),
         "k": oracle.round_to_bf16(rng.standard_normal((8, 16)) * 0.1)}
    G = {n: (rng.standard_normal(w.shape) * 1e-3).astype(np.float32) for n, w in W.items()}
    att = dict(q="q", k="k", q_rows_per_head=4, q_c_rows=4, k_rows_per_head=4)
    new_w, _, _, _ = oracle.muonclip_step(W, G, {}, np.array([1.0, 1.0]), att, lr=0.02)
    for i in range(3):
        one, _, _, _ = oracle.muonclip_step({"e": W["e"][i], "q": W["q"], "k": W["k"]},
                                            {"e": G["e"][i], "q": G["q"], "k": G["k"]}, {}, np.array([1.0, 1.0]),
                                            att, lr=0.02)
        np.testing.assert_array_equal(new_w["e"][i], one["e"])


# ------------------------------------------------------------- total clip ----
def test_total_clip_brings_the_largest_head_to_tau_and_scales_all_heads(rng):
    # Total clip: one gamma = tau / max_h S^h for every head.  Recomputed on the
    # clipped weights, the largest head max equals tau, every head's logits
    # (so every S^h) scale by the same gamma, and the shared rotary key stays.
    H, dc, dr, d_in = 4, 8, 4, 16
    X = rng.standard_normal((2, 10, d_in))
    Wq, Wkc, Wkr = _mla_weights(rng, H, dc, dr, d_in)
    Wq[(dc + dr):2 * (dc + dr)] *= 20.0  # head 1 far over tau
    Wkc[dc:2 * dc] *= 20.0
    Q, Kc, Kr = _mla_qk(X, Wq, Wkc, Wkr, H)
    S = oracle.max_logit(Q, Kc, Kr)
    tau = float(np.sort(S)[-2]) * 1.5  # only head 1 above tau
    Wq2, Wkc2, gamma, clipped = oracle.qk_clip_total(S, Wq, Wkc, dc + dr, dc, dc, tau=tau, w_dtype="f64")
    assert list(clipped) == [1, 1, 1, 1]
    assert np.all(gamma == tau / S.max())
    Q2, Kc2, Kr2 = _mla_qk(X, Wq2, Wkc2, Wkr, H)
    S2 = oracle.max_logit(Q2, Kc2, Kr2)
    assert S2.max() == pytest.approx(tau, rel=1e-12)
    np.testing.assert_allclose(S2, gamma * S, rtol=1e-12)
    np.testing.assert_array_equal(Kr2, Kr)
    for h in range(H):
        full = Q[0, h] @ np.concatenate([Kc[0, h], Kr[0]], 1).T
        full2 = Q2[0, h] @ np.concatenate([Kc2[0, h], Kr2[0]], 1).T
        np.testing.assert_allclose(full2, gamma[h] * full, rtol=1e-12, atol=1e-12)


def test_total_clip_below_tau_nan_and_single_head(rng):
    Wq = oracle.round_to_bf16(rng.standard_normal((4 * 6, 8)) * 0.02)
    Wk = oracle.round_to_bf16(rng.standard_normal((4 * 4, 8)) * 0.02)
    # largest head exactly at tau: nothing touched (strict >), bit for bit
    Wq2, Wk2, gamma, clipped = oracle.qk_clip_total(np.array([100.0, 3.0, -5.0, 99.0]), Wq, Wk, 6, 4, 4)
    assert list(clipped) == [0] * 4 and np.all(gamma == 1.0)
    np.testing.assert_array_equal(Wq2, Wq)
    np.testing.assert_array_equal(Wk2, Wk)
    # a NaN head is skipped in the max; gamma = 1/4 makes the result exact
    Wq2, Wk2, gamma, clipped = oracle.qk_clip_total(np.array([np.nan, 400.0, 3.0, 50.0]), Wq, Wk, 6, 4, 4,
                                                    w_dtype="f64")
    assert list(clipped) == [1] * 4 and np.all(gamma == 0.25)
    for h in range(4):
        np.testing.assert_array_equal(Wq2[6 * h:6 * h + 4], Wq[6 * h:6 * h + 4] * 0.5)
        np.testing.assert_array_equal(Wq2[6 * h + 4:6 * h + 6], Wq[6 * h + 4:6 * h + 6] * 0.25)
        np.testing.assert_array_equal(Wk2[4 * h:4 * h + 4], Wk[4 * h:4 * h + 4] * 0.5)
    # every head NaN: nothing touched, flagged
    Wq2, Wk2, gamma, clipped = oracle.qk_clip_total(np.full(4, np.nan), Wq, Wk, 6, 4, 4)
    assert list(clipped) == [-1] * 4
    np.testing.assert_array_equal(Wq2, Wq)
    # one head: total clip is per-head clip
    a = oracle.qk_clip_total(np.array([523.25]), Wq[:6], Wk[:4], 6, 4, 4)
    b = oracle.qk_clip(np.array([523.25]), Wq[:6], Wk[:4], 6, 4, 4)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


# ------------------------------------------------------- rotary q^R, k^R ----
def _rotate_pairs(x, positions, base=10000.0):
    # a position-dependent rotation of consecutive pairs (RoPE-style); any
    # orthogonal map per position serves the invariance below
    d = x.shape[-1]
    freq = base ** (-np.arange(0, d, 2) / d)
    ang = positions[:, None] * freq[None, :]
    c, s = np.cos(ang), np.sin(ang)
    out = np.empty_like(x)
    out[..., 0::2] = x[..., 0::2] * c - x[..., 1::2] * s
    out[..., 1::2] = x[..., 0::2] * s + x[..., 1::2] * c
    return out


def test_clip_with_rotated_rotary_parts(rng):
    # The rotary parts q^R and k^R are rotated by position before the logits.
    # The rotation is linear, so scaling W_qr by gamma scales every rotated
    # q^R by gamma, and the clipped head's recomputed max is tau again; the
    # rotation lives upstream of the max logit (it rotates its inputs).
    H, dc, dr, d_in, S_len = 3, 8, 4, 16, 12
    X = rng.standard_normal((2, S_len, d_in))
    Wq, Wkc, Wkr = _mla_weights(rng, H, dc, dr, d_in)
    Wq[:dc + dr] *= 20.0
    Wkc[:dc] *= 20.0
    pos = np.arange(S_len, dtype=np.float64)

    def rotated(Wq_, Wkc_):
        Q, Kc, Kr = _mla_qk(X, Wq_, Wkc_, Wkr, H)
        Q = Q.copy()
        Q[..., dc:] = _rotate_pairs(Q[..., dc:], pos)
        return Q, Kc, _rotate_pairs(Kr, pos)

    Q, Kc, Kr = rotated(Wq, Wkc)
    S = oracle.max_logit(Q, Kc, Kr)
    tau = float(np.sort(S)[-2]) * 1.5
    Wq2, Wkc2, gamma, clipped = oracle.qk_clip(S, Wq, Wkc, dc + dr, dc, dc, tau=tau, w_dtype="f64")
    assert list(clipped) == [1, 0, 0]
    S2 = oracle.max_logit(*rotated(Wq2, Wkc2))
    assert S2[0] == pytest.approx(tau, rel=1e-12)
    np.testing.assert_array_equal(S2[1:], S[1:])
