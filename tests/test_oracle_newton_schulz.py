"""Pins of the oracle's Newton-Schulz orthogonalisation and update (no GPU).

Each pin ties the oracle to something other than itself: the SVD closed form
of an odd matrix polynomial (LAPACK), the polar factor U V^T of a full-rank
matrix (LAPACK), orthogonal invariance, and exact special cases.
"""

import numpy as np
import pytest

import oracle


def _spectral_form(M, coeffs, eps=oracle.NS_EPS):
    """U diag(p(sigma / (||M||_F + eps))) V^T from LAPACK's SVD."""
    U, s, Vt = np.linalg.svd(np.asarray(M, dtype=np.float64), full_matrices=False)
    nrm = np.sqrt(np.sum(s ** 2))  # ||M||_F from the singular values
    return (U * oracle.ns_polynomial_scalar(s / (nrm + eps), coeffs)) @ Vt


@pytest.mark.parametrize("shape", [(64, 64), (48, 168), (168, 48), (1, 40), (40, 1), (96, 97)])
def test_ns_equals_svd_closed_form(rng, shape):
    M = rng.standard_normal(shape)
    got = oracle.newton_schulz(M)
    ref = _spectral_form(M, oracle.NS_COEFFS)
    assert np.linalg.norm(got - ref) <= 1e-12 * np.linalg.norm(ref)


def test_ns_closed_form_catches_a_wrong_coefficient(rng):
    # The closed form is sensitive to each coefficient and to the order of the
    # polynomial terms: a swapped b/c gives a clearly different matrix.
    M = rng.standard_normal((32, 80))
    a, b, c = oracle.NS_COEFFS[0]
    swapped = ((a, c, b),) * oracle.NS_STEPS
    assert np.linalg.norm(oracle.newton_schulz(M, swapped) - _spectral_form(M, oracle.NS_COEFFS)) > 1e-2


def test_ns_cubic_converges_to_polar_factor(rng):
    # The textbook cubic (1.5, -0.5) converges to U V^T for a full-rank input
    # whose singular values, after the Frobenius pre-scale, lie in (0, sqrt(3)).
    U, _ = np.linalg.qr(rng.standard_normal((12, 12)))
    V, _ = np.linalg.qr(rng.standard_normal((20, 12)))
    s = np.linspace(1.0, 3.0, 12)
    M = (U * s) @ V.T
    got = oracle.newton_schulz(M, ((1.5, -0.5, 0.0),) * 40)
    Uf, _, Vtf = np.linalg.svd(M, full_matrices=False)
    assert np.max(np.abs(got - Uf @ Vtf)) <= 1e-12


def test_ns_symmetries(rng):
    M = rng.standard_normal((24, 56))
    O = oracle.newton_schulz(M)
    np.testing.assert_allclose(oracle.newton_schulz(-M), -O, rtol=0, atol=1e-13)
    np.testing.assert_allclose(oracle.newton_schulz(M.T), O.T, rtol=0, atol=1e-13)
    P, _ = np.linalg.qr(rng.standard_normal((24, 24)))
    R, _ = np.linalg.qr(rng.standard_normal((56, 56)))
    np.testing.assert_allclose(oracle.newton_schulz(P @ M @ R), P @ O @ R, rtol=0, atol=1e-12)
    # scale invariance: exact with eps = 0; with eps the pre-scale differs by
    # about eps / ||M||_F (2.7e-9 relative here), amplified at most ~5x per step
    O0 = oracle.newton_schulz(M, eps=0.0)
    np.testing.assert_allclose(oracle.newton_schulz(1e3 * M, eps=0.0), O0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(oracle.newton_schulz(1e3 * M), O, rtol=0, atol=1e-8)


def test_ns_zero_and_orthonormal_rows(rng):
    assert np.all(oracle.newton_schulz(np.zeros((8, 16))) == 0.0)
    Q, _ = np.linalg.qr(rng.standard_normal((30, 10)))
    Q = Q.T  # 10 x 30 with orthonormal rows: every singular value is 1, ||Q||_F = sqrt(10)
    expect = oracle.ns_polynomial_scalar(1.0 / (np.sqrt(10.0) + oracle.NS_EPS)) * Q
    np.testing.assert_allclose(oracle.newton_schulz(Q), expect, rtol=0, atol=1e-13)


def test_quintic_band():
    # Singular values are moved close to 1: after 5 steps of the fixed quintic,
    # every normalised singular value >= 1e-2 lands in [0.68, 1.14], one at
    # >= 3e-3 in [0.68, 1.21].  Checked on a dense grid of the scalar map.
    s = np.linspace(1e-2, 1.0, 200_001)
    p = oracle.ns_polynomial_scalar(s)
    assert 0.68 <= p.min() and p.max() <= 1.135
    s = np.linspace(3e-3, 1.0, 200_001)
    p = oracle.ns_polynomial_scalar(s)
    assert 0.68 <= p.min() and p.max() <= 1.21
    # p(1) is not 1: 1 is not a fixed point of the quintic
    assert abs(oracle.ns_polynomial_scalar(1.0, oracle.NS_COEFFS[:1]) - 0.701) < 1e-3


def test_rms_match_factor(rng):
    # O = NS(M) sqrt(max(n,m)) 0.2 has RMS 0.2 ||NS(M)||_F / sqrt(min(n,m)); with
    # every singular value of NS(M) in the band above, the RMS is 0.2 x [0.68, 1.14].
    M = rng.standard_normal((128, 448))  # the 2048 x 7168 expert aspect ratio
    O = oracle.muon_orthogonalised_update(M)
    rms = np.sqrt(np.mean(O ** 2))
    assert 0.2 * 0.68 <= rms <= 0.2 * 1.14
    sv = np.linalg.svd(oracle.newton_schulz(M), compute_uv=False)
    assert sv.min() >= 0.68 and sv.max() <= 1.14


def test_update_special_cases(rng):
    W = oracle.round_to_bf16(rng.standard_normal((16, 32)) * 0.02)
    O = rng.standard_normal((16, 32)) * 0.2
    np.testing.assert_array_equal(oracle.apply_update(W, O, lr=0.0), W)  # eta = 0: bit-unchanged
    got = oracle.apply_update(W, np.zeros_like(W), lr=2e-4, weight_decay=0.1)
    np.testing.assert_array_equal(got, oracle.round_to_bf16(W * (1 - 2e-4 * 0.1)))
    got = oracle.apply_update(W, O, lr=0.02, weight_decay=0.0, w_dtype="f64")
    np.testing.assert_allclose(got, W - 0.02 * O, rtol=1e-15, atol=0)
