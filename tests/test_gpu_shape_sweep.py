"""Seeded random shapes against the oracle: the Newton-Schulz call, the fused
step, the max logit and the attention forward.

The hand-picked cases in the other files cover each kernel's paths on
purpose. This sweep draws shapes at random, log-uniformly, once from a fixed
seed, so that ragged tails, tile counts and batch sizes no one chose also
meet the oracle. The draw is the same on every run, so every case has a
fixed id. Tolerances are those of the other tests.
- Newton-Schulz relative Frobenius error <= 2e-2, with min(rows, cols) >= 16:
  below that every bf16 chain sits near the tolerance.
- The fused step: momentum bit-exact and the change of W within 2e-2, at
  lr 1, so that the update and not W's rounding dominates.
- The max logit: <= 1e-2 relative for bf16 and <= 1e-5 for float32.
- The attention forward: the per-element bound derived in
  test_gpu_attention.py.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import f64, rel_err, rel_fro, say
from test_gpu_attention import _check as attention_check
from test_gpu_attention import _inputs as attention_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda"
DTYPES = (torch.float32, torch.bfloat16)


def _logu(rng, lo, hi):
    return int(round(float(np.exp(rng.uniform(np.log(lo), np.log(hi))))))


def _ns_cases(seed=90210, count=12):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(count):
        n = _logu(rng, 16, 700)
        m = max(n, _logu(rng, n, 1500))
        rows, cols = (n, m) if rng.random() < 0.5 else (m, n)
        cases.append((int(rng.integers(1, 3)), rows, cols, int(rng.integers(2)), int(rng.integers(2))))
    return cases


def _fused_cases(seed=90211, count=6):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(count):
        n = _logu(rng, 16, 600)
        m = max(n, _logu(rng, n, 1200))
        rows, cols = (n, m) if rng.random() < 0.5 else (m, n)
        cases.append((int(rng.integers(1, 3)), rows, cols, int(rng.integers(2))))
    return cases


MAXLOGIT_HEADS = [(128, 64), (64, 0), (128, 0), (192, 0), (64, 64), (96, 32), (40, 0)]


def _maxlogit_cases(seed=90212, count=10):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(count):
        dc, dr = MAXLOGIT_HEADS[i % len(MAXLOGIT_HEADS)]
        f32 = i % 5 == 4
        # every other case with at least one key block of 64 (the MFMA kernel for its head shapes)
        sk = _logu(rng, 64, 1200) if i % 2 == 0 else _logu(rng, 1, 200)
        cases.append((int(rng.integers(1, 4)), int(rng.integers(1, 5)), _logu(rng, 1, 1200), sk, dc, dr, f32))
    return cases


def _attention_cases(seed=90213, count=8):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(count):
        dc, dr, dv = ((128, 64, 128), (64, 0, 64))[i % 2]
        causal = bool(rng.integers(2))
        sk = _logu(rng, 64, 600)
        sq = _logu(rng, 1, sk) if causal else _logu(rng, 1, 600)
        cases.append((int(rng.integers(1, 3)), int(rng.integers(1, 4)), sq, sk, dc, dr, dv, causal))
    return cases


@pytest.fixture(scope="module")
def mc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import muonclip_muon_amd
    return muonclip_muon_amd


@pytest.mark.parametrize("case", _ns_cases())
def test_sweep_newton_schulz(mc, case):
    batch, rows, cols, mi, oi = case
    say("sweep newton-schulz", case)
    g = workloads.generator(rows * 7 + cols, "cpu")
    M = workloads.normal((batch, rows, cols), 1e-3, g, "cpu", DTYPES[mi])
    O = mc.muon_ns_orthogonalize_batched(M.to(DEV), out_scale=mc.muon_out_scale(rows, cols), out_dtype=DTYPES[oi])
    torch.cuda.synchronize()
    for b in range(batch):
        err = rel_fro(f64(O[b]), oracle.muon_orthogonalised_update(f64(M[b])))
        assert err <= 2e-2, (b, err)


@pytest.mark.parametrize("case", _fused_cases())
def test_sweep_fused_step(mc, case):
    batch, rows, cols, wi = case
    say("sweep fused step", case)
    g = workloads.generator(rows * 11 + cols, "cpu")
    M0 = workloads.normal((batch, rows, cols), 1e-3, g, "cpu")
    G = workloads.normal((batch, rows, cols), 1e-3, g, "cpu")
    W0 = workloads.normal((batch, rows, cols), 0.02, g, "cpu", DTYPES[wi])
    M, W = M0.to(DEV), W0.to(DEV)
    mc.muon_momentum_ns_update_batched(M, G.to(DEV), W, 1.0)
    torch.cuda.synchronize()
    wname = "bf16" if DTYPES[wi] == torch.bfloat16 else "f32"
    for b in range(batch):
        m_ref = np.asarray(oracle.momentum_update(M0[b].numpy(), G[b].numpy(), 0.95), np.float32)
        assert np.array_equal(M[b].cpu().numpy().view(np.int32), m_ref.view(np.int32))
        w_ref = oracle.apply_update(f64(W0[b]), oracle.muon_orthogonalised_update(m_ref.astype(np.float64)), 1.0,
                                    0.1, wname)
        err = rel_fro(f64(W[b]) - f64(W0[b]), np.asarray(w_ref, np.float64) - f64(W0[b]))
        assert err <= 2e-2, (b, err)


@pytest.mark.parametrize("case", _maxlogit_cases())
def test_sweep_max_logit(mc, case):
    B, H, Sq, Sk, dc, dr, f32 = case
    say("sweep max logit", case)
    dt = torch.float32 if f32 else torch.bfloat16
    g = workloads.generator(Sq * 13 + Sk, "cpu")
    Q = workloads.normal((B, H, Sq, dc + dr), 1.0, g, "cpu", dt)
    Kc = workloads.normal((B, H, Sk, dc), 1.0, g, "cpu", dt)
    Kr = workloads.normal((B, Sk, dr), 1.0, g, "cpu", dt) if dr else None
    s = mc.qk_maxlogit(Q.to(DEV), Kc.to(DEV), Kr.to(DEV) if dr else None)
    torch.cuda.synchronize()
    ref = oracle.max_logit(f64(Q), f64(Kc), f64(Kr) if dr else None)
    assert rel_err(s.cpu().numpy(), ref).max() <= (1e-5 if f32 else 1e-2)


@pytest.mark.parametrize("case", _attention_cases())
def test_sweep_attention(mc, case):
    B, H, Sq, Sk, dc, dr, dv, causal = case
    say("sweep attention", case)
    Q, Kc, Kr, V = attention_inputs(Sq * 17 + Sk, B, H, Sq, Sk, dc, dr, dv)
    attention_check(mc, Q, Kc, Kr, V, causal)
