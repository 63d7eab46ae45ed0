"""GPU parity of the attention forward with the max logit as a by-product
(``attention_fwd_maxlogit``) against the fp64 oracle, through the C ABI.

Tolerances, from the arithmetic: the logits and the row sums are float32
sums of exact bf16 products (relative error ~1e-6); the softmax weights p_j
are rounded to bf16 (2^-9 relative) before the second product, and O is
rounded once to bf16 (2^-9 relative), so per element
    |O - O_ref| <= 2^-9 (sum_j p_j |V_j| + |O_ref|) + float32 noise,
with p the exact softmax row.  The tests assert twice that,
2^-8 (sum_j p_j |V_j| + |O_ref|) + 1e-6, element by element (p from the
oracle's logits and log-sum-exp).  S_max relative error <= 1e-3 (the bound
stated for bf16 inputs is 1e-2), log-sum-exp absolute error <= 1e-3.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import f64, rel_err, say

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def mc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import muonclip_muon_amd
    return muonclip_muon_amd


def _inputs(seed, B, H, Sq, Sk, dc, dr, dv, scale=1.0):
    g = workloads.generator(seed, "cpu")
    Q = workloads.normal((B, H, Sq, dc + dr), scale, g, "cpu", torch.bfloat16)
    Kc = workloads.normal((B, H, Sk, dc), scale, g, "cpu", torch.bfloat16)
    Kr = workloads.normal((B, Sk, dr), scale, g, "cpu", torch.bfloat16) if dr else None
    V = workloads.normal((B, H, Sk, dv), 1.0, g, "cpu", torch.bfloat16)
    return Q, Kc, Kr, V


def _o_bound(Q, Kc, Kr, V, causal, rO, rlse):
    """Per-element bound 2^-8 (sum_j p_j |V_j| + |O_ref|) + 1e-6, with p the
    exact softmax weights exp(L - lse) of the oracle's log-sum-exp."""
    a = lambda x: x if isinstance(x, np.ndarray) else f64(x)  # noqa: E731
    Q, Kc, V = a(Q), a(Kc), a(V)
    K = Kc if Kr is None else np.concatenate(
        [Kc, np.broadcast_to(a(Kr)[:, None], (Kc.shape[0], Kc.shape[1]) + a(Kr).shape[1:])], axis=-1)
    L = Q @ np.swapaxes(K, -1, -2) / math.sqrt(Q.shape[-1])
    if causal:
        Sq, Sk = L.shape[-2], L.shape[-1]
        L = np.where(np.arange(Sk)[None, :] <= np.arange(Sq)[:, None] + (Sk - Sq), L, -np.inf)
    P = np.exp(L - rlse[..., None])
    return 2.0 ** -8 * (P @ np.abs(V) + np.abs(rO)) + 1e-6


def _check(mc, Q, Kc, Kr, V, causal):
    B, H, Sq, _ = Q.shape
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=DEV)
    O, smax = mc.attention_fwd_maxlogit(Q.to(DEV), Kc.to(DEV), Kr.to(DEV) if Kr is not None else None, V.to(DEV),
                                        causal=causal, lse=lse)
    torch.cuda.synchronize()
    rO, rlse, rsmax = oracle.attention_forward(f64(Q), f64(Kc), f64(Kr) if Kr is not None else None, f64(V), causal)
    err = np.abs(f64(O) - rO)
    bound = _o_bound(Q, Kc, Kr, V, causal, rO, rlse)
    assert np.all(err <= bound), float((err / bound).max())
    assert rel_err(smax.cpu().numpy(), rsmax).max() <= 1e-3
    assert np.abs(f64(lse) - rlse).max() <= 1e-3
    return O, smax


ATTENTION_CASES = [
    # B, H, Sq, Sk, d_c, d_r, d_v, causal, scale
    (1, 2, 256, 256, 64, 0, 64, False, 1.0),     # one workgroup row block, 4 key blocks
    (2, 3, 300, 200, 64, 0, 64, False, 1.0),     # ragged rows (duplicated tail) and keys (shifted last block)
    (1, 2, 200, 200, 64, 0, 64, True, 1.0),      # causal, square
    (1, 2, 100, 300, 64, 0, 64, True, 1.0),      # causal, queries are the last 100 of 300 positions
    (1, 1, 5, 70, 64, 0, 64, False, 1.0),        # last block shifted by 58: one phase wholly masked
    (1, 2, 320, 128, 128, 64, 128, False, 1.0),  # the MLA head (128 + shared 64, d_v 128)
    (2, 2, 256, 320, 128, 64, 128, True, 1.0),
    (1, 1, 64, 64, 128, 64, 128, True, 1.0),
    (1, 2, 130, 260, 128, 64, 128, False, 3.0),  # logits of std ~9: the reference point moves often
]


@pytest.mark.parametrize("case", ATTENTION_CASES)
def test_attention_fwd(mc, case):
    B, H, Sq, Sk, dc, dr, dv, causal, scale = case
    say("attention", case)
    Q, Kc, Kr, V = _inputs(hash(case) % 1000, B, H, Sq, Sk, dc, dr, dv, scale)
    _check(mc, Q, Kc, Kr, V, causal)


def test_attention_hot_head_and_max_logit_agree(mc):
    """One head's logits ~500 (a clipped head): softmax stays exact, and S_max
    equals the stand-alone max-logit kernel's."""
    say("attention hot head")
    Q, Kc, Kr, V = _inputs(77, 2, 3, 192, 256, 128, 64, 128)
    Q[:, 1] *= 12.0
    Kc[:, 1] *= 12.0
    O, smax = _check(mc, Q, Kc, Kr, V, False)
    s2 = mc.qk_maxlogit(Q.to(DEV), Kc.to(DEV), Kr.to(DEV)).cpu().numpy()
    assert rel_err(smax.cpu().numpy(), s2).max() <= 1e-5
    assert smax[1].item() > 100.0


def test_attention_accumulate_over_batch_split(mc):
    say("attention batch split")
    Q, Kc, Kr, V = _inputs(78, 2, 2, 128, 128, 64, 0, 64)
    smax = torch.empty(2, dtype=torch.float32, device=DEV)
    mc.attention_fwd_maxlogit(Q[:1].to(DEV), Kc[:1].to(DEV), None, V[:1].to(DEV), smax=smax)
    mc.attention_fwd_maxlogit(Q[1:].to(DEV), Kc[1:].to(DEV), None, V[1:].to(DEV), smax=smax, accumulate=True)
    _, _, ref = oracle.attention_forward(f64(Q), f64(Kc), None, f64(V))
    assert rel_err(smax.cpu().numpy(), ref).max() <= 1e-3


def test_attention_rejects_unsupported(mc):
    Q, Kc, Kr, V = _inputs(79, 1, 1, 64, 32, 64, 0, 64)
    with pytest.raises(mc.MuonClipError):  # fewer than 64 keys
        mc.attention_fwd_maxlogit(Q.to(DEV), Kc.to(DEV), None, V.to(DEV))
    Q, Kc, Kr, V = _inputs(79, 1, 1, 128, 64, 64, 0, 64)
    with pytest.raises(mc.MuonClipError):  # causal with more queries than keys
        mc.attention_fwd_maxlogit(Q.to(DEV), Kc.to(DEV), None, V.to(DEV), causal=True)


@pytest.mark.parametrize("causal", [False, True])
def test_attention_fullsize_8x4096(mc, causal):
    """Kimi K2's MLA head at the max-logit workload's size (8 x 4096 tokens, 64
    heads, q/k 128 + 64 through the projections, one hot head set): S_max of
    every head against the stand-alone kernel (same logits, pinned against the
    oracle at this size) and, when not causal, the oracle's heads; O and LSE on
    sampled rows against the oracle row by row."""
    say("full size attention", causal)
    L = workloads.mla_logits(seed=3, device=DEV)
    g = workloads.generator(3 + 3000, DEV)
    V = workloads.normal((8, 64, 4096, 128), 1.0, g, DEV, torch.bfloat16)
    lse = torch.empty((8, 64, 4096), dtype=torch.float32, device=DEV)
    O, smax = mc.attention_fwd_maxlogit(L.Q, L.Kc, L.Kr, V, causal=causal, lse=lse)
    s = smax.cpu().numpy()
    if not causal:
        s2 = mc.qk_maxlogit(L.Q, L.Kc, L.Kr).cpu().numpy()
        assert rel_err(s, s2).max() <= 1e-5
        for h in (0, int(L.hot[0])):
            ref = oracle.max_logit(f64(L.Q[:, h:h + 1]), f64(L.Kc[:, h:h + 1]), f64(L.Kr))[0]
            assert rel_err(s[h], ref) <= 1e-3
        assert sorted(np.nonzero(s > 100.0)[0].tolist()) == sorted(L.hot.tolist())
    rng = np.random.default_rng(5)
    for b, h, i in zip(rng.integers(0, 8, 6), rng.integers(0, 64, 6), rng.integers(0, 4096, 6)):
        b, h, i = int(b), int(h), int(i)
        i = i if not causal else max(i, 1)
        Sk = 4096 if not causal else i + 1
        q = f64(L.Q[b:b + 1, h:h + 1, i:i + 1])
        kc = f64(L.Kc[b:b + 1, h:h + 1, :Sk])
        kr = f64(L.Kr[b:b + 1, :Sk])
        v = f64(V[b:b + 1, h:h + 1, :Sk])
        rO, rlse, rs = oracle.attention_forward(q, kc, kr, v)
        bound = _o_bound(q, kc, kr, v, False, rO, rlse)
        assert np.all(np.abs(f64(O[b, h, i]) - rO[0, 0, 0]) <= bound[0, 0, 0])
        assert abs(float(lse[b, h, i]) - rlse[0, 0, 0]) <= 1e-3
        assert rs[0] <= s[h] * (1 + 1e-3) + 1e-6
