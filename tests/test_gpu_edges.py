"""Empty and degenerate calls through the binding on the GPU.

Zero-element momentum and update, an empty Newton-Schulz batch (alone and
fused), a matrix with no rows (rejected), 1 x 1 matrices (including M = 0),
the max logit and the attention forward with no batch, query or key rows,
and the clip with no heads or no layers.  Each returns without touching any
tensor, with outputs of the right (possibly empty) shape; where the oracle
defines the result (the 1 x 1 matrices, a head that sees no logit = -inf,
the attention forward of an empty batch) the two agree.  The page-level step
with no matrices and no attention layer is a no-op.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import rel_fro, say

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def mc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import muonclip_muon_amd
    return muonclip_muon_amd


def test_empty_elementwise(mc):
    say("empty momentum and update")
    M, G = torch.empty(0, device=DEV), torch.empty(0, device=DEV)
    assert mc.muonclip_momentum(M, G, 0.95).numel() == 0
    W, O = torch.empty(0, dtype=torch.bfloat16, device=DEV), torch.empty(0, dtype=torch.bfloat16, device=DEV)
    assert mc.muon_apply_update(W, O, 2e-4).numel() == 0
    torch.cuda.synchronize()


@pytest.mark.parametrize("rows,cols", [(64, 128), (300, 20)])
def test_empty_newton_schulz_batch(mc, rows, cols):
    say("empty batch", rows, cols)
    M = torch.empty(0, rows, cols, device=DEV)
    O = mc.muon_ns_orthogonalize_batched(M)
    assert O.shape == (0, rows, cols)
    G = torch.empty(0, rows, cols, device=DEV)
    W = torch.empty(0, rows, cols, dtype=torch.bfloat16, device=DEV)
    assert mc.muon_momentum_ns_update_batched(M, G, W, 2e-4).shape == (0, rows, cols)
    torch.cuda.synchronize()


def test_matrix_without_rows_is_rejected(mc):
    say("0 x 128 matrix")
    with pytest.raises(mc.MuonClipError):
        mc.muon_ns_orthogonalize_batched(torch.empty(0, 128, device=DEV))


@pytest.mark.parametrize("value", [3.0, -2.0, 1e-30, 0.0])
def test_newton_schulz_one_by_one(mc, value):
    """X_0 = m / (|m| + eps) is +-1 (or 0), so O = p(...p(sign m)) on one value."""
    say("1 x 1 matrix", value)
    M = torch.full((1, 1), value, device=DEV)
    O = mc.muon_ns_orthogonalize_batched(M, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.newton_schulz(np.array([[value]], dtype=np.float64))
    if value == 0.0:
        assert O.item() == 0.0
    else:
        assert rel_fro(O.cpu().double().numpy(), ref) <= 2e-2


def test_maxlogit_without_rows_or_keys(mc):
    say("max logit: empty batch, queries, keys, heads")
    for B, H, Sq, Sk in ((0, 4, 16, 64), (1, 4, 0, 64), (1, 4, 16, 0)):
        Q = torch.empty(B, H, Sq, 192, dtype=torch.bfloat16, device=DEV)
        Kc = torch.empty(B, H, Sk, 128, dtype=torch.bfloat16, device=DEV)
        Kr = torch.empty(B, Sk, 64, dtype=torch.bfloat16, device=DEV)
        smax = mc.qk_maxlogit(Q, Kc, Kr)
        torch.cuda.synchronize()
        # no logit in any head: the oracle's max over nothing
        assert torch.all(smax == -float("inf")), (B, H, Sq, Sk)
        # accumulate keeps what an earlier call found
        prior = torch.tensor([1.0, -2.0, 300.0, float("-inf")], device=DEV)
        out = mc.qk_maxlogit(Q, Kc, Kr, smax=prior.clone(), accumulate=True)
        torch.cuda.synchronize()
        assert torch.equal(out, prior)
    Q = torch.empty(1, 0, 16, 192, dtype=torch.bfloat16, device=DEV)
    Kc = torch.empty(1, 0, 64, 128, dtype=torch.bfloat16, device=DEV)
    Kr = torch.empty(1, 64, 64, dtype=torch.bfloat16, device=DEV)
    assert mc.qk_maxlogit(Q, Kc, Kr).numel() == 0


def test_attention_without_query_rows(mc):
    say("attention: empty batch and queries")
    for B, Sq in ((0, 32), (1, 0)):
        Q = torch.empty(B, 4, Sq, 192, dtype=torch.bfloat16, device=DEV)
        Kc = torch.empty(B, 4, 64, 128, dtype=torch.bfloat16, device=DEV)
        Kr = torch.empty(B, 64, 64, dtype=torch.bfloat16, device=DEV)
        V = torch.empty(B, 4, 64, 128, dtype=torch.bfloat16, device=DEV)
        lse = torch.empty(B, 4, Sq, device=DEV)
        O, smax = mc.attention_fwd_maxlogit(Q, Kc, Kr, V, lse=lse)
        torch.cuda.synchronize()
        assert O.shape == (B, 4, Sq, 128) and torch.all(smax == -float("inf"))
    # queries but no keys: the softmax is undefined, the call is rejected
    Q = torch.zeros(1, 4, 8, 192, dtype=torch.bfloat16, device=DEV)
    Kc = torch.empty(1, 4, 0, 128, dtype=torch.bfloat16, device=DEV)
    Kr = torch.empty(1, 0, 64, dtype=torch.bfloat16, device=DEV)
    V = torch.empty(1, 4, 0, 128, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(mc.MuonClipError):
        mc.attention_fwd_maxlogit(Q, Kc, Kr, V)


def test_clip_without_heads_or_layers(mc):
    say("clip: no heads, no layers")
    Wq = torch.empty(0, 32, dtype=torch.bfloat16, device=DEV)
    Wk = torch.empty(0, 32, dtype=torch.bfloat16, device=DEV)
    gamma, clipped = mc.qk_clip_apply(torch.empty(0, device=DEV), Wq, Wk, 6, 4, 4)
    assert gamma.numel() == 0 and clipped.numel() == 0
    gamma, clipped = mc.qk_clip_apply_layers(torch.empty(0, 4, device=DEV), [], [], 6, 4, 4)
    assert gamma.shape == (0, 4) and clipped.shape == (0, 4)
    torch.cuda.synchronize()


def test_step_with_nothing_to_do(mc):
    say("empty page-level step")
    for fused in (True, False):
        assert mc.muonclip_step({}, {}, {}, None, None, 2e-4, fused=fused) == (None, None)
