"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times, on outputs the oracle can compute one by one: sampled
elements of the element-wise steps, whole matrices of a Newton-Schulz batch,
whole heads of the max logit, and the clipped rows of every clipped head.

Tolerances as in test_gpu_parity.py.  These take tens of seconds of oracle
CPU time each.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import bf16_bits, bf16_ulp_diff, f64, rel_err, rel_fro, say

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def mc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import muonclip_muon_amd
    return muonclip_muon_amd


def _sample(n, k, seed):
    return np.sort(np.random.default_rng(seed).choice(n, size=k, replace=False))


def test_expert_batch_momentum_ns_update(mc):
    """64 expert matrices 2048 x 7168: momentum over the batch (sampled elements
    bit-exact), Newton-Schulz x5 with the Muon scale in one 64-matrix call on
    the new momentum (two whole matrices against the oracle's own momentum
    and Newton-Schulz of the same inputs), and the update with a seeded O
    (sampled)."""
    say("full size: 64 x 2048 x 7168 momentum + NS + update")
    batch, rows, cols = 64, 2048, 7168
    eb = workloads.expert_batch(seed=2, device=DEV, batch=batch, rows=rows, cols=cols, std=1e-3)
    M, G = eb.M_prev, eb.G
    idx = _sample(M.numel(), 1 << 20, 1)
    idx_t = torch.from_numpy(idx).to(DEV)
    m0 = M.view(-1)[idx_t].cpu().numpy()
    g0 = G.view(-1)[idx_t].cpu().numpy()
    picks = (0, 37)
    m_in = {b: M[b].cpu().numpy() for b in picks}
    g_in = {b: G[b].cpu().numpy() for b in picks}
    mc.muonclip_momentum(M, G, 0.95)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(M.view(-1)[idx_t].cpu().numpy(), oracle.momentum_update(m0, g0, 0.95))
    del G

    scale = mc.muon_out_scale(rows, cols)
    O = mc.muon_ns_orthogonalize_batched(M, out_scale=scale, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    for b in picks:
        say("  oracle momentum and NS of matrix", b)
        ref = oracle.muon_orthogonalised_update(oracle.momentum_update(m_in[b], g_in[b], 0.95).astype(np.float64))
        err = rel_fro(f64(O[b]), ref)
        assert err <= 2e-2, (b, err)
    del O

    gen = workloads.generator(9, DEV)
    W = workloads.normal((batch, rows, cols), 0.02, gen, DEV, torch.bfloat16)
    O = workloads.normal((batch, rows, cols), 0.2, gen, DEV, torch.bfloat16)
    w0 = W.view(-1)[idx_t].clone()
    o0 = O.view(-1)[idx_t].clone()
    mc.muon_apply_update(W, O, 2e-4, 0.1)
    torch.cuda.synchronize()
    ref = oracle.apply_update(f64(w0), f64(o0), 2e-4, 0.1, "bf16")
    d = bf16_ulp_diff(bf16_bits(W.view(-1)[idx_t]), oracle.bf16_bits(ref))
    assert d.max() <= 1


def test_transposed_expert_batch_ns(mc):
    """Down-projection shape 7168 x 2048 (iterated on the transpose)."""
    say("full size: 8 x 7168 x 2048 NS")
    rows, cols = 7168, 2048
    M = workloads.normal((8, rows, cols), 1e-3, workloads.generator(21, DEV), DEV)
    O = mc.muon_ns_orthogonalize_batched(M, out_scale=mc.muon_out_scale(rows, cols), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref = oracle.muon_orthogonalised_update(f64(M[5]))
    assert rel_fro(f64(O[5]), ref) <= 2e-2


def test_attention_projection_ns(mc):
    """W_kc 8192 x 7168 (n = 7168, one matrix, 28 x 28 tiles) and W_kr 64 x 7168."""
    for rows, cols in ((8192, 7168), (64, 7168)):
        say("full size: NS of", rows, "x", cols)
        M = workloads.normal((rows, cols), 1e-4, workloads.generator(22 + rows, DEV), DEV)
        O = mc.muon_ns_orthogonalize_batched(M, out_scale=mc.muon_out_scale(rows, cols),
                                             out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        ref = oracle.muon_orthogonalised_update(f64(M))
        assert rel_fro(f64(O), ref) <= 2e-2


def test_maxlogit_and_clip_8x4096(mc):
    """64 heads, q/k 128 + 64, X 8 x 4096 x 7168: every head's S_max against the
    oracle, identical clipped set, then QK-Clip of the full W_q / W_kc."""
    say("full size: max logit 8 x 4096 x 64 heads")
    Wq, Wkc, Wkr, hot = workloads.mla_weights(seed=3, device=DEV)
    X = workloads.normal((8, 4096, 7168), 1.0, workloads.generator(3 + 2000, DEV), DEV, torch.bfloat16)
    Q, Kc, Kr = workloads.mla_project(X, Wq, Wkc, Wkr, 64)
    del X
    s = mc.qk_maxlogit(Q, Kc, Kr).cpu().numpy()
    Kr_h = f64(Kr)
    ref = np.empty(64)
    for h in range(64):
        ref[h] = oracle.max_logit(f64(Q[:, h:h + 1]), f64(Kc[:, h:h + 1]), Kr_h)[0]
    assert rel_err(s, ref).max() <= 1e-2
    assert rel_err(s, ref).max() <= 1e-4
    gclip, cclip = oracle.clip_factors(ref, 100.0)
    gpu_set = sorted(np.nonzero(s > 100.0)[0].tolist())
    assert gpu_set == sorted(np.nonzero(cclip == 1)[0].tolist()) == sorted(hot.tolist())

    say("full size: QK-Clip of W_q 12288 x 7168, W_kc 8192 x 7168")
    smax = torch.from_numpy(s).to(DEV)
    Wq0, Wkc0, Wkr0 = Wq.clone(), Wkc.clone(), Wkr.clone()
    gamma, clipped = mc.qk_clip_apply(smax, Wq, Wkc, 192, 128, 128)
    torch.cuda.synchronize()
    assert sorted(np.nonzero(clipped.cpu().numpy() == 1)[0].tolist()) == gpu_set
    for h in range(64):
        qs, ks = slice(192 * h, 192 * h + 192), slice(128 * h, 128 * h + 128)
        if h in gpu_set:
            # the oracle's clip from its own S_max (within 1e-4 of the library's,
            # far inside one bf16 ulp of the scaled rows)
            rq, rk, _, _ = oracle.qk_clip(np.array([ref[h]]), f64(Wq0[qs]), f64(Wkc0[ks]), 192, 128, 128)
            assert bf16_ulp_diff(bf16_bits(Wq[qs]), oracle.bf16_bits(rq)).max() <= 1
            assert bf16_ulp_diff(bf16_bits(Wkc[ks]), oracle.bf16_bits(rk)).max() <= 1
        else:
            assert torch.equal(Wq[qs].view(torch.int16), Wq0[qs].view(torch.int16))
            assert torch.equal(Wkc[ks].view(torch.int16), Wkc0[ks].view(torch.int16))
    assert torch.equal(Wkr.view(torch.int16), Wkr0.view(torch.int16))  # the shared rotary key


def test_maxlogit_long_context_32k(mc):
    """Batch 1 x 32768 tokens, 64 heads, no hot head: two heads against the
    oracle, and no head clipped."""
    say("full size: max logit 1 x 32768 x 64 heads")
    L = workloads.mla_logits(seed=5, device=DEV, batch=1, seq=32768, n_hot=0)
    s = mc.qk_maxlogit(L.Q, L.Kc, L.Kr).cpu().numpy()
    assert np.all(s < 100.0)
    Kr_h = f64(L.Kr)
    for h in (0, 41):
        say("  oracle head", h)
        ref = oracle.max_logit(f64(L.Q[:, h:h + 1]), f64(L.Kc[:, h:h + 1]), Kr_h, block=4096)[0]
        assert rel_err(s[h], ref) <= 1e-4


@pytest.mark.parametrize("shape", [(64, 2048, 7168), (64, 7168, 2048), (1, 12288, 7168), (1, 8192, 7168),
                                   (1, 64, 7168)])
def test_fused_expert_batch(mc, shape):
    """The fused momentum + Newton-Schulz + update call at every shape the
    benchmark times, in its launch configuration: chunks of 64 gate/up
    experts and of 64 down-projection experts (iterated on the transpose),
    and W_q, W_kc, W_kr one matrix per call.  Sampled momentum elements
    bit-exact, and W_t - W_{t-1} of the first and last matrix against the
    oracle (lr 1 so that the update, not the bf16 rounding of W, dominates
    the difference)."""
    batch, rows, cols = shape
    say("full size fused:", shape)
    gen = workloads.generator(31 + rows, DEV)
    M = workloads.normal(shape, 1e-4, gen, DEV)
    G = workloads.normal(shape, 1e-4, gen, DEV)
    W = workloads.normal(shape, 0.02, gen, DEV, torch.bfloat16)
    idx_t = torch.from_numpy(_sample(M.numel(), min(1 << 20, M.numel()), 3)).to(DEV)
    m0 = M.view(-1)[idx_t].cpu().numpy()
    g0 = G.view(-1)[idx_t].cpu().numpy()
    picks = (0, batch - 1)
    M_pick = {b: M[b].clone() for b in picks}
    G_pick = {b: G[b].clone() for b in picks}
    W_pick = {b: W[b].clone() for b in picks}
    mc.muon_momentum_ns_update_batched(M, G, W, 1.0, 0.1, 0.95)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(M.view(-1)[idx_t].cpu().numpy(), oracle.momentum_update(m0, g0, 0.95))
    for b in picks:
        say("  oracle step of matrix", b)
        Mn = oracle.momentum_update(M_pick[b].cpu().numpy(), G_pick[b].cpu().numpy(), 0.95)
        W0 = f64(W_pick[b])
        ref = oracle.apply_update(W0, oracle.muon_orthogonalised_update(Mn.astype(np.float64)), 1.0, 0.1, "bf16")
        err = rel_fro(f64(W[b]) - W0, ref - W0)
        assert err <= 2e-2, (b, err)
