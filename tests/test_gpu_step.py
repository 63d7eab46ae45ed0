"""GPU parity of the page-level step: QK-Clip of every attention layer in one
call (qk_clip_apply_layers) and muonclip_step over several attention layers
and stacked expert matrices, against the fp64 oracle.  (Algorithm 1 of "Kimi
K2 内部机制" clips every head of every attention layer; the Zhihu MuonClip
formula indexes S_max by layer and head.)

Tolerances as in test_gpu_parity.py: clipped sets identical, gamma <= 1e-6
relative, clipped rows <= 1 bf16 ulp (2 float32 ulps), untouched heads bit
for bit; weight updates within the Newton-Schulz tolerance 2e-2.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import bf16_bits, bf16_ulp_diff, f32_ulp_diff, f64, rel_err, rel_fro, say

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def mc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import muonclip_muon_amd
    return muonclip_muon_amd


def _check_layer(wname, got_q, got_k, src_q, src_k, ref_q, ref_k, rc, qph, kph):
    iv = torch.int16 if wname == "bf16" else torch.int32
    for got, ref, src, rows in ((got_q, ref_q, src_q, qph), (got_k, ref_k, src_k, kph)):
        for h in range(len(rc)):
            sl = slice(h * rows, (h + 1) * rows)
            if rc[h] != 1:
                assert torch.equal(got[sl].cpu().view(iv), src[sl].view(iv))
            elif wname == "bf16":
                assert bf16_ulp_diff(bf16_bits(got[sl]), oracle.bf16_bits(ref[sl])).max() <= 1
            else:
                assert f32_ulp_diff(got[sl].cpu().numpy(), ref[sl]).max() <= 2


@pytest.mark.parametrize("L,H,wdt,d_in", [(3, 8, torch.bfloat16, 64), (2, 5, torch.float32, 36),
                                          (70, 4, torch.bfloat16, 32), (61, 64, torch.bfloat16, 8)])
def test_qk_clip_apply_layers(mc, L, H, wdt, d_in):
    """MLA split (q^C x sqrt(gamma), q^R x gamma, k^C x sqrt(gamma)); 70 layers
    take two launches; 61 x 64 heads is Kimi K2's layer and head count."""
    say("qk_clip_apply_layers", L, H, wdt, d_in)
    dc, dr = 8, 4
    qph, kph = dc + dr, dc
    g = workloads.generator(300 + L, "cpu")
    Wq = [workloads.normal((H * qph, d_in), 0.02, g, "cpu", wdt) for _ in range(L)]
    Wk = [workloads.normal((H * kph, d_in), 0.02, g, "cpu", wdt) for _ in range(L)]
    smax = workloads.normal((L, H), 60.0, g, "cpu").abs() + 40.0  # about a third of the heads over tau
    smax[0, 0] = float("nan")
    smax[L - 1, H - 1] = 100.0  # a tie at tau: not clipped
    Wqd, Wkd = [w.to(DEV) for w in Wq], [w.to(DEV) for w in Wk]
    gamma, clipped = mc.qk_clip_apply_layers(smax.to(DEV), Wqd, Wkd, qph, dc, kph, tau=100.0)
    torch.cuda.synchronize()
    wname = "bf16" if wdt == torch.bfloat16 else "f32"
    assert gamma.shape == (L, H) and clipped.shape == (L, H)
    for layer in range(L):
        rq, rk, rg, rc = oracle.qk_clip(f64(smax[layer]), f64(Wq[layer]), f64(Wk[layer]), qph, dc, kph, 100.0, 0.5,
                                        wname)
        assert clipped[layer].cpu().tolist() == rc.tolist(), layer
        assert rel_err(gamma[layer].cpu().numpy(), rg).max() <= 1e-6
        _check_layer(wname, Wqd[layer], Wkd[layer], Wq[layer], Wk[layer], rq, rk, rc, qph, kph)


def test_two_layer_step_with_stacked_experts(mc):
    """muonclip_step on two fp32 MHA attention layers (d_model 256, 4 heads of
    64, a different hot head per layer) plus a stack of 3 expert matrices:
    S_max [2, 4] measured by the library on each layer's forward, then one
    step; the oracle runs the same step from its own projections and S_max."""
    say("two-layer step")
    H, hd, d = 4, 64, 256
    g = workloads.generator(400, "cpu")
    X = workloads.normal((2, 128, d), 1.0, g, "cpu")
    W, att = {}, []
    for layer, hot in ((0, 0), (1, 2)):
        for n in ("q", "k", "v"):
            w = workloads.normal((d, d), 0.1414, g, "cpu")
            if n != "v":
                w[hot * hd:(hot + 1) * hd] *= 8.0
            W[f"{n}{layer}"] = w
        att.append(dict(q=f"q{layer}", k=f"k{layer}", q_rows_per_head=hd, q_c_rows=hd, k_rows_per_head=hd))
    W["experts"] = workloads.normal((3, 96, 320), 0.02, g, "cpu")
    G = {n: workloads.normal(w.shape, 1e-3, g, "cpu") for n, w in W.items()}

    # the oracle's own forward and step
    Wn = {n: f64(w) for n, w in W.items()}
    ref_s = np.stack([oracle.max_logit(oracle.project_heads(f64(X), Wn[f"q{l}"], H),
                                       oracle.project_heads(f64(X), Wn[f"k{l}"], H)) for l in range(2)])
    new_w, new_m, rg, rc = oracle.muonclip_step(Wn, {n: G[n].numpy() for n in G}, {}, ref_s, att, lr=0.02,
                                                w_dtype="f32")
    assert rc[0, 0] == 1 and rc[1, 2] == 1

    # the library's
    Xd = X.to(DEV)
    Wd = {n: w.to(DEV) for n, w in W.items()}
    Gd = {n: g_.to(DEV) for n, g_ in G.items()}
    smax = torch.empty(2, H, device=DEV)
    for l in range(2):
        Q = (Xd @ Wd[f"q{l}"].t().contiguous()).view(2, 128, H, hd).transpose(1, 2).contiguous()
        K = (Xd @ Wd[f"k{l}"].t().contiguous()).view(2, 128, H, hd).transpose(1, 2).contiguous()
        mc.qk_maxlogit(Q, K, smax=smax[l])
    momenta = {}
    gamma, clipped = mc.muonclip_step(Wd, Gd, momenta, smax, att, lr=0.02)
    torch.cuda.synchronize()
    assert rel_err(smax.cpu().numpy(), ref_s).max() <= 1e-5
    assert clipped.cpu().numpy().tolist() == rc.tolist()
    assert rel_err(gamma.cpu().numpy(), rg).max() <= 1e-5
    for n in W:
        np.testing.assert_array_equal(momenta[n].cpu().numpy(), new_m[n])  # M_1 = G bit for bit
        if n == "experts":
            for i in range(3):
                assert rel_fro(f64(Wd[n][i]) - Wn[n][i], new_w[n][i] - Wn[n][i]) <= 2e-2, (n, i)
        else:
            assert rel_fro(f64(Wd[n]) - Wn[n], new_w[n] - Wn[n]) <= 2e-2, n


def test_step_chunks_share_one_workspace(mc):
    """A stack larger than the chunk goes through several fused calls on one
    workspace; the result equals one call per matrix (same kernels), and the
    three-call path agrees to the Newton-Schulz tolerance."""
    say("step chunks")
    g = workloads.generator(401, "cpu")
    W0 = workloads.normal((5, 256, 512), 0.02, g, "cpu", torch.bfloat16)
    G = workloads.normal((5, 256, 512), 1e-3, g, "cpu")
    smax = torch.full((1,), 1.0, device=DEV)
    Wq = torch.zeros(8, 16, device=DEV, dtype=torch.bfloat16)
    att = dict(q="q", k="k", q_rows_per_head=8, q_c_rows=8, k_rows_per_head=8)
    ws = torch.empty(mc.muon_ns_workspace_bytes(2, 256, 512), dtype=torch.uint8, device=DEV)
    Wa = {"e": W0.to(DEV), "q": Wq.clone(), "k": Wq.clone()}
    mc.muonclip_step(Wa, {"e": G.to(DEV), "q": torch.zeros(8, 16, device=DEV), "k": torch.zeros(8, 16, device=DEV)},
                     {}, smax, att, lr=1.0, chunk=2, workspace=ws)
    Wb = W0.to(DEV)
    for i in range(5):
        mc.muon_momentum_ns_update_batched(torch.zeros(256, 512, device=DEV), G[i].to(DEV), Wb[i], 1.0, 0.1, 0.95)
    Wc = {"e": W0.to(DEV), "q": Wq.clone(), "k": Wq.clone()}
    mc.muonclip_step(Wc, {"e": G.to(DEV), "q": torch.zeros(8, 16, device=DEV), "k": torch.zeros(8, 16, device=DEV)},
                     {}, smax, att, lr=1.0, chunk=2, fused=False)
    torch.cuda.synchronize()
    assert torch.equal(Wa["e"].view(torch.int16), Wb.view(torch.int16))
    for i in range(5):
        assert rel_fro(f64(Wc["e"][i]) - f64(W0[i]), f64(Wa["e"][i]) - f64(W0[i])) <= 2e-2
    with pytest.raises(ValueError):  # a workspace for chunks of 2, not 4
        mc.muonclip_step(Wa, {"e": G.to(DEV), "q": torch.zeros(8, 16, device=DEV), "k": torch.zeros(8, 16, device=DEV)},
                         {}, smax, att, lr=1.0, chunk=4, workspace=ws)


def test_invalid_step_changes_nothing(mc):
    """muonclip_step checks every argument before its first launch, so a call
    that raises leaves every weight and momentum as it was and creates no
    momentum (no partial step): attention weights that are missing or do not
    hold the heads of the row split, an S_max of the wrong shape, a missing
    or mis-shaped gradient, tau, alpha, lr, steps or coefficients out of
    range, a workspace too small."""
    say("invalid step")
    g = workloads.generator(402, "cpu")
    W0 = workloads.normal((3, 256, 512), 0.02, g, "cpu", torch.bfloat16).to(DEV)
    G = workloads.normal((3, 256, 512), 1e-3, g, "cpu").to(DEV)
    M0 = workloads.normal((3, 256, 512), 1e-3, g, "cpu").to(DEV)
    Wq0 = workloads.normal((8, 16), 0.02, g, "cpu", torch.bfloat16).to(DEV)
    zeros = torch.zeros(8, 16, device=DEV)
    att = dict(q="q", k="k", q_rows_per_head=8, q_c_rows=8, k_rows_per_head=8)
    smax = torch.full((1,), 1000.0, device=DEV)
    grads = {"e": G, "q": zeros, "k": zeros}
    small_ws = torch.empty(mc.muon_ns_workspace_bytes(1, 256, 512), dtype=torch.uint8, device=DEV)
    cases = {
        "unknown weight": dict(attention=dict(att, k="v")),
        "row split": dict(attention=dict(att, k_rows_per_head=4)),
        "smax heads": dict(smax=torch.full((2,), 1000.0, device=DEV)),
        "smax layers": dict(smax=torch.full((2, 1), 1000.0, device=DEV)),
        "no gradient": dict(grads={"e": G, "q": zeros}),
        "gradient shape": dict(grads={"e": G[:2], "q": zeros, "k": zeros}),
        "gradient dtype": dict(grads={"e": G.bfloat16(), "q": zeros, "k": zeros}),
        "tau": dict(tau=0.0),
        "alpha": dict(alpha=1.5),
        "lr": dict(lr=float("nan")),
        "steps": dict(steps=0),
        "coefficients": dict(coeffs=((3.4445, float("inf"), 2.0315),) * 5),
        "workspace": dict(workspace=small_ws),
    }
    for name, over in cases.items():
        W = {"e": W0.clone(), "q": Wq0.clone(), "k": Wq0.clone()}
        M = {"e": M0.clone()}
        kw = dict(weights=W, grads=grads, momenta=M, smax=smax, attention=att, lr=2e-4)
        kw.update(over)
        with pytest.raises(ValueError):
            mc.muonclip_step(**kw)
        torch.cuda.synchronize()
        assert torch.equal(W["e"].view(torch.int16), W0.view(torch.int16)), name
        assert torch.equal(W["q"].view(torch.int16), Wq0.view(torch.int16)), name
        assert torch.equal(W["k"].view(torch.int16), Wq0.view(torch.int16)), name
        assert torch.equal(M["e"], M0) and set(M) == {"e"}, name


def test_resume_from_saved_state_is_bit_exact(mc):
    """The optimizer state is W and the momentum M (M_0 = 0; the method keeps
    nothing else).  Two steps run straight through, and the same second step
    run again on fresh tensors restored from a host copy of (W, M) taken after
    the first, give bit-identical W, M, gamma and clip flags: the step is
    deterministic (the max reductions are exact and order-free), so resuming
    from a checkpoint of (W, M) reproduces the run."""
    say("resume from (W, M)")
    H, hd, d = 4, 64, 256
    g = workloads.generator(402, "cpu")
    W = {"q": workloads.normal((H * hd, d), 0.02, g, "cpu", torch.bfloat16),
         "k": workloads.normal((H * hd, d), 0.02, g, "cpu", torch.bfloat16),
         "experts": workloads.normal((3, 256, 384), 0.02, g, "cpu", torch.bfloat16),
         "down": workloads.normal((2, 384, 256), 0.02, g, "cpu", torch.bfloat16)}
    grads = [{n: workloads.normal(w.shape, 1e-3, g, "cpu") for n, w in W.items()} for _ in range(2)]
    smaxes = [torch.tensor([150.0, 20.0, 300.0, 99.0]), torch.tensor([101.0, 180.0, 5.0, 250.0])]
    att = dict(q="q", k="k", q_rows_per_head=hd, q_c_rows=hd, k_rows_per_head=hd)

    def step(Wd, Md, t):
        Gd = {n: x.to(DEV) for n, x in grads[t].items()}
        return mc.muonclip_step(Wd, Gd, Md, smaxes[t].to(DEV), att, lr=2e-3, weight_decay=0.1, chunk=2)

    Wd = {n: w.to(DEV) for n, w in W.items()}
    Md = {}
    step(Wd, Md, 0)
    torch.cuda.synchronize()
    ckpt_w = {n: w.cpu().clone() for n, w in Wd.items()}
    ckpt_m = {n: m.cpu().clone() for n, m in Md.items()}
    gamma1, clipped1 = step(Wd, Md, 1)
    torch.cuda.synchronize()

    Wr = {n: w.to(DEV) for n, w in ckpt_w.items()}
    Mr = {n: m.to(DEV) for n, m in ckpt_m.items()}
    gamma2, clipped2 = step(Wr, Mr, 1)
    torch.cuda.synchronize()
    assert torch.equal(gamma1, gamma2) and torch.equal(clipped1, clipped2)
    assert clipped1.cpu().tolist() == [1, 1, 0, 1]
    for n in W:
        assert torch.equal(Wd[n].view(torch.int16), Wr[n].view(torch.int16)), n
        assert torch.equal(Md[n].view(torch.int32), Mr[n].view(torch.int32)), n
