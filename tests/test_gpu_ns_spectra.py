"""Newton-Schulz parity beyond Gaussian momentum: decaying spectra (four
decades), low rank plus noise, exact rank 1 and rank 4 (what rarely routed
experts produce), at the expert, down-projection and attention shapes.

The iteration maps a small normalised singular value s to about a^5 s
(a = 3.4445, some 490-fold over five steps), so any error the arithmetic
puts into those directions grows as much.  The library carries X as a bf16
high part plus a one-byte code of the rounding residual and adds the linear
term a X in float32, which keeps these inputs inside the tolerance: relative Frobenius error <= 2e-2
against the fp64 oracle ("Kimi K2, explained.", the Muon update bullets:
Newton-Schulz drives the singular values toward 1; the internals page's
Algorithm 1, O_t = NewtonSchulz(M_t)).
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import f64, rel_fro, say

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def mc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import muonclip_muon_amd
    return muonclip_muon_amd


CASES = [(k, 2048, 7168) for k in workloads.SPECTRAL_KINDS] + \
        [(k, 7168, 2048) for k in ("decay4", "rank16_noise", "rank1", "rank4")] + \
        [("decay4", 640, 1000), ("rank1", 300, 260), ("rank1", 4, 300), ("rank1", 16, 256),
         ("decay4", 16, 256), ("rank4", 16, 256)]


@pytest.mark.parametrize("kind,rows,cols", CASES)
def test_ns_spectral_classes(mc, kind, rows, cols):
    say("NS spectrum", kind, rows, cols)
    M = workloads.spectral_momentum(kind, rows, cols, seed=rows + cols + len(kind))
    O = mc.muon_ns_orthogonalize_batched(M.to(DEV), out_scale=1.0, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.newton_schulz(f64(M))
    err = rel_fro(f64(O), ref)
    say("  relative Frobenius error", f"{err:.3e}")
    assert err <= 2e-2, err


@pytest.mark.parametrize("kind", ["rank16_noise", "decay4", "rank1", "rank4"])
def test_ns_spectral_attention_shape(mc, kind):
    """W_q's shape, 12288 x 7168 (iterated on the 7168 x 12288 transpose)."""
    rows, cols = 12288, 7168
    say("NS spectrum", kind, rows, cols)
    M = workloads.spectral_momentum(kind, rows, cols, seed=7 + len(kind))
    O = mc.muon_ns_orthogonalize_batched(M.to(DEV), out_scale=1.0, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.newton_schulz(f64(M))
    err = rel_fro(f64(O), ref)
    say("  relative Frobenius error", f"{err:.3e}")
    assert err <= 2e-2, err


@pytest.mark.parametrize("kind", ["rank1", "rank16_noise"])
def test_fused_step_low_rank_momentum(mc, kind):
    """The fused momentum + Newton-Schulz + update call on a batch whose
    momentum is low rank (M_{t-1} = 0, so M_t = G): W_t - W_{t-1} against the
    oracle's step, lr 1 so the update dominates the bf16 rounding of W."""
    batch, rows, cols = 2, 2048, 7168
    say("fused low-rank", kind)
    G = torch.stack([workloads.spectral_momentum(kind, rows, cols, seed=50 + b) for b in range(batch)])
    W0 = workloads.normal((batch, rows, cols), 0.02, workloads.generator(51, "cpu"), "cpu", torch.bfloat16)
    M = torch.zeros(batch, rows, cols, device=DEV)
    W = W0.to(DEV)
    mc.muon_momentum_ns_update_batched(M, G.to(DEV), W, 1.0, 0.1, 0.95)
    torch.cuda.synchronize()
    assert torch.equal(M.cpu(), G)  # M_0 = 0: M_1 = G exactly
    for b in range(batch):
        ref = oracle.apply_update(f64(W0[b]), oracle.muon_orthogonalised_update(f64(G[b])), 1.0, 0.1, "bf16")
        err = rel_fro(f64(W[b]) - f64(W0[b]), ref - f64(W0[b]))
        say("  relative Frobenius error", b, f"{err:.3e}")
        assert err <= 2e-2, (b, err)
