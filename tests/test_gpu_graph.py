"""A whole step captured in a HIP graph (torch.cuda.graph): the
allocation-free fused Muon call, the max logit and QK-Clip, every output
preallocated, so nothing is allocated while capturing (the release library
issues no memset, copy or synchronisation of its own).  Capturing runs
nothing; the graph is then replayed three times, with unrelated eager work
and synchronisations between the replays, and after every replay W, M, the
clipped W_q / W_k, S_max, gamma and the clip flags are bit-identical to the
same number of steps run eagerly.
"""

import pytest
import torch

import workloads
from gpu_helpers import say

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def mc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import muonclip_muon_amd
    return muonclip_muon_amd


def test_step_replayed_from_a_hip_graph(mc):
    say("step in a HIP graph")
    batch, rows, cols = 2, 256, 512
    B, H, S, dc, dr = 1, 4, 128, 128, 64
    qph, qc, kph, d_in = 12, 8, 8, 64
    g = workloads.generator(600, "cpu")
    W0 = workloads.normal((batch, rows, cols), 0.02, g, "cpu", torch.bfloat16)
    G = workloads.normal((batch, rows, cols), 1e-3, g, "cpu").to(DEV)
    Q = workloads.normal((B, H, S, dc + dr), 1.0, g, "cpu", torch.bfloat16)
    Q[:, 0] = (Q[:, 0].float() * 40).to(torch.bfloat16)  # head 0 over tau
    Q = Q.to(DEV)
    Kc = workloads.normal((B, H, S, dc), 1.0, g, "cpu", torch.bfloat16).to(DEV)
    Kr = workloads.normal((B, S, dr), 1.0, g, "cpu", torch.bfloat16).to(DEV)
    Wq0 = workloads.normal((H * qph, d_in), 0.02, g, "cpu", torch.bfloat16)
    Wk0 = workloads.normal((H * kph, d_in), 0.02, g, "cpu", torch.bfloat16)

    def fresh():
        return [W0.to(DEV), torch.zeros(batch, rows, cols, device=DEV), Wq0.to(DEV), Wk0.to(DEV),
                torch.empty(H, device=DEV), torch.empty(H, device=DEV), torch.empty(H, dtype=torch.int32, device=DEV)]

    def step(W, M, Wq, Wk, smax, gamma, clipped):
        mc.muon_momentum_ns_update_batched_noalloc(M, G, W, 2e-3)
        mc.qk_maxlogit(Q, Kc, Kr, smax=smax)
        mc.qk_clip_apply(smax, Wq, Wk, qph, qc, kph, gamma=gamma, clipped=clipped)

    eager = fresh()
    ref = []
    for _ in range(3):
        step(*eager)
        torch.cuda.synchronize()
        ref.append([t.clone() for t in eager])
    assert ref[0][6].tolist() == [1, 0, 0, 0]

    state = fresh()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(*state)
    torch.cuda.synchronize()
    assert torch.equal(state[1], torch.zeros_like(state[1]))  # capturing ran nothing
    for r in range(3):
        graph.replay()
        torch.cuda.synchronize()
        other = torch.randn(1 << 20, device=DEV)  # unrelated eager work between replays
        float(other.sum())
        for k, (got, want) in enumerate(zip(state, ref[r])):
            assert torch.equal(got, want), (r, k)
