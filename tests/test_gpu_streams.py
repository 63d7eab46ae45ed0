"""Calls on a stream other than torch's current one, with the scratch memory
(Newton-Schulz workspace, output buffers, new momenta) allocated by the binding: the
results equal, bit for bit, the same calls on the current stream, although
the current stream allocates and overwrites memory of the same size while
the side stream's kernels still run.  The binding allocates such scratch in
the launch stream's pool, so the caching allocator cannot hand it to the
current stream early.  The first call is also checked against the fp64
oracle (the Newton-Schulz tolerance, relative Frobenius error 2e-2).
"""

import pytest
import torch

import oracle
import workloads
from gpu_helpers import f64, rel_fro, say

pytestmark = pytest.mark.gpu

DEV = "cuda"
BATCH, ROWS, COLS = 4, 1024, 4096


@pytest.fixture(scope="module")
def mc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import muonclip_muon_amd
    return muonclip_muon_amd


def _clobber(nbytes):
    # what another part of a program does on the current stream meanwhile:
    # allocate blocks of the workspace's size class and fill them
    return [torch.full((nbytes,), 0x7f, dtype=torch.uint8, device=DEV) for _ in range(3)]


def test_ns_on_side_stream(mc):
    say("NS on a side stream")
    g = workloads.generator(91, "cpu")
    M = workloads.normal((BATCH, ROWS, COLS), 1e-3, g, "cpu").to(DEV)
    ref = mc.muon_ns_orthogonalize_batched(M, out_dtype=torch.float32)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    O = mc.muon_ns_orthogonalize_batched(M, out_dtype=torch.float32, stream=s)
    junk = _clobber(mc.muon_ns_workspace_bytes(BATCH, ROWS, COLS))
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(O, ref)
    assert all(int(j[0]) == 0x7f for j in junk)
    err = rel_fro(f64(O[0]), oracle.newton_schulz(f64(M[0])))
    assert err <= 2e-2, err


def test_fused_on_side_stream(mc):
    say("fused step on a side stream")
    g = workloads.generator(92, "cpu")
    M0 = workloads.normal((BATCH, ROWS, COLS), 1e-3, g, "cpu").to(DEV)
    G = workloads.normal((BATCH, ROWS, COLS), 1e-3, g, "cpu").to(DEV)
    W0 = workloads.normal((BATCH, ROWS, COLS), 0.02, g, "cpu", torch.bfloat16).to(DEV)
    M_ref, W_ref = M0.clone(), W0.clone()
    mc.muon_momentum_ns_update_batched(M_ref, G, W_ref, 2e-2, 0.1, 0.95)
    torch.cuda.synchronize()
    M, W = M0.clone(), W0.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    mc.muon_momentum_ns_update_batched(M, G, W, 2e-2, 0.1, 0.95, stream=s)
    _clobber(mc.muon_ns_workspace_bytes(BATCH, ROWS, COLS))
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(M, M_ref)
    assert torch.equal(W, W_ref)


def test_page_step_on_side_stream(mc):
    """muonclip_step on a side stream with momenta it creates itself (zero-filled
    on that stream) and its own workspace, no attention layer: bit-identical to
    the same step on the current stream."""
    say("page-level step on a side stream")
    g = workloads.generator(93, "cpu")
    W0 = workloads.normal((3, 256, 1024), 0.02, g, "cpu", torch.bfloat16).to(DEV)
    G = {"experts": workloads.normal((3, 256, 1024), 1e-3, g, "cpu").to(DEV)}
    W_ref, mom_ref = {"experts": W0.clone()}, {}
    assert mc.muonclip_step(W_ref, G, mom_ref, None, None, lr=2e-2) == (None, None)
    torch.cuda.synchronize()
    W, mom = {"experts": W0.clone()}, {}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    mc.muonclip_step(W, G, mom, None, None, lr=2e-2, stream=s)
    _clobber(mc.muon_ns_workspace_bytes(3, 256, 1024))
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(mom["experts"], mom_ref["experts"])
    assert torch.equal(W["experts"], W_ref["experts"])


def test_concurrent_host_threads(mc):
    """Two host threads drive the library at once, each on its own stream with
    its own inputs, workspace and outputs (the C calls run without the GIL,
    so argument checking and launching overlap): every result is bit-identical
    to the same call made alone, since the library keeps no mutable state
    between calls (the allocation-free entry point's shared scratch aside)."""
    import threading
    say("two host threads")
    g = workloads.generator(93, "cpu")
    jobs = []
    for t in range(2):
        M = workloads.normal((2, 512, 1536), 1e-3, g, "cpu").to(DEV)
        G = workloads.normal((2, 512, 1536), 1e-3, g, "cpu").to(DEV)
        W = workloads.normal((2, 512, 1536), 0.02, g, "cpu", torch.bfloat16).to(DEV)
        ws = torch.empty(mc.muon_ns_workspace_bytes(2, 512, 1536), dtype=torch.uint8, device=DEV)
        jobs.append(dict(M=M, G=G, W=W, ws=ws, stream=torch.cuda.Stream()))
    # alone, one after the other: three fused steps each
    ref = []
    for j in jobs:
        M, W = j["M"].clone(), j["W"].clone()
        for _ in range(3):
            mc.muon_momentum_ns_update_batched(M, j["G"], W, 2e-3, workspace=j["ws"])
        torch.cuda.synchronize()
        ref.append((M, W))
    # at once, from two threads
    outs = [None, None]
    errors = []

    def run(k):
        try:
            j = jobs[k]
            M, W = j["M"].clone(), j["W"].clone()
            torch.cuda.synchronize()
            for _ in range(3):
                mc.muon_momentum_ns_update_batched(M, j["G"], W, 2e-3, workspace=j["ws"], stream=j["stream"])
            j["stream"].synchronize()
            outs[k] = (M, W)
        except Exception as e:  # noqa: BLE001  (reported below)
            errors.append(e)

    threads = [threading.Thread(target=run, args=(k,)) for k in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not errors, errors
    for (M, W), (Mr, Wr) in zip(outs, ref):
        assert torch.equal(M.view(torch.int32), Mr.view(torch.int32))
        assert torch.equal(W.view(torch.int16), Wr.view(torch.int16))
