"""The allocation-free entry point (muon_momentum_ns_update_batched_noalloc,
for callers that cannot allocate) against the workspace entry point it
varies: the same kernels on the same inputs, so M and W agree bit for bit,
and the update agrees with the fp64 oracle to the Newton-Schulz tolerance
(relative Frobenius error <= 2e-2).  Two calls in a row, the second smaller,
then a size beyond the static scratch (rejected before anything runs)."""

import ctypes

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


def _inputs(seed, batch, rows, cols, wdt):
    g = workloads.generator(seed, "cpu")
    M0 = workloads.normal((batch, rows, cols), 1e-3, g, "cpu")
    G = workloads.normal((batch, rows, cols), 1e-3, g, "cpu")
    W0 = workloads.normal((batch, rows, cols), 0.02, g, "cpu", wdt)
    return M0, G, W0


def _noalloc_c(mc, M, G, W, lr, wd, mu):
    """Call the entry point through the C ABI directly (no binding logic)."""
    batch, rows, cols = M.shape
    coeffs = (ctypes.c_float * 15)(*[x for abc in mc.NS_COEFFS for x in abc])
    st = mc.lib.muon_momentum_ns_update_batched_noalloc(
        M.data_ptr(), G.data_ptr(), mu, W.data_ptr(), 1 if W.dtype == torch.bfloat16 else 0, batch, rows, cols,
        rows * cols, 5, coeffs, mc.NS_EPS, -1.0, lr, wd, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, mc.lib.mc_status_string(st)


@pytest.mark.parametrize("first,second", [((2, 512, 1024, torch.bfloat16), (1, 300, 520, torch.bfloat16)),
                                          ((1, 1000, 600, torch.float32), (3, 256, 256, torch.float32))])
def test_noalloc_matches_workspace_entry_point(mc, first, second):
    for k, (batch, rows, cols, wdt) in enumerate((first, second)):
        say("no-alloc fused call", k, batch, rows, cols, wdt)
        M0, G, W0 = _inputs(4000 + 7 * k + rows, batch, rows, cols, wdt)
        lr = 1.0 if wdt == torch.bfloat16 else 0.02
        Ma, Wa = M0.to(DEV), W0.to(DEV)
        mc.muon_momentum_ns_update_batched(Ma, G.to(DEV), Wa, lr, 0.1, 0.95)
        Mb, Wb = M0.to(DEV), W0.to(DEV)
        _noalloc_c(mc, Mb, G.to(DEV), Wb, lr, 0.1, 0.95)
        torch.cuda.synchronize()
        assert torch.equal(Ma, Mb)
        assert torch.equal(Wa.view(torch.int16) if wdt == torch.bfloat16 else Wa.view(torch.int32),
                           Wb.view(torch.int16) if wdt == torch.bfloat16 else Wb.view(torch.int32))
        M_ref = oracle.momentum_update(M0.numpy(), G.numpy(), 0.95)
        np.testing.assert_array_equal(Mb.cpu().numpy(), M_ref)
        wname = "bf16" if wdt == torch.bfloat16 else "f32"
        for b in range(batch):
            O_ref = oracle.muon_orthogonalised_update(M_ref[b].astype(np.float64))
            W_ref = oracle.apply_update(f64(W0[b]), O_ref, lr, 0.1, wname)
            assert rel_fro(f64(Wb[b]) - f64(W0[b]), W_ref - f64(W0[b])) <= 2e-2, (k, b)


def test_noalloc_rejects_sizes_beyond_the_scratch(mc):
    say("no-alloc size limit")
    limit = 192 << 20
    assert mc.lib.muon_ns_workspace_bytes(4, 2048, 7168) > limit
    M = torch.zeros(4, 2048, 7168, device=DEV)
    W = torch.zeros(4, 2048, 7168, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(mc.MuonClipError) as e:
        mc.muon_momentum_ns_update_batched_noalloc(M, M, W, 2e-4)
    assert e.value.status == 5  # MC_EWORKSPACE
    assert torch.count_nonzero(W).item() == 0 and torch.count_nonzero(M).item() == 0
