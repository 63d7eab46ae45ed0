"""Batches whose matrices sit further apart than rows x cols elements.

The C ABI's Newton-Schulz calls take a batch stride (elements from one
matrix to the next, at least rows x cols); the binding always passes packed
stacks, so these tests call the library through ctypes. A strided call must
give bit for bit what the same matrices give packed, read nothing from the
gaps and write nothing into them. The gaps of M and G hold NaN, so a kernel
that read them would spread NaN into the results. The gaps of O and W hold a
sentinel pattern that must survive.

Cases: a straight matrix with the stride a multiple of 8 (the vector
pre-scale), a transposed one with an odd gap (the element-wise pre-scale),
and a ragged transposed one. One result is also checked against the oracle.
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import f64, rel_fro, say

pytestmark = pytest.mark.gpu

DEV = "cuda"
MC_F32, MC_BF16 = 0, 1
SENTINEL = 0x7FC1  # a bf16 quiet NaN with a payload no kernel writes

CASES = [(256, 512, 8), (512, 256, 3), (300, 260, 5)]  # rows, cols, gap in elements


@pytest.fixture(scope="module")
def mc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import muonclip_muon_amd
    return muonclip_muon_amd


def spread(x, stride, gap_value):
    """[B, r, c] -> a flat buffer with matrix b at [b * stride, b * stride + r c)
    and gap_value in between (and after the last matrix)."""
    B, r, c = x.shape
    buf = torch.full((B * stride,), gap_value, dtype=x.dtype, device=x.device)
    buf.view(B, stride)[:, : r * c] = x.reshape(B, r * c)
    return buf


def matrices(buf, B, r, c, stride):
    return buf.view(B, stride)[:, : r * c].reshape(B, r, c)


def gaps(buf, B, r, c, stride):
    return buf.view(B, stride)[:, r * c:]


@pytest.mark.parametrize("rows,cols,gap", CASES)
def test_newton_schulz_strided_batch(mc, rows, cols, gap):
    say(f"strided Newton-Schulz {rows}x{cols}, gap {gap}")
    B, L = 3, rows * cols
    g = workloads.generator(71, "cpu")
    M = workloads.normal((B, rows, cols), 1e-3, g, "cpu").to(DEV)
    Ms = spread(M, L + gap, float("nan"))
    Ms_before = Ms.clone()
    o_stride = L + gap + 2
    Os = spread(torch.zeros(B, rows, cols, dtype=torch.bfloat16, device=DEV), o_stride, 0.0)
    gaps(Os.view(torch.int16), B, rows, cols, o_stride).fill_(SENTINEL)
    ws = torch.empty(mc.muon_ns_workspace_bytes(B, rows, cols), dtype=torch.uint8, device=DEV)
    status = mc.lib.muon_ns_orthogonalize_batched(
        Ms.data_ptr(), MC_F32, B, rows, cols, L + gap, Os.data_ptr(), MC_BF16, o_stride, 5, mc._coeffs(5, None),
        mc.NS_EPS, 1.0, ws.data_ptr(), ws.numel(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream), None)
    assert status == 0, mc.lib.mc_status_string(status)
    packed = mc.muon_ns_orthogonalize_batched(M, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    got = matrices(Os, B, rows, cols, o_stride)
    assert torch.equal(got.view(torch.int16), packed.view(torch.int16))
    assert bool((gaps(Os.view(torch.int16), B, rows, cols, o_stride) == SENTINEL).all())
    assert torch.equal(Ms.view(torch.int32), Ms_before.view(torch.int32))  # M only read, gaps included
    ref = oracle.newton_schulz(f64(M[1]))
    assert rel_fro(f64(got[1]), ref) <= 2e-2


@pytest.mark.parametrize("rows,cols,gap", CASES)
def test_fused_step_strided_batch(mc, rows, cols, gap):
    say(f"strided fused step {rows}x{cols}, gap {gap}")
    B, L = 3, rows * cols
    S = L + gap
    g = workloads.generator(72, "cpu")
    M0 = workloads.normal((B, rows, cols), 1e-3, g, "cpu").to(DEV)
    G = workloads.normal((B, rows, cols), 1e-3, g, "cpu").to(DEV)
    W0 = workloads.normal((B, rows, cols), 0.02, g, "cpu", torch.bfloat16).to(DEV)
    Ms, Gs = spread(M0, S, float("nan")), spread(G, S, float("nan"))
    Ws = spread(W0, S, 0.0)
    gaps(Ws.view(torch.int16), B, rows, cols, S).fill_(SENTINEL)
    Ms_gaps = gaps(Ms, B, rows, cols, S).clone()
    ws = torch.empty(mc.muon_ns_workspace_bytes(B, rows, cols), dtype=torch.uint8, device=DEV)
    status = mc.lib.muon_momentum_ns_update_batched(
        Ms.data_ptr(), Gs.data_ptr(), 0.95, Ws.data_ptr(), MC_BF16, B, rows, cols, S, 5, mc._coeffs(5, None),
        mc.NS_EPS, mc.OUT_SCALE_RMS_MATCH, 1.0, 0.1, ws.data_ptr(), ws.numel(),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream), None)
    assert status == 0, mc.lib.mc_status_string(status)
    M, W = M0.clone(), W0.clone()
    mc.muon_momentum_ns_update_batched(M, G, W, 1.0)
    torch.cuda.synchronize()
    assert torch.equal(matrices(Ms, B, rows, cols, S).view(torch.int32), M.view(torch.int32))
    assert torch.equal(matrices(Ws, B, rows, cols, S).view(torch.int16), W.view(torch.int16))
    assert torch.equal(gaps(Ms, B, rows, cols, S).view(torch.int32), Ms_gaps.view(torch.int32))
    assert bool((gaps(Ws.view(torch.int16), B, rows, cols, S) == SENTINEL).all())
    # the update itself is the oracle's (momentum exact, W within the
    # Newton-Schulz tolerance; lr 1 so that the update, not the bf16 rounding
    # of W, dominates the change of W)
    m_ref = oracle.momentum_update(M0[2].cpu().numpy(), G[2].cpu().numpy(), 0.95)
    assert np.array_equal(M[2].cpu().numpy().view(np.int32), np.asarray(m_ref, np.float32).view(np.int32))
    w_ref = oracle.apply_update(f64(W0[2]), oracle.muon_orthogonalised_update(np.asarray(m_ref, np.float64)),
                                1.0, 0.1, "bf16")
    assert rel_fro(f64(W[2]) - f64(W0[2]), np.asarray(w_ref, np.float64) - f64(W0[2])) <= 2e-2
