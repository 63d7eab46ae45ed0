"""The largest Newton-Schulz shape the C ABI accepts (min(rows, cols) 16384,
max(rows, cols) 65536), in both orientations and through the fused call, on
momentum of exact rank 4 whose SVD is known from its factors
(workloads.orthonormal_factors): the exact result is
U diag(p(sigma / (||sigma|| + eps))) V^T with p the five steps of the
polynomial (oracle.ns_polynomial_scalar), so sampled rows of the output are
checked against it in fp64 without an SVD of the whole matrix.  The float32
momentum the device forms from the factors differs from the exact one by its
roundings (~1e-7 relative), far inside the Newton-Schulz tolerance 2e-2.
About 16 GB of device memory per case.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import rel_fro, say

pytestmark = pytest.mark.gpu

DEV = "cuda"
SIGMA = (30.0, 9.0, 1.5, 0.3)  # two decades; entries of M ~1e-3


@pytest.fixture(scope="module")
def mc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import muonclip_muon_amd
    return muonclip_muon_amd


def _case(rows, cols, seed):
    U, sigma, V = workloads.orthonormal_factors(rows, cols, SIGMA, seed=seed)
    M = (U * sigma).to(torch.float32).to(DEV) @ V.T.contiguous().to(torch.float32).to(DEV)
    p = oracle.ns_polynomial_scalar(sigma.numpy() / (np.linalg.norm(sigma.numpy()) + oracle.NS_EPS))
    sample = np.sort(np.random.default_rng(seed).choice(rows, size=64, replace=False))
    expect = (U.numpy()[sample] * p) @ V.numpy().T  # exact rows of NS(M)
    return M, sample, expect


@pytest.mark.parametrize("rows,cols", [(16384, 65536), (65536, 16384)])
def test_newton_schulz_at_the_largest_shape(mc, rows, cols):
    say("largest Newton-Schulz shape", rows, cols)
    M, sample, expect = _case(rows, cols, seed=71)
    O = mc.muon_ns_orthogonalize_batched(M, out_dtype=torch.float32)
    torch.cuda.synchronize()
    got = O[torch.from_numpy(sample).to(DEV)].double().cpu().numpy()
    err = rel_fro(got, expect)
    say("  sampled rows, relative Frobenius error", f"{err:.2e}")
    assert err <= 2e-2, err


def test_fused_call_at_the_largest_shape(mc):
    """M_0 = 0, W = 0: the momentum becomes G bit for bit and W becomes
    -lr * s * NS(G) rounded to bf16 (s the Muon scale), so NS(G) is read back
    from W to bf16 precision."""
    rows, cols = 16384, 65536
    say("largest shape, fused call", rows, cols)
    G, sample, expect = _case(rows, cols, seed=72)
    M = torch.zeros_like(G)
    W = torch.zeros(rows, cols, dtype=torch.bfloat16, device=DEV)
    lr = 1e-3
    mc.muon_momentum_ns_update_batched(M, G, W, lr, weight_decay=0.1, mu=0.95)
    torch.cuda.synchronize()
    rows_t = torch.from_numpy(sample).to(DEV)
    assert torch.equal(M[rows_t], G[rows_t])
    s = mc.muon_out_scale(rows, cols)
    got = -W[rows_t].double().cpu().numpy() / (lr * s)
    err = rel_fro(got, expect)
    say("  sampled rows, relative Frobenius error", f"{err:.2e}")
    assert err <= 2e-2, err
