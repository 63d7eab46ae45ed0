"""The C ABI driven from plain C: tests/c_client/step_client (built with the
library by muonclip_muon_amd/build.py) takes device memory and a stream from
the HIP runtime alone -- no Python, no torch -- and runs one MuonClip step:
the fused Muon call on a stack of float32 matrices, the per-head max logit
of bf16 Q, K (MLA: shared rotary key), and QK-Clip of float32 W_q, W_k.  Its
outputs are checked against the fp64 oracle on the same seeded inputs, at
the tolerances of the other parity tests: momentum bit-exact, the weight
update within the Newton-Schulz tolerance 2e-2, S_max within 1e-2 (bf16
inputs), the clip flags identical; gamma and the clipped rows, against the
oracle's clip from its own S_max, within S_max's measured relative error
(plus one float32 rounding), the unclipped heads' rows untouched.
"""

import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import f64, rel_err, rel_fro, say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLIENT = os.path.join(ROOT, "tests", "c_client", "step_client")


def test_one_step_from_a_c_client(tmp_path):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(CLIENT), "tests/c_client/step_client is not built (python muonclip_muon_amd/build.py)"
    say("C client step")
    batch, rows, cols = 3, 96, 320
    B, H, S, dc, dr = 2, 4, 128, 128, 64
    qph, qc, kph, d_in = 12, 8, 8, 32
    g = workloads.generator(500, "cpu")
    M = workloads.normal((batch, rows, cols), 1e-3, g, "cpu")
    G = workloads.normal((batch, rows, cols), 1e-3, g, "cpu")
    W = workloads.normal((batch, rows, cols), 0.02, g, "cpu")
    Q = workloads.normal((B, H, S, dc + dr), 1.0, g, "cpu", torch.bfloat16)
    Kc = workloads.normal((B, H, S, dc), 1.0, g, "cpu", torch.bfloat16)
    Kr = workloads.normal((B, S, dr), 1.0, g, "cpu", torch.bfloat16)
    Q[:, 0] = (Q[:, 0].float() * 40).to(torch.bfloat16)   # head 0 at S about 165
    Q[:, 2] = (Q[:, 2].float() * 30).to(torch.bfloat16)   # head 2 at S about 124; the others about 4
    Wq = workloads.normal((H * qph, d_in), 0.02, g, "cpu")
    Wk = workloads.normal((H * kph, d_in), 0.02, g, "cpu")

    hdr = np.array([batch, rows, cols, B, H, S, S, dc, dr, qph, qc, kph, d_in], dtype=np.int64)
    inp, outp = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as f:
        f.write(hdr.tobytes())
        for t in (M, G, W):
            f.write(t.numpy().astype(np.float32).tobytes())
        for t in (Q, Kc, Kr):
            f.write(t.view(torch.int16).numpy().tobytes())
        for t in (Wq, Wk):
            f.write(t.numpy().astype(np.float32).tobytes())
    r = subprocess.run([CLIENT, str(inp), str(outp)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    raw = open(outp, "rb").read()
    sizes = [batch * rows * cols, batch * rows * cols, H, H, H, H * qph * d_in, H * kph * d_in]
    parts, o = [], 0
    for k, n in enumerate(sizes):
        dt = np.int32 if k == 4 else np.float32
        parts.append(np.frombuffer(raw, dtype=dt, count=n, offset=o))
        o += 4 * n
    assert o == len(raw)
    M1, W1, smax, gamma, clipped, Wq1, Wk1 = parts

    # Muon part against the oracle
    ref_m = oracle.momentum_update(M.numpy(), G.numpy(), 0.95)
    np.testing.assert_array_equal(M1.reshape(batch, rows, cols), ref_m)
    for b in range(batch):
        O = oracle.muon_orthogonalised_update(ref_m[b].astype(np.float64))
        ref_w = oracle.apply_update(f64(W[b]), O, 2e-3, 0.1, "f32")
        got_w = W1.reshape(batch, rows, cols)[b].astype(np.float64)
        assert rel_fro(got_w - f64(W[b]), ref_w - f64(W[b])) <= 2e-2, b
    # max logit, the clip decision and the clipped rows, against the oracle's
    # own S_max: gamma and the rows then differ from the oracle's by S_max's
    # relative error (gamma^alpha by alpha times it), plus one float32 rounding
    ref_s = oracle.max_logit(Q.float().numpy(), Kc.float().numpy(), Kr.float().numpy())
    e_s = rel_err(smax, ref_s).max()
    assert e_s <= 1e-2
    rq, rk, ref_g, ref_c = oracle.qk_clip(ref_s, f64(Wq), f64(Wk), qph, qc, kph, w_dtype="f32")
    assert clipped.tolist() == ref_c.tolist() and clipped.tolist() == [1, 0, 1, 0]
    assert rel_err(gamma, ref_g).max() <= e_s + 1e-6
    tol = e_s + 2.0 ** -23
    for got, ref, src in ((Wq1.reshape(H * qph, d_in), rq, f64(Wq)), (Wk1.reshape(H * kph, d_in), rk, f64(Wk))):
        assert np.all(np.abs(got - ref) <= tol * np.abs(ref) + 1e-30)
        rows = got.shape[0] // H
        for h in (1, 3):  # unclipped heads: untouched, bit for bit
            assert np.array_equal(got[h * rows:(h + 1) * rows], src[h * rows:(h + 1) * rows].astype(np.float32))
