"""GPU parity of every step against the fp64 oracle, on seeded inputs at sizes
the oracle finishes in seconds (several tiles, ragged tails, edge cases).

Tolerances: momentum bit-exact; update and rescale within 1 bf16 ulp (2 float32
ulps for float32 weights) and bit-exact for untouched heads; S_max and gamma
relative error <= 1e-2 for bf16 inputs and <= 1e-5 for float32; clipped sets
identical; Newton-Schulz relative Frobenius error <= 2e-2.
"""

import math

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


# ------------------------------------------------------------------ momentum --
@pytest.mark.parametrize("numel,offset", [(1, 0), (7, 0), (4099, 1), (1 << 20, 0), (1_000_003, 3)])
def test_momentum_bitexact(mc, numel, offset):
    say("momentum", numel, offset)
    g = workloads.generator(100 + numel % 97, "cpu")
    M = workloads.normal((numel + offset,), 1e-3, g, "cpu")
    G = workloads.normal((numel + offset,), 1e-3, g, "cpu")
    Md, Gd = M.to(DEV), G.to(DEV)
    mc.muonclip_momentum(Md[offset:], Gd[offset:], 0.95)
    torch.cuda.synchronize()
    ref = oracle.momentum_update(M[offset:].numpy(), G[offset:].numpy(), 0.95)
    np.testing.assert_array_equal(Md[offset:].cpu().numpy(), ref)
    np.testing.assert_array_equal(Md[:offset].cpu().numpy(), M[:offset].numpy())  # untouched head


def test_momentum_zero_state_and_mu_zero(mc):
    say("momentum special cases")
    g = workloads.generator(5, "cpu")
    G = workloads.normal((10_000,), 1.0, g, "cpu")
    M = torch.zeros(10_000, device=DEV)
    mc.muonclip_momentum(M, G.to(DEV), 0.95)
    assert torch.equal(M.cpu(), G)
    M2 = workloads.normal((10_000,), 1.0, g, "cpu").to(DEV)
    mc.muonclip_momentum(M2, G.to(DEV), 0.0)
    assert torch.equal(M2.cpu(), G)


# ------------------------------------------------------------------ update --
@pytest.mark.parametrize("wdt,odt", [(torch.bfloat16, torch.bfloat16), (torch.float32, torch.float32),
                                     (torch.bfloat16, torch.float32), (torch.float32, torch.bfloat16)])
@pytest.mark.parametrize("numel,lr", [(100_003, 2e-4), (4096, 0.02), (5, 0.02)])
def test_update(mc, wdt, odt, numel, lr):
    say("update", wdt, odt, numel, lr)
    g = workloads.generator(7, "cpu")
    W = workloads.normal((numel,), 0.02, g, "cpu", wdt)
    O = workloads.normal((numel,), 0.2, g, "cpu", odt)
    Wd = W.to(DEV)
    mc.muon_apply_update(Wd, O.to(DEV), lr, 0.1)
    torch.cuda.synchronize()
    wname = "bf16" if wdt == torch.bfloat16 else "f32"
    ref = oracle.apply_update(f64(W), f64(O), lr, 0.1, wname)
    if wname == "bf16":
        d = bf16_ulp_diff(bf16_bits(Wd), oracle.bf16_bits(ref))
        assert d.max() <= 1
        assert np.mean(d == 0) > 0.99
    else:
        # float32: t = wd*w, s = o + t, v = lr*s, r = w - v each round once
        # (u = 2^-24 relative), so |r - exact| <= u (|r| + 2|v| + lr*wd*|w|);
        # the oracle's single rounding adds u |r|.  Ulps of r are the wrong
        # yardstick: w - v cancels.
        w64, o64 = f64(W), f64(O)
        v = np.abs(lr * (o64 + 0.1 * w64))
        bound = 2.0 ** -24 * (2 * np.abs(ref) + 2 * v + lr * 0.1 * np.abs(w64)) * 1.01 + 1e-45
        assert np.all(np.abs(f64(Wd) - ref) <= bound)


def test_update_lr_zero_is_bitwise(mc):
    say("update lr=0")
    g = workloads.generator(8, "cpu")
    W = workloads.normal((9999,), 0.02, g, "cpu", torch.bfloat16).to(DEV)
    O = workloads.normal((9999,), 0.2, g, "cpu", torch.bfloat16).to(DEV)
    before = W.clone()
    mc.muon_apply_update(W, O, 0.0, 0.1)
    assert torch.equal(W.view(torch.int16), before.view(torch.int16))


# ------------------------------------------------------------------ QK-Clip --
@pytest.mark.parametrize("wdt", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("d_in", [256, 136])
def test_qk_clip_mla(mc, wdt, d_in):
    say("qk_clip", wdt, d_in)
    H, dc, dr = 8, 8, 4
    qph, kph = dc + dr, dc
    g = workloads.generator(9, "cpu")
    Wq = workloads.normal((H * qph, d_in), 0.02, g, "cpu", wdt)
    Wk = workloads.normal((H * kph, d_in), 0.02, g, "cpu", wdt)
    smax = torch.tensor([523.25, 100.0, float("nan"), -3.0, 1e4, 99.99, 100.0001, 250.0], dtype=torch.float32)
    Wqd, Wkd = Wq.to(DEV), Wk.to(DEV)
    gamma, clipped = mc.qk_clip_apply(smax.to(DEV), Wqd, Wkd, qph, dc, kph, tau=100.0, alpha=0.5)
    torch.cuda.synchronize()
    wname = "bf16" if wdt == torch.bfloat16 else "f32"
    rq, rk, rg, rc = oracle.qk_clip(f64(smax), f64(Wq), f64(Wk), qph, dc, kph, 100.0, 0.5, wname)
    assert clipped.cpu().tolist() == rc.tolist()
    assert rel_err(gamma.cpu().numpy(), rg).max() <= 1e-6
    for got, ref, src, rows in ((Wqd, rq, Wq, qph), (Wkd, rk, Wk, kph)):
        for h in range(H):
            sl = slice(h * rows, (h + 1) * rows)
            if rc[h] != 1:
                assert torch.equal(got[sl].cpu().view(torch.int16 if wname == "bf16" else torch.int32),
                                   src[sl].view(torch.int16 if wname == "bf16" else torch.int32))
            elif wname == "bf16":
                assert bf16_ulp_diff(bf16_bits(got[sl]), oracle.bf16_bits(ref[sl])).max() <= 1
            else:
                assert f32_ulp_diff(got[sl].cpu().numpy(), ref[sl]).max() <= 2


def test_qk_clip_mha_general_alpha(mc):
    say("qk_clip MHA alpha=0.3")
    H, hd, d_in = 4, 16, 64
    g = workloads.generator(10, "cpu")
    Wq = workloads.normal((H * hd, d_in), 0.05, g, "cpu")
    Wk = workloads.normal((H * hd, d_in), 0.05, g, "cpu")
    smax = torch.tensor([300.0, 50.0, 1000.0, 100.0])
    Wqd, Wkd = Wq.to(DEV), Wk.to(DEV)
    gamma, clipped = mc.qk_clip_apply(smax.to(DEV), Wqd, Wkd, hd, hd, hd, tau=100.0, alpha=0.3)
    rq, rk, rg, rc = oracle.qk_clip(f64(smax), f64(Wq), f64(Wk), hd, hd, hd, 100.0, 0.3, "f32")
    assert clipped.cpu().tolist() == rc.tolist()
    assert f32_ulp_diff(Wqd.cpu().numpy(), rq).max() <= 4  # powf is within a few ulps
    assert f32_ulp_diff(Wkd.cpu().numpy(), rk).max() <= 4


@pytest.mark.parametrize("H", [300, 1024, 1100])
def test_qk_clip_many_heads(mc, H):
    """Head lists longer than one 256-thread round (compact kernel up to 1024
    heads) and the per-head grid beyond that; about a third of the heads
    clipped, some NaN."""
    say("qk_clip heads", H)
    qph, q_c, kph, d_in = 3, 2, 2, 64
    g = workloads.generator(12, "cpu")
    Wq = workloads.normal((H * qph, d_in), 0.02, g, "cpu", torch.bfloat16)
    Wk = workloads.normal((H * kph, d_in), 0.02, g, "cpu", torch.bfloat16)
    smax = torch.rand(H, generator=g) * 150.0
    smax[::97] = float("nan")
    Wqd, Wkd = Wq.to(DEV), Wk.to(DEV)
    gamma, clipped = mc.qk_clip_apply(smax.to(DEV), Wqd, Wkd, qph, q_c, kph, tau=100.0, alpha=0.5)
    torch.cuda.synchronize()
    rq, rk, rg, rc = oracle.qk_clip(f64(smax), f64(Wq), f64(Wk), qph, q_c, kph, 100.0, 0.5, "bf16")
    assert clipped.cpu().tolist() == rc.tolist()
    assert 0 < int((rc == 1).sum()) < H
    assert rel_err(gamma.cpu().numpy(), rg).max() <= 1e-6
    assert bf16_ulp_diff(bf16_bits(Wqd), oracle.bf16_bits(rq)).max() <= 1
    assert bf16_ulp_diff(bf16_bits(Wkd), oracle.bf16_bits(rk)).max() <= 1
    for got, src, rows in ((Wqd, Wq, qph), (Wkd, Wk, kph)):
        keep = torch.from_numpy(rc != 1).repeat_interleave(rows)
        assert torch.equal(got.cpu()[keep].view(torch.int16), src[keep].view(torch.int16))


@pytest.mark.parametrize("wdt", [torch.bfloat16, torch.float32])
def test_qk_clip_total(mc, wdt):
    say("qk_clip total", wdt)
    H, dc, dr, d_in = 8, 8, 4, 136
    qph, kph = dc + dr, dc
    g = workloads.generator(11, "cpu")
    Wq = workloads.normal((H * qph, d_in), 0.02, g, "cpu", wdt)
    Wk = workloads.normal((H * kph, d_in), 0.02, g, "cpu", wdt)
    wname = "bf16" if wdt == torch.bfloat16 else "f32"
    ibits = torch.int16 if wname == "bf16" else torch.int32
    nan = float("nan")
    for vals in ([523.25, 100.0, nan, -3.0, 1e4, 99.99, 100.0001, 250.0],  # largest 1e4: all clipped
                 [100.0, 3.0, -5.0, 99.0, 1.0, 2.0, 3.0, 4.0],             # largest at tau: none
                 [nan] * 8):                                               # all NaN: none, flagged
        smax = torch.tensor(vals, dtype=torch.float32)
        Wqd, Wkd = Wq.to(DEV), Wk.to(DEV)
        gamma, clipped = mc.qk_clip_apply_total(smax.to(DEV), Wqd, Wkd, qph, dc, kph, tau=100.0, alpha=0.5)
        torch.cuda.synchronize()
        rq, rk, rg, rc = oracle.qk_clip_total(f64(smax), f64(Wq), f64(Wk), qph, dc, kph, 100.0, 0.5, wname)
        assert clipped.cpu().tolist() == rc.tolist()
        assert rel_err(gamma.cpu().numpy(), rg).max() <= 1e-6
        for got, ref, src in ((Wqd, rq, Wq), (Wkd, rk, Wk)):
            if rc[0] != 1:
                assert torch.equal(got.cpu().view(ibits), src.view(ibits))
            elif wname == "bf16":
                assert bf16_ulp_diff(bf16_bits(got), oracle.bf16_bits(ref)).max() <= 1
            else:
                assert f32_ulp_diff(got.cpu().numpy(), ref).max() <= 2


# ------------------------------------------------------------------ max logit --
MAXLOGIT_CASES = [
    # (dtype, B, H, Sq, Sk, d_c, d_r): MFMA path (d in 64/128/192) and generic path
    (torch.bfloat16, 2, 3, 130, 200, 128, 64),
    (torch.bfloat16, 1, 2, 513, 65, 64, 0),
    (torch.bfloat16, 1, 2, 1024, 1024, 128, 0),
    (torch.bfloat16, 1, 1, 1, 1, 128, 64),
    (torch.bfloat16, 1, 2, 300, 333, 192, 0),  # 384-byte key rows
    (torch.bfloat16, 2, 2, 200, 129, 64, 64),  # 128-byte rows in both key parts
    (torch.bfloat16, 2, 2, 77, 90, 64, 16),   # d = 80: generic kernel
    (torch.float32, 2, 4, 128, 128, 64, 0),   # the tiny fp32 attention layer's shape
    (torch.float32, 1, 3, 100, 37, 96, 32),
]


@pytest.mark.parametrize("case", MAXLOGIT_CASES)
def test_maxlogit(mc, case):
    dt, B, H, Sq, Sk, dc, dr = case
    say("maxlogit", case)
    g = workloads.generator(11 + Sq, "cpu")
    Q = workloads.normal((B, H, Sq, dc + dr), 1.0, g, "cpu", dt)
    Kc = workloads.normal((B, H, Sk, dc), 1.0, g, "cpu", dt)
    Kr = workloads.normal((B, Sk, dr), 1.0, g, "cpu", dt) if dr else None
    s = mc.qk_maxlogit(Q.to(DEV), Kc.to(DEV), Kr.to(DEV) if dr else None)
    torch.cuda.synchronize()
    ref = oracle.max_logit(f64(Q), f64(Kc), f64(Kr) if dr else None)
    err = rel_err(s.cpu().numpy(), ref)
    bound = 1e-2 if dt == torch.bfloat16 else 1e-5
    assert err.max() <= bound, (err, s.cpu().numpy(), ref)
    assert err.max() <= 1e-4  # float32 accumulation of exact bf16 products is far tighter


def test_maxlogit_accumulate_over_batch_split(mc):
    say("maxlogit accumulate")
    g = workloads.generator(12, "cpu")
    Q = workloads.normal((4, 2, 256, 192), 1.0, g, "cpu", torch.bfloat16).to(DEV)
    Kc = workloads.normal((4, 2, 256, 128), 1.0, g, "cpu", torch.bfloat16).to(DEV)
    Kr = workloads.normal((4, 256, 64), 1.0, g, "cpu", torch.bfloat16).to(DEV)
    whole = mc.qk_maxlogit(Q, Kc, Kr)
    part = mc.qk_maxlogit(Q[:1].contiguous(), Kc[:1].contiguous(), Kr[:1].contiguous())
    mc.qk_maxlogit(Q[1:].contiguous(), Kc[1:].contiguous(), Kr[1:].contiguous(), smax=part, accumulate=True)
    assert torch.equal(whole, part)


def test_maxlogit_nan_is_skipped(mc):
    say("maxlogit NaN")
    g = workloads.generator(13, "cpu")
    Q = workloads.normal((1, 2, 128, 64), 1.0, g, "cpu", torch.bfloat16)
    Kc = workloads.normal((1, 2, 128, 64), 1.0, g, "cpu", torch.bfloat16)
    Q[0, 0, 5, 3] = float("nan")
    Q[0, 1] = float("nan")
    s = mc.qk_maxlogit(Q.to(DEV), Kc.to(DEV)).cpu().numpy()
    ref = oracle.max_logit(f64(Q), f64(Kc))
    assert ref[1] == -np.inf and s[1] == -np.inf
    assert rel_err(s[:1], ref[:1]).max() <= 1e-4


@pytest.mark.parametrize("dtype,d_c,d_r,Sk", [(torch.float32, 64, 0, 128), (torch.float32, 48, 16, 100),
                                              (torch.bfloat16, 40, 0, 70)])
def test_maxlogit_nan_is_skipped_generic_kernel(mc, dtype, d_c, d_r, Sk):
    """The same on the float32 LDS-tiled kernel (float32 inputs and head dims
    the MFMA kernel does not take), which is built with IEEE NaN semantics."""
    say("maxlogit NaN, generic kernel", dtype, d_c, d_r, Sk)
    g = workloads.generator(14 + d_c, "cpu")
    Q = workloads.normal((2, 3, 90, d_c + d_r), 1.0, g, "cpu", dtype)
    Kc = workloads.normal((2, 3, Sk, d_c), 1.0, g, "cpu", dtype)
    Kr = workloads.normal((2, Sk, d_r), 1.0, g, "cpu", dtype) if d_r else None
    Q[1, 0, 7, 2] = float("nan")      # one NaN row of logits in head 0
    Kc[0, 2, 11, 0] = float("nan")    # one NaN key in head 2
    Q[:, 1] = float("nan")            # head 1: every logit NaN
    s = mc.qk_maxlogit(Q.to(DEV), Kc.to(DEV), Kr.to(DEV) if Kr is not None else None).cpu().numpy()
    ref = oracle.max_logit(f64(Q), f64(Kc), f64(Kr) if Kr is not None else None)
    assert ref[1] == -np.inf and s[1] == -np.inf
    keep = [0, 2]
    assert np.all(np.isfinite(s[keep]))
    assert rel_err(s[keep], ref[keep]).max() <= (1e-5 if dtype == torch.float32 else 1e-4)


def test_maxlogit_signed_and_closed_form(mc):
    say("maxlogit closed form")
    d, S, c = 64, 96, 3.0
    Q = torch.zeros(1, 1, S, d)
    K = torch.zeros(1, 1, S, d)
    for i in range(S):
        Q[0, 0, i, i % d] = c
        K[0, 0, i, (i + 1) % d] = c
    s = mc.qk_maxlogit(Q.to(DEV, torch.bfloat16), K.to(DEV, torch.bfloat16)).item()
    assert s == pytest.approx(c * c / math.sqrt(d), rel=1e-6)
    s = mc.qk_maxlogit(torch.ones(1, 1, S, d, device=DEV, dtype=torch.bfloat16),
                       -torch.ones(1, 1, S, d, device=DEV, dtype=torch.bfloat16)).item()
    assert s == pytest.approx(-d / math.sqrt(d), rel=1e-6)  # signed max, no abs


# ------------------------------------------------------------------ Newton-Schulz --
NS_CASES = [
    # (batch, rows, cols, M dtype, O dtype)
    (1, 256, 256, torch.float32, torch.float32),
    (3, 200, 300, torch.bfloat16, torch.bfloat16),
    (2, 300, 200, torch.float32, torch.bfloat16),   # rows > cols: transposed path
    (1, 64, 7168, torch.float32, torch.bfloat16),   # the shared rotary key projection's shape
    (2, 512, 1792, torch.float32, torch.bfloat16),
    (1, 1, 40, torch.float32, torch.float32),
    (1, 600, 1000, torch.float32, torch.bfloat16),  # 3 x 3 tile grid: mirrored off-diagonal tiles
    (2, 1100, 700, torch.bfloat16, torch.float32),  # transposed, 3 x 3 grid, ragged padding
    # 16-byte vector and element-wise variants of the pre-scale and output copies
    (2, 256, 1024, torch.bfloat16, torch.float32),  # bf16 M, vector loads; float32 O, vector stores
    (1, 700, 96, torch.bfloat16, torch.bfloat16),   # transposed, vector paths
    (1, 130, 50, torch.float32, torch.bfloat16),    # transposed, element-wise paths
]


@pytest.mark.parametrize("case", NS_CASES)
def test_newton_schulz(mc, case):
    batch, rows, cols, mdt, odt = case
    say("newton-schulz", case)
    g = workloads.generator(20 + rows, "cpu")
    M = workloads.normal((batch, rows, cols), 1e-3, g, "cpu", mdt)
    scale = mc.muon_out_scale(rows, cols)
    O = mc.muon_ns_orthogonalize_batched(M.to(DEV), out_scale=scale, out_dtype=odt)
    torch.cuda.synchronize()
    for b in range(batch):
        ref = oracle.muon_orthogonalised_update(f64(M[b]))
        err = rel_fro(f64(O[b]), ref)
        assert err <= 2e-2, (b, err)


@pytest.mark.parametrize("rows,cols,odt", [(192, 320, torch.bfloat16), (320, 192, torch.bfloat16),
                                           (320, 192, torch.float32)])
def test_newton_schulz_misaligned(mc, rows, cols, odt):
    """M and O that start one element past a 16-byte boundary (row length a
    multiple of 8): the pre-scale and the output epilogue (straight and, for
    a tall matrix, transposed) must fall back to element-wise access."""
    say("newton-schulz misaligned", rows, cols, odt)
    batch = 2
    g = workloads.generator(77, "cpu")
    M = workloads.normal((batch, rows, cols), 1e-3, g, "cpu", torch.float32)
    Mbuf = torch.zeros(batch * rows * cols + 1, device=DEV)
    Mbuf[1:] = M.reshape(-1).to(DEV)
    Obuf = torch.full((batch * rows * cols + 1,), 7.0, device=DEV, dtype=odt)
    Mv = Mbuf[1:].view(batch, rows, cols)
    Ov = Obuf[1:].view(batch, rows, cols)
    scale = mc.muon_out_scale(rows, cols)
    mc.muon_ns_orthogonalize_batched(Mv, Ov, out_scale=scale)
    torch.cuda.synchronize()
    assert Obuf[0].item() == 7.0
    for b in range(batch):
        ref = oracle.muon_orthogonalised_update(f64(M[b]))
        assert rel_fro(f64(Ov[b]), ref) <= 2e-2


@pytest.mark.parametrize("case", [
    # (batch, rows, cols, O dtype, steps): with one step the first GEMMs'
    # normalisation and the output epilogue are the same launch
    (2, 300, 520, torch.float32, 1),
    (1, 520, 300, torch.bfloat16, 1),
    (2, 256, 768, torch.bfloat16, 2),
])
def test_newton_schulz_few_steps(mc, case):
    batch, rows, cols, odt, steps = case
    say("newton-schulz few steps", case)
    g = workloads.generator(40 + rows + steps, "cpu")
    M = workloads.normal((batch, rows, cols), 1e-3, g, "cpu", torch.float32)
    coeffs = mc.NS_COEFFS[:steps]
    scale = mc.muon_out_scale(rows, cols)
    O = mc.muon_ns_orthogonalize_batched(M.to(DEV), steps=steps, coeffs=coeffs, out_scale=scale, out_dtype=odt)
    torch.cuda.synchronize()
    for b in range(batch):
        ref = oracle.muon_orthogonalised_update(f64(M[b]), coeffs=coeffs)
        assert rel_fro(f64(O[b]), ref) <= 2e-2, b


@pytest.mark.parametrize("rows,cols", [(384, 640), (700, 260)])
def test_newton_schulz_cubic_ten_steps(mc, rows, cols):
    """Another polynomial through the same kernels: the textbook cubic
    p(x) = 1.5 x - 0.5 x^3 (c = 0, so B = b A) for 10 steps, against the
    oracle with the same coefficients."""
    say("newton-schulz cubic x10", rows, cols)
    g = workloads.generator(70 + rows, "cpu")
    M = workloads.normal((2, rows, cols), 1e-3, g, "cpu")
    coeffs = ((1.5, -0.5, 0.0),) * 10
    O = mc.muon_ns_orthogonalize_batched(M.to(DEV), steps=10, coeffs=coeffs, out_scale=1.0,
                                         out_dtype=torch.float32)
    torch.cuda.synchronize()
    for b in range(2):
        ref = oracle.newton_schulz(f64(M[b]), coeffs=coeffs)
        assert rel_fro(f64(O[b]), ref) <= 2e-2, b


def test_newton_schulz_output_over_input(mc):
    """O may be M's own buffer (same dtype and strides): M is read only by the
    pre-scale, before the last step writes O."""
    say("newton-schulz O = M")
    batch, rows, cols = 2, 384, 640
    g = workloads.generator(61, "cpu")
    M = workloads.normal((batch, rows, cols), 1e-3, g, "cpu", torch.float32)
    Md = M.to(DEV)
    scale = mc.muon_out_scale(rows, cols)
    mc.muon_ns_orthogonalize_batched(Md, Md, out_scale=scale)
    torch.cuda.synchronize()
    for b in range(batch):
        ref = oracle.muon_orthogonalised_update(f64(M[b]))
        assert rel_fro(f64(Md[b]), ref) <= 2e-2, b


FUSED_CASES = [
    # (batch, rows, cols, W dtype, NS steps)
    (2, 256, 512, torch.bfloat16, 5),   # vector paths throughout
    (3, 200, 328, torch.float32, 5),    # ragged padding; cols % 8 != 0: element-wise momentum pass
    (2, 300, 200, torch.bfloat16, 5),   # rows > cols: iterated on M^T, W updated transposed
    (1, 130, 50, torch.float32, 5),     # tall and ragged
    (2, 257, 330, torch.bfloat16, 5),   # cols % 4 != 0: element-wise W update
    (1, 600, 1000, torch.bfloat16, 1),  # one step: the normalising step is also the updating one
]


@pytest.mark.parametrize("case", FUSED_CASES)
def test_fused_momentum_ns_update(mc, case):
    """muon_momentum_ns_update_batched against the oracle's momentum (bit-exact),
    Newton-Schulz and update.  lr is large for bf16 W so that the update, not
    W's own rounding, dominates W_t - W_{t-1}."""
    batch, rows, cols, wdt, steps = case
    say("fused momentum + NS + update", case)
    g = workloads.generator(90 + rows + cols, "cpu")
    M0 = workloads.normal((batch, rows, cols), 1e-3, g, "cpu", torch.float32)
    G = workloads.normal((batch, rows, cols), 1e-3, g, "cpu", torch.float32)
    W0 = workloads.normal((batch, rows, cols), 0.02, g, "cpu", wdt)
    lr = 1.0 if wdt == torch.bfloat16 else 0.02
    coeffs = mc.NS_COEFFS[:steps]
    M, W = M0.to(DEV), W0.to(DEV)
    mc.muon_momentum_ns_update_batched(M, G.to(DEV), W, lr, 0.1, 0.95, steps=steps, coeffs=coeffs)
    torch.cuda.synchronize()
    M_ref = oracle.momentum_update(M0.numpy(), G.numpy(), 0.95)
    np.testing.assert_array_equal(M.cpu().numpy(), M_ref)
    wname = "bf16" if wdt == torch.bfloat16 else "f32"
    for b in range(batch):
        O_ref = oracle.muon_orthogonalised_update(M_ref[b].astype(np.float64), coeffs=coeffs)
        W_ref = oracle.apply_update(f64(W0[b]), O_ref, lr, 0.1, wname)
        d_gpu = f64(W[b]) - f64(W0[b])
        d_ref = W_ref - f64(W0[b])
        err = rel_fro(d_gpu, d_ref)
        assert err <= 2e-2, (b, err)


def test_fused_matches_separate_calls(mc):
    """The fused call and momentum + NS + update as three calls agree to the
    Newton-Schulz tolerance (same M bit for bit)."""
    say("fused vs separate calls")
    batch, rows, cols = 2, 512, 1024
    g = workloads.generator(5150, "cpu")
    M0 = workloads.normal((batch, rows, cols), 1e-3, g, "cpu", torch.float32).to(DEV)
    G = workloads.normal((batch, rows, cols), 1e-3, g, "cpu", torch.float32).to(DEV)
    W0 = workloads.normal((batch, rows, cols), 0.02, g, "cpu", torch.float32).to(DEV)
    M1, W1 = M0.clone(), W0.clone()
    mc.muon_momentum_ns_update_batched(M1, G, W1, 0.02, 0.1, 0.95)
    M2, W2 = M0.clone(), W0.clone()
    mc.muonclip_momentum(M2, G, 0.95)
    O = mc.muon_ns_orthogonalize_batched(M2, out_scale=mc.muon_out_scale(rows, cols), out_dtype=torch.float32)
    mc.muon_apply_update(W2, O, 0.02, 0.1)
    torch.cuda.synchronize()
    assert torch.equal(M1, M2)
    assert rel_fro(f64(W1 - W0), f64(W2 - W0)) <= 2e-2


def test_newton_schulz_zero_matrix(mc):
    say("newton-schulz zero")
    O = mc.muon_ns_orthogonalize_batched(torch.zeros(2, 64, 128, device=DEV), out_scale=2.0)
    assert torch.count_nonzero(O).item() == 0


def test_newton_schulz_non_finite_momentum(mc):
    """A NaN or an infinity in one matrix of a batch: that matrix's result is
    NaN everywhere, as the oracle's is (the norm is NaN or infinite, and the
    iteration spreads the non-finite entry to every element by its second
    product), and the batch's other matrices are untouched by it.  Checks
    that the carried low part never turns a non-finite value into a finite
    one, in the Newton-Schulz call and in the fused step."""
    say("newton-schulz non-finite momentum")
    g = workloads.generator(61, "cpu")
    M = workloads.normal((3, 256, 512), 1e-3, g, "cpu")
    M[1, 17, 300] = float("nan")
    M[2, 200, 5] = float("inf")
    O = mc.muon_ns_orthogonalize_batched(M.to(DEV), out_scale=1.0, out_dtype=torch.float32).cpu()
    with np.errstate(invalid="ignore"):  # inf / inf in the oracle's normalisation
        refs = [oracle.newton_schulz(f64(M[b])) for b in range(3)]
    assert np.isnan(refs[1]).all() and np.isnan(refs[2]).all()
    assert torch.isnan(O[1]).all() and torch.isnan(O[2]).all()
    assert torch.isfinite(O[0]).all() and rel_fro(f64(O[0]), refs[0]) <= 2e-2
    # the fused step: momentum element-wise, W of the non-finite matrices NaN
    W0 = workloads.normal((3, 256, 512), 0.02, g, "cpu", torch.bfloat16)
    Md, W = torch.zeros(3, 256, 512, device=DEV), W0.to(DEV)
    mc.muon_momentum_ns_update_batched(Md, M.to(DEV), W, 2e-2, 0.1, 0.95)
    Md, W = Md.cpu(), W.cpu().float()
    assert torch.isnan(Md[1, 17, 300]) and torch.isfinite(Md[1]).sum() == 256 * 512 - 1
    assert torch.isnan(W[1]).all() and torch.isnan(W[2]).all() and torch.isfinite(W[0]).all()


def test_newton_schulz_gemm_events(mc):
    say("newton-schulz events")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(6 * 5)]
    M = torch.randn(4, 256, 512, device=DEV)
    mc.muon_ns_orthogonalize_batched(M, gemm_events=ev)
    torch.cuda.synchronize()
    times = [ev[2 * k].elapsed_time(ev[2 * k + 1]) for k in range(15)]
    assert all(t > 0 for t in times)


# ------------------------------------------------------------------ whole step --
@pytest.mark.parametrize("reading", ["std", "variance"])
def test_full_step_tiny_attention(mc, reading):
    """One MuonClip step on the tiny fp32 attention layer (d_model 256, 4 heads of 64,
    lr 0.02, 5 NS steps, tau 100, alpha 0.5), GPU against the oracle."""
    say("full step tiny", reading)
    t = workloads.tiny_attention(seed=1, device="cpu", weight_reading=reading)
    H, hd = t.n_heads, t.head_dim
    Xd = t.X.to(DEV)
    W = {n: w.to(DEV) for n, w in t.W.items()}
    G = {n: g_.to(DEV) for n, g_ in t.G.items()}
    # forward at W_{t-1}: Q, K per head (harness projection on the device, an
    # input of both sides); S_max from the library for the library's step and
    # the oracle's own S_max of the same Q, K for the oracle's
    Qd = (Xd @ W["q"].t().contiguous()).view(2, 128, H, hd).transpose(1, 2).contiguous()
    Kd = (Xd @ W["k"].t().contiguous()).view(2, 128, H, hd).transpose(1, 2).contiguous()
    smax = mc.qk_maxlogit(Qd, Kd)
    ref_s = oracle.max_logit(f64(Qd), f64(Kd))
    assert rel_err(smax.cpu().numpy(), ref_s).max() <= 1e-5
    att = dict(q="q", k="k", q_rows_per_head=hd, q_c_rows=hd, k_rows_per_head=hd)
    gamma, clipped = mc.muonclip_step(W, G, {}, smax, att, lr=0.02)
    torch.cuda.synchronize()
    new_w, _, rg, rc = oracle.muonclip_step({n: f64(w) for n, w in t.W.items()},
                                            {n: g_.numpy() for n, g_ in t.G.items()}, {},
                                            ref_s, att, lr=0.02, w_dtype="f32")
    assert clipped.cpu().tolist() == rc.tolist()
    if reading == "variance":
        assert rc[0] == 1  # head 0 is clipped in this reading
    else:
        assert not np.any(rc == 1)  # std reading: every head stays under tau
    assert rel_err(gamma.cpu().numpy(), rg).max() <= 1e-5
    for n in ("q", "k", "v"):
        dg = f64(W[n]) - f64(t.W[n])
        do = new_w[n] - f64(t.W[n])
        assert rel_fro(dg, do) <= 2e-2, n


@pytest.mark.parametrize("reading", ["std", "variance"])
def test_full_step_tiny_attention_from_oracle_smax(mc, reading):
    """The tiny fp32 layer end to end with nothing shared between the two
    sides: the oracle projects Q, K itself (fp64, CPU), takes its own S_max and
    runs its own step; the GPU path projects on the device, measures S_max with
    qk_maxlogit and runs muonclip_step.  Clipped sets identical, gamma and
    S_max within 1e-5 relative, weight deltas within 2e-2."""
    say("full step tiny from the oracle's S_max", reading)
    t = workloads.tiny_attention(seed=1, device="cpu", weight_reading=reading)
    H, hd = t.n_heads, t.head_dim
    # the oracle's own forward
    Wn = {n: f64(w) for n, w in t.W.items()}
    rq = oracle.project_heads(f64(t.X), Wn["q"], H)
    rk = oracle.project_heads(f64(t.X), Wn["k"], H)
    ref_s = oracle.max_logit(rq, rk)
    att = dict(q="q", k="k", q_rows_per_head=hd, q_c_rows=hd, k_rows_per_head=hd)
    new_w, _, rg, rc = oracle.muonclip_step(Wn, {n: g_.numpy() for n, g_ in t.G.items()}, {}, ref_s, att,
                                            lr=0.02, w_dtype="f32")
    # the library's
    Xd = t.X.to(DEV)
    W = {n: w.to(DEV) for n, w in t.W.items()}
    G = {n: g_.to(DEV) for n, g_ in t.G.items()}
    Qd = (Xd @ W["q"].t().contiguous()).view(2, 128, H, hd).transpose(1, 2).contiguous()
    Kd = (Xd @ W["k"].t().contiguous()).view(2, 128, H, hd).transpose(1, 2).contiguous()
    smax = mc.qk_maxlogit(Qd, Kd)
    gamma, clipped = mc.muonclip_step(W, G, {}, smax, att, lr=0.02)
    torch.cuda.synchronize()
    assert rel_err(smax.cpu().numpy(), ref_s).max() <= 1e-5
    assert clipped.cpu().tolist() == rc.tolist()
    assert (rc[0] == 1) == (reading == "variance")
    assert rel_err(gamma.cpu().numpy(), rg).max() <= 1e-5
    for n in ("q", "k", "v"):
        assert rel_fro(f64(W[n]) - Wn[n], new_w[n] - Wn[n]) <= 2e-2, n


def test_binding_rejects_bad_tensors(mc):
    """Caller-supplied outputs of the wrong size, dtype or device, and inputs
    whose dtype differs from the one the call reads them in, raise before
    anything is launched (the kernels write exactly the call's element count,
    so a smaller tensor would be overrun); inputs stay untouched."""
    say("binding output validation")
    g = workloads.generator(62, "cpu")
    Q = workloads.normal((1, 4, 64, 192), 1.0, g, "cpu", torch.bfloat16).to(DEV)
    Kc = workloads.normal((1, 4, 64, 128), 1.0, g, "cpu", torch.bfloat16).to(DEV)
    Kr = workloads.normal((1, 64, 64), 1.0, g, "cpu", torch.bfloat16).to(DEV)
    V = workloads.normal((1, 4, 64, 128), 1.0, g, "cpu", torch.bfloat16).to(DEV)
    with pytest.raises(ValueError):
        mc.qk_maxlogit(Q, Kc, Kr, smax=torch.empty(3, device=DEV))
    with pytest.raises(ValueError):
        mc.qk_maxlogit(Q, Kc, Kr, smax=torch.empty(4, dtype=torch.float64, device=DEV))
    with pytest.raises(ValueError):
        mc.attention_fwd_maxlogit(Q, Kc, Kr, V, O=torch.empty(1, 4, 64, 64, dtype=torch.bfloat16, device=DEV))
    with pytest.raises(ValueError):
        mc.attention_fwd_maxlogit(Q, Kc, Kr, V, lse=torch.empty(1, 4, 32, device=DEV))
    with pytest.raises(ValueError):  # a one-byte key read as bf16 would run past its end
        mc.attention_fwd_maxlogit(Q, Kc.to(torch.float8_e4m3fn), Kr, V)
    with pytest.raises(ValueError):
        mc.attention_fwd_maxlogit(Q, Kc, Kr, V.float())
    Wq = workloads.normal((4 * 6, 32), 0.02, g, "cpu", torch.bfloat16).to(DEV)
    Wk = workloads.normal((4 * 4, 32), 0.02, g, "cpu", torch.bfloat16).to(DEV)
    before = (Wq.clone(), Wk.clone())
    smax = torch.full((4,), 1000.0, device=DEV)
    with pytest.raises(ValueError):
        mc.qk_clip_apply(smax, Wq, Wk, 6, 4, 4, gamma=torch.empty(2, device=DEV))
    with pytest.raises(ValueError):
        mc.qk_clip_apply(smax, Wq, Wk, 6, 4, 4, clipped=torch.empty(4, device=DEV))  # float32, not int32
    with pytest.raises(ValueError):
        mc.qk_clip_apply_layers(smax.view(1, 4), [Wq], [Wk], 6, 4, 4, gamma=torch.empty(1, 3, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(Wq, before[0]) and torch.equal(Wk, before[1])
