"""The measurement aids of include/muonclip_probe.h on the GPU: the MFMA probe
runs and leaves finite checksums (zero operands give exactly zero), and the
copy probe copies every byte, including a ragged tail of whole 16-byte
vectors."""

import pytest
import torch

from gpu_helpers import say

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def mc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import muonclip_muon_amd
    return muonclip_muon_amd


def test_mfma_probe_checksums(mc):
    say("probe mfma")
    out, fl = mc.probe_mfma_bf16(16, 50, device=DEV)
    torch.cuda.synchronize()
    assert fl == 16 * 4 * 50 * 16 * 32768
    assert torch.isfinite(out).all() and out.abs().sum() > 0
    out0, _ = mc.probe_mfma_bf16(16, 50, zero_operands=True, device=DEV)
    torch.cuda.synchronize()
    assert (out0 == 0).all()


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (64 << 20) + 16 * 7])
def test_copy_probe_copies_every_byte(mc, nbytes):
    say("probe copy", nbytes)
    g = torch.Generator(device=DEV)
    g.manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=DEV, generator=g)
    dst = torch.zeros(nbytes + 32, dtype=torch.uint8, device=DEV)
    mc.probe_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src)
    assert (dst[nbytes:] == 0).all()
