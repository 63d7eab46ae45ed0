"""Host-side checks of libmuonclip.so (no GPU): it loads, exports every entry
point include/*.h declares (the step in muonclip.h, the measurement aids in
muonclip_probe.h), and rejects invalid arguments before any HIP call
(argument validation never touches the device)."""

import ctypes
import glob
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "muonclip.h")
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))


def _declared():
    text = "".join(open(h).read() for h in HEADERS)
    return re.findall(r"MC_API\s+[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text)


@pytest.fixture(scope="module")
def mc():
    import muonclip_muon_amd
    return muonclip_muon_amd


def test_header_declares_the_entry_points():
    names = set(_declared())
    assert {"muonclip_momentum", "muon_ns_orthogonalize_batched", "muon_apply_update", "qk_maxlogit",
            "qk_clip_apply", "muon_ns_workspace_bytes", "mc_abi_version", "mc_status_string",
            "muon_momentum_ns_update_batched", "qk_clip_apply_total", "attention_fwd_maxlogit",
            "mc_probe_mfma_bf16", "mc_probe_copy"} <= names


def test_library_exports_every_declared_symbol(mc):
    for name in _declared():
        assert hasattr(mc.lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", mc.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert exported == set(_declared())  # nothing internal leaks


def test_abi_version_and_status_strings(mc):
    text = open(HEADER).read()
    assert mc.abi_version() == int(re.search(r"#define MC_ABI_VERSION (\d+)", text).group(1))
    for code in range(8):
        assert mc.lib.mc_status_string(code) != b"unknown status"
    assert mc.lib.mc_status_string(99) == b"unknown status"


def test_binding_constants_match_oracle_constants(mc):
    # The product and the oracle each define the Newton-Schulz constants; they
    # must agree (they share no code).
    import oracle
    assert tuple(mc.NS_COEFFS) == tuple(oracle.NS_COEFFS)
    assert mc.NS_EPS == oracle.NS_EPS and mc.NS_STEPS == oracle.NS_STEPS


EINVAL, ESHAPE, EDTYPE, EALIGN, EWORKSPACE = 1, 2, 3, 4, 5
FAKE = ctypes.c_void_p(0x100000)  # never dereferenced: every call below fails validation first


def test_momentum_validation(mc):
    L = mc.lib
    assert L.muonclip_momentum(None, None, 0, 0.95, None) == 0  # empty: nothing enqueued
    assert L.muonclip_momentum(None, FAKE, 8, 0.95, None) == EINVAL
    assert L.muonclip_momentum(FAKE, FAKE, -1, 0.95, None) == EINVAL
    assert L.muonclip_momentum(FAKE, FAKE, 8, float("nan"), None) == EINVAL
    assert L.muonclip_momentum(ctypes.c_void_p(0x100002), FAKE, 8, 0.95, None) == EALIGN


def test_ns_validation(mc):
    L = mc.lib
    coeffs = (ctypes.c_float * 15)(*([3.4445, -4.775, 2.0315] * 5))
    ws_bytes = L.muon_ns_workspace_bytes(4, 256, 512)
    assert ws_bytes > 0
    assert L.muon_ns_workspace_bytes(4, 0, 512) == 0
    assert L.muon_ns_workspace_bytes(1, 20000, 20000) == 0
    # batches beyond the grid limits: rejected before any size is computed
    # (a batch of 2^40 would wrap the byte count)
    assert L.muon_ns_workspace_bytes(65536, 256, 256) == 0
    assert L.muon_ns_workspace_bytes(1 << 40, 256, 256) == 0
    assert L.muon_ns_workspace_bytes(65535, 256, 256) > 0

    def call(**kw):
        a = dict(M=FAKE, m_dtype=1, batch=4, rows=256, cols=512, mstride=256 * 512, O=FAKE, o_dtype=1,
                 ostride=256 * 512, steps=5, coeffs=coeffs, eps=1e-7, scale=1.0, ws=ctypes.c_void_p(0x200000),
                 wsb=ws_bytes, stream=None, ev=None)
        a.update(kw)
        return L.muon_ns_orthogonalize_batched(a["M"], a["m_dtype"], a["batch"], a["rows"], a["cols"],
                                               a["mstride"], a["O"], a["o_dtype"], a["ostride"], a["steps"],
                                               a["coeffs"], a["eps"], a["scale"], a["ws"], a["wsb"],
                                               a["stream"], a["ev"])
    assert call(batch=0) == 0
    assert call(rows=0) == EINVAL
    assert call(m_dtype=7) == EDTYPE
    assert call(rows=20000, cols=20000) == ESHAPE
    assert call(batch=1 << 40, wsb=(1 << 64) - 1) == ESHAPE
    assert call(batch=65536, wsb=(1 << 64) - 1) == ESHAPE
    assert call(M=None) == EINVAL
    assert call(steps=0) == EINVAL
    assert call(eps=-1.0) == EINVAL
    assert call(mstride=10) == EINVAL
    assert call(ws=ctypes.c_void_p(0x200010)) == EALIGN
    assert call(wsb=ws_bytes - 1) == EWORKSPACE
    bad = (ctypes.c_float * 15)(*([float("inf")] * 15))
    assert call(coeffs=bad) == EINVAL


def test_fused_validation(mc):
    L = mc.lib
    coeffs = (ctypes.c_float * 15)(*([3.4445, -4.775, 2.0315] * 5))
    ws_bytes = L.muon_ns_workspace_bytes(4, 256, 512)

    def call(**kw):
        a = dict(M=FAKE, G=FAKE, mu=0.95, W=FAKE, w_dtype=1, batch=4, rows=256, cols=512, stride=256 * 512,
                 steps=5, coeffs=coeffs, eps=1e-7, scale=4.5, lr=0.02, wd=0.1, ws=ctypes.c_void_p(0x200000),
                 wsb=ws_bytes, stream=None, ev=None)
        a.update(kw)
        return L.muon_momentum_ns_update_batched(a["M"], a["G"], a["mu"], a["W"], a["w_dtype"], a["batch"],
                                                 a["rows"], a["cols"], a["stride"], a["steps"], a["coeffs"],
                                                 a["eps"], a["scale"], a["lr"], a["wd"], a["ws"], a["wsb"],
                                                 a["stream"], a["ev"])
    assert call(batch=0) == 0
    assert call(cols=0) == EINVAL
    assert call(w_dtype=3) == EDTYPE
    assert call(rows=70000, cols=8) == ESHAPE
    assert call(G=None) == EINVAL
    assert call(W=None) == EINVAL
    assert call(stride=100) == EINVAL
    assert call(mu=float("nan")) == EINVAL
    assert call(lr=float("inf")) == EINVAL
    assert call(steps=65) == EINVAL
    assert call(coeffs=None) == EINVAL
    assert call(M=ctypes.c_void_p(0x100002)) == EALIGN
    assert call(W=ctypes.c_void_p(0x100001)) == EALIGN
    assert call(ws=ctypes.c_void_p(0x200080)) == EALIGN
    assert call(wsb=ws_bytes - 1) == EWORKSPACE


def test_update_validation(mc):
    L = mc.lib
    assert L.muon_apply_update(FAKE, 1, FAKE, 1, 0, 0.02, 0.1, None) == 0
    assert L.muon_apply_update(FAKE, 5, FAKE, 1, 8, 0.02, 0.1, None) == EDTYPE
    assert L.muon_apply_update(None, 1, FAKE, 1, 8, 0.02, 0.1, None) == EINVAL
    assert L.muon_apply_update(FAKE, 1, FAKE, 1, 8, float("inf"), 0.1, None) == EINVAL
    assert L.muon_apply_update(ctypes.c_void_p(0x100001), 1, FAKE, 1, 8, 0.02, 0.1, None) == EALIGN


def test_maxlogit_validation(mc):
    L = mc.lib
    assert L.qk_maxlogit(FAKE, FAKE, FAKE, 1, 1, 0, 8, 8, 128, 64, FAKE, 0, None) == 0  # H = 0
    assert L.qk_maxlogit(FAKE, FAKE, None, 1, 1, 2, 8, 8, 128, 64, FAKE, 0, None) == EINVAL  # Kr missing
    assert L.qk_maxlogit(FAKE, FAKE, FAKE, 1, 1, 2, 8, 8, 128, 0, FAKE, 0, None) == EINVAL  # Kr given, d_r 0
    assert L.qk_maxlogit(FAKE, FAKE, None, 9, 1, 2, 8, 8, 64, 0, FAKE, 0, None) == EDTYPE
    assert L.qk_maxlogit(FAKE, FAKE, None, 1, 1, 2, 8, 8, 600, 0, FAKE, 0, None) == ESHAPE
    assert L.qk_maxlogit(FAKE, FAKE, None, 1, 1, 2, 8, 8, 64, 0, None, 0, None) == EINVAL
    assert L.qk_maxlogit(ctypes.c_void_p(0x100001), FAKE, None, 1, 1, 2, 8, 8, 64, 0, FAKE, 0, None) == EALIGN
    # element counts beyond any buffer (their products would leave int64)
    assert L.qk_maxlogit(FAKE, FAKE, None, 1, 60000, 60000, 1 << 30, 8, 64, 0, FAKE, 0, None) == ESHAPE


def test_attention_validation(mc):
    L = mc.lib
    # (Q, Kc, Kr, V, dtype, B, H, Sq, Sk, d_c, d_r, d_v, causal, O, lse, smax, accumulate, stream)
    ok = (FAKE, FAKE, FAKE, FAKE, 1, 1, 4, 256, 256, 128, 64, 128, 0, FAKE, None, FAKE, 0, None)

    def call(**kw):
        names = ["Q", "Kc", "Kr", "V", "dtype", "B", "H", "Sq", "Sk", "d_c", "d_r", "d_v", "causal", "O",
                 "lse", "smax", "acc", "stream"]
        args = dict(zip(names, ok))
        args.update(kw)
        return L.attention_fwd_maxlogit(*[args[n] for n in names])

    # no head: nothing is read or written, every pointer may be null
    assert call(Q=None, Kc=None, Kr=None, V=None, O=None, smax=None, H=0) == 0
    assert call(dtype=0) == EDTYPE                      # bf16 only
    assert call(d_c=96) == ESHAPE                       # head dims (128, 64, 128) or (64, 0, 64)
    assert call(Q=None) == EINVAL
    assert call(V=None) == EINVAL
    assert call(O=None) == EINVAL
    assert call(Kr=None) == EINVAL                      # d_r > 0 needs the rotary keys
    assert call(smax=None) == EINVAL
    assert call(smax=None, Sq=0) == EINVAL              # an empty call still writes S_max
    assert call(Sk=63) == ESHAPE                        # at least one key block
    assert call(causal=1, Sq=300, Sk=256) == ESHAPE     # causal needs Sq <= Sk
    assert call(B=-1) == EINVAL
    assert call(Q=ctypes.c_void_p(0x100008)) == EALIGN  # 16-byte operands
    assert call(O=ctypes.c_void_p(0x100004)) == EALIGN
    assert call(B=1 << 20, H=60000, Sq=1 << 30) == ESHAPE  # element counts beyond any buffer


@pytest.mark.parametrize("fn", ["qk_clip_apply", "qk_clip_apply_total"])
def test_clip_validation(mc, fn):
    f = getattr(mc.lib, fn)
    assert f(FAKE, 0, 100.0, 0.5, FAKE, FAKE, 1, 16, 6, 4, 4, None, None, None) == 0
    assert f(FAKE, 4, 0.0, 0.5, FAKE, FAKE, 1, 16, 6, 4, 4, None, None, None) == EINVAL
    assert f(FAKE, 4, float("inf"), 0.5, FAKE, FAKE, 1, 16, 6, 4, 4, None, None, None) == EINVAL
    assert f(FAKE, 4, 100.0, 1.5, FAKE, FAKE, 1, 16, 6, 4, 4, None, None, None) == EINVAL
    assert f(FAKE, 4, 100.0, 0.5, FAKE, FAKE, 1, 16, 6, 8, 4, None, None, None) == EINVAL
    assert f(FAKE, 4, 100.0, 0.5, FAKE, FAKE, 4, 16, 6, 4, 4, None, None, None) == EDTYPE
    assert f(None, 4, 100.0, 0.5, FAKE, FAKE, 1, 16, 6, 4, 4, None, None, None) == EINVAL
    assert f(FAKE, 4, 100.0, 0.5, ctypes.c_void_p(0x100001), FAKE, 1, 16, 6, 4, 4, None, None,
             None) == EALIGN
    # sizes whose products would leave int64 are shape errors (checked before
    # any is formed)
    assert f(FAKE, 4, 100.0, 0.5, FAKE, FAKE, 1, 1 << 40, 6, 4, 4, None, None, None) == ESHAPE
    assert f(FAKE, 4, 100.0, 0.5, FAKE, FAKE, 1, 16, 1 << 40, 4, 4, None, None, None) == ESHAPE
    assert f(FAKE, 4, 100.0, 0.5, FAKE, FAKE, 1, 16, 6, 4, 1 << 40, None, None, None) == ESHAPE


def test_probe_validation(mc):
    L = mc.lib
    assert L.mc_probe_mfma_bf16(0, 10, 0, FAKE, None) == EINVAL
    assert L.mc_probe_mfma_bf16(65537, 10, 0, FAKE, None) == EINVAL
    assert L.mc_probe_mfma_bf16(8, 0, 0, FAKE, None) == EINVAL
    assert L.mc_probe_mfma_bf16(8, (1 << 30) + 1, 0, FAKE, None) == EINVAL
    assert L.mc_probe_mfma_bf16(8, 10, 0, None, None) == EINVAL
    assert L.mc_probe_mfma_bf16(8, 10, 0, ctypes.c_void_p(0x100002), None) == EINVAL
    assert L.mc_probe_copy(FAKE, FAKE, 0, None) == 0  # empty: nothing enqueued
    assert L.mc_probe_copy(FAKE, FAKE, -16, None) == EINVAL
    assert L.mc_probe_copy(FAKE, FAKE, 24, None) == EINVAL
    assert L.mc_probe_copy(None, FAKE, 16, None) == EINVAL
    assert L.mc_probe_copy(ctypes.c_void_p(0x100008), FAKE, 16, None) == EALIGN


C_CLIENT = r"""
#include <stdio.h>
#include "muonclip.h"
#include "muonclip_probe.h"

int main(void) {
  /* plain C99 against the C ABI: version, status strings, validation paths
     (no device pointer is ever dereferenced: every call fails its checks
     or is empty) */
  if (mc_abi_version() != MC_ABI_VERSION) return 1;
  if (mc_status_string(MC_EINVAL) == NULL) return 2;
  if (muonclip_momentum(NULL, NULL, 0, 0.95f, NULL) != MC_OK) return 3;
  if (muonclip_momentum(NULL, NULL, 8, 0.95f, NULL) != MC_EINVAL) return 4;
  if (muon_ns_workspace_bytes(1, 0, 8) != 0) return 5;
  if (muon_ns_workspace_bytes(4, 256, 512) == 0) return 6;
  if (qk_clip_apply(NULL, 0, 100.0f, 0.5f, NULL, NULL, MC_BF16, 64, 3, 2, 2, NULL, NULL, NULL) != MC_OK) return 7;
  if (mc_probe_copy(NULL, NULL, 24, NULL) != MC_EINVAL) return 8;
  printf("ok\n");
  return 0;
}
"""


def test_headers_compile_as_c_and_link(mc, tmp_path):
    """The public headers are plain C: a C99 client compiles with -Wall
    -Werror, links against the library and runs its validation paths."""
    src = tmp_path / "client.c"
    src.write_text(C_CLIENT)
    exe = tmp_path / "client"
    libdir = os.path.dirname(mc.LIB_PATH)
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
                        str(src), "-o", str(exe), "-L", libdir, "-lmuonclip", "-Wl,-rpath," + libdir],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.returncode, r.stdout, r.stderr)


def test_rms_match_scale_in_the_library(mc):
    # O_t = NewtonSchulz(M_t) * sqrt(max(n, m)) * 0.2 (the internals page's
    # Algorithm 1; the Zhihu MuonClip formula): the factor comes from the C
    # library, rounded once to float32; 0.2 is the pages' constant.
    import json

    import numpy as np
    golden = json.load(open(os.path.join(ROOT, "tests", "golden", "page_constants.json")))
    k = float(golden["rms_match_factor"]["value"])
    for rows, cols in ((2048, 7168), (7168, 2048), (12288, 7168), (64, 7168), (256, 256), (1, 1), (3, 5)):
        want = np.float32(np.sqrt(float(max(rows, cols))) * k)
        assert mc.lib.muon_rms_match_scale(rows, cols) == want
        assert mc.muon_out_scale(rows, cols) == want
    assert mc.lib.muon_rms_match_scale(0, 7) == 0.0 and mc.lib.muon_rms_match_scale(7, -1) == 0.0
    assert mc.OUT_SCALE_RMS_MATCH < 0
    text = open(HEADER).read()
    assert float(re.search(r"#define MC_OUT_SCALE_RMS_MATCH \((-?[\d.]+)f\)", text).group(1)) < 0


def test_noalloc_validation(mc):
    # the allocation-free entry point rejects bad arguments and sizes beyond
    # its static scratch before any HIP call (no device is touched here)
    L = mc.lib
    coeffs = (ctypes.c_float * 15)(*([3.4445, -4.775, 2.0315] * 5))
    text = open(HEADER).read()
    limit = int(re.search(r"#define MC_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << 20\)", text).group(1)) << 20
    assert L.muon_ns_workspace_bytes(1, 2048, 7168) <= limit < L.muon_ns_workspace_bytes(4, 2048, 7168)
    args = (0.95, FAKE, 1, 4, 2048, 7168, 2048 * 7168, 5, coeffs, 1e-7, -1.0, 2e-4, 0.1, None)
    assert L.muon_momentum_ns_update_batched_noalloc(FAKE, FAKE, *args) == EWORKSPACE
    assert L.muon_momentum_ns_update_batched_noalloc(FAKE, FAKE, 0.95, FAKE, 1, 0, 256, 256, 0, 5, coeffs, 1e-7,
                                                     -1.0, 2e-4, 0.1, None) == 0  # empty batch: nothing enqueued
    assert L.muon_momentum_ns_update_batched_noalloc(FAKE, FAKE, 0.95, FAKE, 1, 1, 0, 256, 0, 5, coeffs, 1e-7,
                                                     -1.0, 2e-4, 0.1, None) == EINVAL
    assert L.muon_momentum_ns_update_batched_noalloc(FAKE, FAKE, 0.95, FAKE, 1, 1, 20000, 20000, 0, 5, coeffs,
                                                     1e-7, -1.0, 2e-4, 0.1, None) == ESHAPE
    # a batch whose byte count would wrap is a shape error, not a fit
    assert L.muon_momentum_ns_update_batched_noalloc(FAKE, FAKE, 0.95, FAKE, 1, 1 << 40, 256, 256, 65536, 5,
                                                     coeffs, 1e-7, -1.0, 2e-4, 0.1, None) == ESHAPE


def test_binding_keeps_a_call_on_one_device(mc):
    """The binding rejects a call whose tensors (or whose stream) sit on
    different devices before anything reaches the library: the kernels run on
    the stream's device and would take the other device's addresses as they
    are.  Only each object's device matters to the check."""
    import torch

    class On:
        def __init__(self, device):
            self.device = torch.device(device)

    mc._one_device(None, On("cuda:0"), None, On("cuda:0"))
    mc._one_device(On("cuda:1"), On("cuda:1"), On("cuda:1"))
    with pytest.raises(ValueError):
        mc._one_device(None, On("cuda:0"), On("cuda:1"))
    with pytest.raises(ValueError):
        mc._one_device(None, On("cuda:0"), None, On("cuda:0"), On("cuda:2"))
    with pytest.raises(ValueError):
        mc._one_device(On("cuda:1"), On("cuda:0"), On("cuda:0"))
