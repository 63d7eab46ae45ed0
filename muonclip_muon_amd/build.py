"""Build libmuonclip.so in-tree with hipcc for gfx950.

    python muonclip_muon_amd/build.py        # or __graft_entry__.build()

(Run as a script, not with -m: importing the package loads the library.)

Each translation unit under csrc/ is compiled to an object in _build/ (in
parallel), then linked into muonclip_muon_amd/libmuonclip.so.  Always
recompiles: the build is the check that every kernel compiles.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmuonclip.so")
ARCH = "gfx950"

SOURCES = ["api.cpp", "elementwise.hip", "qkclip.hip", "ns_prep.hip", "ns_gemm.hip", "maxlogit.hip",
           "maxlogit_generic.hip", "attention.hip", "probe.hip"]

COMMON_FLAGS = [
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Werror",
    "-fvisibility=hidden",
    f"--offload-arch={ARCH}",
    # Packed FP32 instructions (v_pk_add/mul/fma_f32) are kept out of every
    # kernel; the host pass warns that it does not know the feature.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]


# Per-source additions.  maxlogit.hip (the bf16 MFMA kernel only): MFMA
# results in VGPRs (the query fragments then sit in AGPRs, which MFMA reads
# directly), so the running max reads the logits without a v_accvgpr_read per
# value; and no NaN semantics for float operations, so fmaxf becomes a bare
# v_max3_f32 instead of first quieting each operand (the hardware maximum
# still skips quiet NaNs, and the file tests for NaN on the bits).  The
# float32 fallback kernel lives in maxlogit_generic.hip, built with the
# default (IEEE) NaN semantics.
SOURCE_FLAGS = {
    "maxlogit.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-fno-honor-nans"],
    "attention.hip": ["-fno-honor-nans"],
}


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmuonclip.so)")


def _compile(hipcc, src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc, *COMMON_FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in line and line.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    return obj, out


def build(verbose=False):
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), max(1, min(8, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(lambda s: _compile(hipcc, s), SOURCES))
    for (obj, out) in results:
        if out and verbose:
            print(out, file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *[o for o, _ in results], "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
