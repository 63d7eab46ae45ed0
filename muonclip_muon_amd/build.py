"""Build libmuonclip.so in-tree with hipcc for gfx950.

    python muonclip_muon_amd/build.py          # release and debug libraries, C client
    python muonclip_muon_amd/build.py release  # or debug: one of them

(Run as a script, not with -m: importing the package loads the library.)

Each translation unit under csrc/ is compiled to an object in _build/ (in
parallel), then linked into muonclip_muon_amd/libmuonclip.so.  Always
recompiles: the build is the check that every kernel compiles.

The debug library, libmuonclip_debug.so (objects in _build_debug/), is the
same code compiled with MC_DEBUG: range checks at the kernels' global
accesses, reported by the C ABI after each call (MC_ECHECK), and the host
code under UndefinedBehaviorSanitizer (any undefined behaviour aborts).  The
binding loads it instead of the release library when MUONCLIP_LIB names it.
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
DEBUG_BUILD = os.path.join(PKG, "_build_debug")
DEBUG_LIB = os.path.join(PKG, "libmuonclip_debug.so")
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


# Debug builds: MC_DEBUG range checks in the kernels; host code with debug
# information and UndefinedBehaviorSanitizer, which aborts on the first
# finding (sanitizers apply to host code only: each flag goes to the host
# compilation through -Xarch_host).
DEBUG_FLAGS = ["-DMC_DEBUG", "-Xarch_host", "-g", "-Xarch_host", "-fsanitize=undefined",
               "-Xarch_host", "-fno-sanitize-recover=undefined"]


def _sanitizer_runtime_dir():
    """The directory of clang's shared UBSan runtime (linked by the debug
    library, found at load time through its rpath)."""
    import glob
    base = os.path.join(os.path.dirname(os.path.realpath(_hipcc())), "..", "lib", "llvm", "lib", "clang")
    for cand in (base, "/opt/rocm/llvm/lib/clang"):
        hits = glob.glob(os.path.join(cand, "*", "lib", "*", "libclang_rt.ubsan_standalone*.so"))
        hits = [h for h in hits if "i386" not in h]
        if hits:
            return os.path.dirname(os.path.realpath(hits[0]))
    raise RuntimeError("clang's shared UBSan runtime was not found (debug build)")


def _compile(hipcc, src, debug=False):
    obj = os.path.join(DEBUG_BUILD if debug else BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc, *COMMON_FLAGS, *(DEBUG_FLAGS if debug else []), *SOURCE_FLAGS.get(src, []), "-c",
           os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in line and line.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    return obj, out


def build(verbose=False, debug=False):
    """Compile and link the release library (debug=False) or the debug one."""
    hipcc = _hipcc()
    os.makedirs(DEBUG_BUILD if debug else BUILD, exist_ok=True)
    jobs = min(len(SOURCES), max(1, min(8, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(lambda s: _compile(hipcc, s, debug), SOURCES))
    for (obj, out) in results:
        if out and verbose:
            print(out, file=sys.stderr)
    lib = DEBUG_LIB if debug else LIB
    tmp = lib + ".tmp"
    cmd = [hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *[o for o, _ in results], "-o", tmp]
    if debug:
        cmd[-2:-2] = ["-Xarch_host", "-fsanitize=undefined", "-shared-libsan",
                      f"-Wl,-rpath,{_sanitizer_runtime_dir()}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, lib)
    return lib


C_CLIENT_SRC = os.path.join(ROOT, "tests", "c_client", "step_client.c")
C_CLIENT = os.path.join(ROOT, "tests", "c_client", "step_client")


def build_c_client():
    """The plain C client of the C ABI (tests/c_client/step_client.c; host
    code only, gcc), linked against the release library in this package."""
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(_hipcc())))
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(rocm, "include"), "-D__HIP_PLATFORM_AMD__", C_CLIENT_SRC, "-L", PKG, "-lmuonclip",
           "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-Wl,-rpath,$ORIGIN/../../muonclip_muon_amd",
           f"-Wl,-rpath,{os.path.join(rocm, 'lib')}", "-o", C_CLIENT]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"C client build failed:\n{r.stdout}{r.stderr}")
    return C_CLIENT


def build_all(verbose=False):
    libs = [build(verbose), build(verbose, debug=True)]
    return libs + [build_c_client()]


if __name__ == "__main__":
    which = sys.argv[1] if len(sys.argv) > 1 else "all"
    if which == "release":
        print(build(verbose=True))
    elif which == "debug":
        print(build(verbose=True, debug=True))
    else:
        print("\n".join(build_all(verbose=True)))
