"""The debug build of the library (libmuonclip_debug.so: the same sources with
MC_DEBUG range checks at the kernels' global accesses, host code under
UndefinedBehaviorSanitizer), on the host: it says it is a debug build, the
release library says it is not, and the whole host ABI suite (exports,
argument validation, the C client) passes against it in a child process,
where the sanitizer aborts on any undefined behaviour of the validation
code."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DEBUG_LIB = os.path.join(ROOT, "muonclip_muon_amd", "libmuonclip_debug.so")


def _child(args, timeout=600):
    env = dict(os.environ, MUONCLIP_LIB=DEBUG_LIB)
    return subprocess.run([sys.executable, *args], cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=timeout)


@pytest.fixture(scope="module")
def debug_lib():
    if not os.path.exists(DEBUG_LIB):
        pytest.skip("libmuonclip_debug.so is not built (python muonclip_muon_amd/build.py)")
    return DEBUG_LIB


def test_release_library_is_not_a_debug_build():
    if os.environ.get("MUONCLIP_LIB"):
        pytest.skip("another library is selected")
    import muonclip_muon_amd as mc
    assert mc.lib.mc_debug_build() == 0


def test_debug_library_says_so(debug_lib):
    r = _child(["-c", "import muonclip_muon_amd as mc; print(mc.LIB_PATH, mc.lib.mc_debug_build())"])
    assert r.returncode == 0, r.stderr[-2000:]
    path, flag = r.stdout.split()
    assert os.path.samefile(path, debug_lib) and flag == "1"


def test_host_abi_suite_under_the_debug_build(debug_lib):
    r = _child(["-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "tests/test_abi_host.py"])
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "runtime error" not in r.stderr  # UBSan reports
