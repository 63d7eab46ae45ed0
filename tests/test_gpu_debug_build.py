"""The GPU parity tests once more against the debug build of the library
(libmuonclip_debug.so: range checks at the kernels' global accesses, host
code under UndefinedBehaviorSanitizer), in a child process that loads it
through MUONCLIP_LIB.  A kernel access outside its buffer makes the call
return MC_ECHECK (the binding raises), undefined behaviour in host code
aborts the child, and the results must still match the oracle as in the
release build.  The small and ragged cases of the parity, step, attention
and stream tests, the empty and degenerate calls, the largest Newton-Schulz
shapes, the fused call at the full step's shapes (expert batches, W_q,
W_kc, W_kr), strided batches and the seeded random shapes."""

import os
import subprocess
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DEBUG_LIB = os.path.join(ROOT, "muonclip_muon_amd", "libmuonclip_debug.so")


def test_gpu_suite_under_the_debug_build():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(DEBUG_LIB), "libmuonclip_debug.so is not built (python muonclip_muon_amd/build.py)"
    env = dict(os.environ, MUONCLIP_LIB=DEBUG_LIB)
    args = [sys.executable, "-u", "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "gpu",
            "tests/test_gpu_parity.py", "tests/test_gpu_step.py", "tests/test_gpu_attention.py",
            "tests/test_gpu_streams.py", "tests/test_gpu_edges.py", "tests/test_gpu_maxsize.py",
            "tests/test_gpu_fullsize.py", "tests/test_gpu_strided.py", "tests/test_gpu_shape_sweep.py",
            "-k", "not fullsize_8x4096 and (not test_gpu_fullsize or fused_expert_batch)"]
    r = subprocess.run(args, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, tail
    assert "range checks" not in r.stderr and "runtime error" not in r.stderr, tail
    assert " passed" in r.stdout and " failed" not in r.stdout, tail
