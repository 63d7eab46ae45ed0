"""Helpers shared by the GPU parity tests (comparisons and dtype plumbing)."""

import sys

import numpy as np
import torch


def say(*args):
    """Print and flush what the next GPU step is, so a failed run names its case."""
    print("[gpu]", *args, flush=True)
    sys.stdout.flush()


def f64(t):
    """Device or host tensor -> float64 numpy (exact for bf16 and float32)."""
    return t.detach().to("cpu", torch.float64).numpy()


def bf16_bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def ordered(bits16):
    """bf16 bit patterns -> integers whose difference counts ulps across zero."""
    b = bits16.astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def bf16_ulp_diff(a_bits, b_bits):
    return np.abs(ordered(a_bits) - ordered(b_bits))


def f32_ulp_diff(a, b):
    a = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    b = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    a = np.where(a < 0, -(a & 0x7FFFFFFF), a)
    b = np.where(b < 0, -(b & 0x7FFFFFFF), b)
    return np.abs(a - b)


def rel_fro(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return np.abs(got - ref) / np.maximum(np.abs(ref), 1e-30)
