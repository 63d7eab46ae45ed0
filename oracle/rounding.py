"""Rounding helpers of the oracle (test infrastructure only; see ``oracle/__init__``).

The oracle computes in fp64 and rounds each stored result once to the storage
type the step keeps it in (fp32 or bfloat16), round-to-nearest-even.  NumPy has
no bfloat16, so bfloat16 values are carried in float64/float32 arrays that hold
exactly representable bfloat16 numbers, and as uint16 bit patterns when they
are compared with device output.

bfloat16 is IEEE binary32 with the significand cut to 8 bits (1 implicit + 7
stored): the same exponent range, so every bfloat16 value is exactly a float32.
"""

import numpy as np

__all__ = [
    "round_to_f32",
    "round_to_bf16",
    "bf16_bits",
    "bf16_from_bits",
    "round_to",
]

_BF16_MAX = float(np.ldexp(np.float64(0xFF) / 128.0, 127))  # 1.1111111b x 2^127
_BF16_MIN_NORMAL_EXP = -126
_BF16_SIG_BITS = 8


def round_to_f32(x):
    """fp64 -> nearest float32 (NumPy's cast is IEEE round-to-nearest-even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def round_to_bf16(x):
    """fp64 -> nearest bfloat16, ties to even, returned as float64 values.

    Rounds directly from fp64 (not through float32, which would round twice).
    Values whose rounded magnitude exceeds the largest finite bfloat16 become
    +-inf; NaN stays NaN; subnormals are rounded on the fixed 2^-133 grid.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    finite = np.isfinite(x)
    out[~finite] = x[~finite]
    xf = x[finite]
    mag = np.abs(xf)
    # frexp: |x| = f * 2^k with 0.5 <= f < 1, so the leading bit has weight 2^(k-1)
    # and a normal bfloat16 quantum is 2^(k-1-7).
    _, k = np.frexp(mag)
    lead = np.maximum(k.astype(np.int64) - 1, _BF16_MIN_NORMAL_EXP)  # subnormals: fixed 2^-133 grid
    q = np.ldexp(1.0, lead - (_BF16_SIG_BITS - 1))
    r = np.rint(xf / q) * q  # np.rint rounds half to even; xf/q is exact (power-of-two divide)
    r = np.where(mag == 0, xf, r)  # keep signed zeros
    r = np.where(np.abs(r) > _BF16_MAX, np.copysign(np.inf, xf), r)
    out[finite] = r
    return out


def bf16_bits(x):
    """Bit patterns (uint16) of values that are exactly representable in bfloat16."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32)
    if np.any((u & 0xFFFF) != 0):
        raise ValueError("value is not exactly representable in bfloat16")
    return (u >> 16).astype(np.uint16)


def bf16_from_bits(bits):
    """uint16 bfloat16 bit patterns -> float64 values (exact)."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def round_to(x, dtype):
    """Round fp64 values once to the storage type named by ``dtype``.

    'f32' and 'bf16' round to nearest even; 'f64' keeps the exact fp64 value
    (used by the pins that check the clip identities without storage rounding).
    """
    if dtype == "f32":
        return round_to_f32(x).astype(np.float64)
    if dtype == "bf16":
        return round_to_bf16(x)
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(f"unknown storage dtype {dtype!r}")
