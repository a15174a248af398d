"""Exact bf16 <-> float64 conversions for the oracle (test infrastructure only).

bf16 is the upper half of an IEEE binary32: 1 sign bit, 8 exponent bits, 7
stored mantissa bits.  Values travel through the oracle as their uint16 bit
patterns so that nothing depends on a bf16 dtype in numpy.

Both functions are pinned in ``tests/test_oracle.py`` (exhaustive round trip of
all 65,536 patterns; rounding checked against torch's CPU cast).
"""

import numpy as np


def bf16_bits_to_f64(bits):
    """uint16 bf16 bit patterns -> float64, exactly (every bf16 is a double)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits_rne(x):
    """float64 -> bf16 bit patterns, one rounding, round-to-nearest-even.

    Rounds directly from the double (no intermediate float32 step, so there is
    no double rounding).  bf16 keeps 8 significant bits; its spacing at
    x = m * 2**e (0.5 <= |m| < 1) is 2**(e-8), never finer than the subnormal
    spacing 2**-133.  Magnitudes that round past the largest finite bf16
    become infinity; NaN stays a quiet NaN.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    finite = np.isfinite(x)
    _, e = np.frexp(np.where(finite, x, 1.0))
    ulp = np.exp2(np.maximum(e - 8, -133).astype(np.float64))
    r = np.rint(np.where(finite, x, 0.0) / ulp) * ulp
    max_bf16 = float(np.array([0x7F7F0000], dtype=np.uint32).view(np.float32)[0])
    r = np.where(np.abs(r) > max_bf16, np.copysign(np.inf, r), r)
    r = np.where(finite, r, x)
    f32 = r.astype(np.float32)  # exact: r has at most 8 significant bits
    bits = (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    bits[nan] = np.uint16(0x7FC0)
    out[...] = bits
    return out
