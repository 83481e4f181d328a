"""bfloat16 conversions (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

bfloat16 is the top 16 bits of an IEEE binary32: 1 sign bit, 8 exponent bits,
7 stored mantissa bits.  Stored here as ``numpy.uint16`` bit patterns.

* widening (bf16 -> float64) is exact: put the 16 bits in the high half of a
  binary32 and widen that.
* narrowing (float64 -> bf16) rounds to nearest, ties to even, directly from
  the float64 value (no intermediate binary32 rounding).  Finite values in the
  normal binary32 range only; the verify step never produces others.

Pinned by: agreement with torch's float32 -> bfloat16 cast on float32 inputs
(including exact halfway cases), and exact round trips
(tests/test_oracle_basics.py).
"""
import numpy as np


def bf16_to_f64(bits):
    """uint16 bf16 bit patterns -> float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16(x):
    """float64 -> uint16 bf16 bits, round to nearest even.

    A binary64 has 52 stored mantissa bits; bf16 keeps 7, so the 45 low bits
    are dropped with round-to-nearest-even on the float64 bit pattern.  The
    exponent range is unchanged for binary32-range values, so the rounded
    float64 is exactly a binary32 whose high 16 bits are the answer.
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("f64_to_bf16: non-finite input")
    u = x.view(np.uint64)
    drop = np.uint64(45)
    lsb = (u >> drop) & np.uint64(1)
    u = (u + (np.uint64((1 << 44) - 1) + lsb)) & ~np.uint64((1 << 45) - 1)
    r = u.view(np.float64).astype(np.float32)  # exact: 8 significant bits
    return (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def round_bf16(x):
    """float64 -> nearest bf16 value, returned as float64."""
    return bf16_to_f64(f64_to_bf16(x))
