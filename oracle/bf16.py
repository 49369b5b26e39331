"""bfloat16 and float32 rounding, written from the formats' definitions.

TEST INFRASTRUCTURE (see the package docstring).

bfloat16 is IEEE binary32 with the significand cut to 8 bits (7 stored):
1 sign bit, 8 exponent bits (bias 127), subnormals below 2**-126 with spacing
2**-133, largest finite value (2 - 2**-7) * 2**127.  The pages round to it at
fixed points ("bf16(...)" in TensorFold PR #1260's two row kernels) and name no
mode; torch's cast, which the pages' model code uses, rounds to nearest with
ties to even, and so does everything here.
"""
from __future__ import annotations

import numpy as np

BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127
BF16_MIN_SUB = 2.0 ** -133
QNAN_BITS = 0x7FC0


def bf16_rne(v) -> np.ndarray:
    """Round float64 values to the nearest bf16 (ties to even); return bits.

    For finite v with binade exponent e = floor(log2|v|) (clamped below at
    -126, where the subnormal spacing begins), the bf16 spacing is
    q = 2**(e - 7); the result is rint(v / q) * q, where dividing by a power
    of two is exact and numpy's rint rounds half to even.  A result of
    magnitude 2**128 or more has left the format and becomes infinity.  NaN
    maps to the canonical quiet NaN; the sign of zero is kept.
    """
    v = np.asarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    with np.errstate(all="ignore"):
        finite = np.isfinite(v)
        _, k = np.frexp(np.where(finite, v, 1.0))      # v = m * 2**k, 0.5 <= |m| < 1
        e = np.maximum(k.astype(np.int64) - 1, -126)
        q_exp = e - 7
        scaled = np.ldexp(np.where(finite, v, 0.0), (-q_exp).astype(np.int32))
        r = np.ldexp(np.rint(scaled), q_exp.astype(np.int32))
        r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, v), r)
        r = np.where(finite, r, v)
        bits = (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    out[...] = bits
    out[np.isnan(v)] = QNAN_BITS
    return out


def bf16_value(bits) -> np.ndarray:
    """bf16 bit patterns -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def bf16_ulp(value) -> np.ndarray:
    """Spacing of bf16 at the binade of ``value`` (float64); 2**-133 at zero."""
    v = np.abs(np.asarray(value, dtype=np.float64))
    with np.errstate(all="ignore"):
        _, k = np.frexp(np.where(np.isfinite(v) & (v > 0), v, 1.0))
        e = np.maximum(k.astype(np.int64) - 1, -126)
        ulp = np.ldexp(1.0, (e - 7).astype(np.int32))
    return np.where(v > 0, ulp, BF16_MIN_SUB)


def fp32_rne(v) -> np.ndarray:
    """Round float64 values to float32, nearest with ties to even (numpy's cast)."""
    return np.asarray(v, dtype=np.float64).astype(np.float32)
