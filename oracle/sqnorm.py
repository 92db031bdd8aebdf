"""Squared L2 norm of a bf16 gradient, computed exactly.

Gradient clipping is not on the pages; the workloads ask for a global-norm
clip, which needs sum(g^2) over every rank's gradient. Each square of a bf16
value is exact in float64 (an 8-bit significand squares into 16 bits), so the
sum has one correct value; both functions return it correctly rounded.
"""
import math

import numpy as np

from .bf16 import bf16_to_f32


def sqnorm_fsum(bits: np.ndarray) -> float:
    """Brute force: math.fsum of the squares (exact, then one rounding)."""
    x = bf16_to_f32(bits).astype(np.float64)
    return math.fsum((x * x).tolist())


def sqnorm(bits: np.ndarray) -> float:
    """Same value as sqnorm_fsum, for large arrays.

    A finite bf16 value with biased exponent e and 7 stored fraction bits f is
    m * 2^(e-134) with m = 128 + f (e > 0) or m * 2^-133 with m = f (e = 0), so
    its square is m^2 * 2^(2e-268) (or m^2 * 2^-266). Per exponent the integer
    parts m^2 are summed exactly (float64 holds integers below 2^53, and
    65025 * n stays below that for n < 1.3e11), then the at most 255 scaled
    partial sums are added by math.fsum. Inf or NaN inputs give inf or nan.
    """
    b = np.asarray(bits, dtype=np.uint16).ravel()
    if b.size == 0:
        return 0.0
    e = ((b >> np.uint16(7)) & np.uint16(0xFF)).astype(np.int64)
    if (e == 0xFF).any():
        x = bf16_to_f32(b[e == 0xFF]).astype(np.float64)
        return float(np.sum(x * x))       # inf, or nan if any NaN is present
    frac = (b & np.uint16(0x7F)).astype(np.int64)
    m = np.where(e > 0, frac + 128, frac).astype(np.float64)
    per_exp = np.bincount(e, weights=m * m, minlength=256)
    terms = []
    for ex in range(255):
        if per_exp[ex] != 0.0:
            scale = 2 * (ex - 134) if ex > 0 else -266
            terms.append(math.ldexp(per_exp[ex], scale))
    return math.fsum(terms)
