"""Squared L2 norm of a bf16 gradient, computed exactly.

Gradient clipping is not on the pages; the workloads ask for a global-norm
clip, which needs sum(g^2) over every rank's gradient. Each square of a bf16
value is exact in float64 (an 8-bit significand squares into 16 bits), so the
sum has one correct value; every function here returns it correctly rounded.
"""
import math

import numpy as np

from .bf16 import bf16_to_f32


def sqnorm_fsum(bits: np.ndarray) -> float:
    """Brute force: math.fsum of the squares (exact, then one rounding)."""
    x = bf16_to_f32(bits).astype(np.float64)
    return math.fsum((x * x).tolist())


class SqnormAccumulator:
    """Exact running sum of squares of bf16 values, fed in chunks.

    A finite bf16 value with biased exponent e and 7 stored fraction bits f is
    m * 2^(e-134) with m = 128 + f (e > 0), or m * 2^-133 with m = f (e = 0), so
    its square is m^2 * 2^(2e-268) (or m^2 * 2^-266). Per exponent the integer
    parts m^2 are summed exactly (float64 holds integers below 2^53, and
    65025 * n stays below that for n < 1.3e11 values); value() adds the at
    most 255 scaled sums with math.fsum, one rounding in all. Inf and NaN
    inputs make the value inf or nan.
    """

    def __init__(self):
        self.per_exp = np.zeros(256, dtype=np.float64)
        self.count = 0
        self.special = 0.0

    def add(self, bits: np.ndarray) -> "SqnormAccumulator":
        b = np.asarray(bits, dtype=np.uint16).ravel()
        if b.size == 0:
            return self
        e = ((b >> np.uint16(7)) & np.uint16(0xFF)).astype(np.intp)
        frac = (b & np.uint16(0x7F)).astype(np.float64)
        m = np.where(e > 0, frac + 128.0, frac)
        self.per_exp += np.bincount(e, weights=m * m, minlength=256)
        self.count += b.size
        if self.per_exp[255] != 0.0 or (e == 0xFF).any():
            x = bf16_to_f32(b[e == 0xFF]).astype(np.float64)
            self.special += float(np.sum(x * x))   # inf, or nan if a NaN is present
        if self.count >= (1 << 53) // 65025:
            raise OverflowError("too many values for exact per-exponent sums")
        return self

    def merge(self, other: "SqnormAccumulator") -> "SqnormAccumulator":
        """Adds another accumulator's values (exact: integer sums per exponent)."""
        self.per_exp += other.per_exp
        self.count += other.count
        self.special += other.special
        if self.count >= (1 << 53) // 65025:
            raise OverflowError("too many values for exact per-exponent sums")
        return self

    def value(self) -> float:
        if self.special != 0.0:
            return self.special
        terms = []
        for ex in range(255):
            if self.per_exp[ex] != 0.0:
                scale = 2 * (ex - 134) if ex > 0 else -266
                terms.append(math.ldexp(self.per_exp[ex], scale))
        return math.fsum(terms)


def sqnorm(bits: np.ndarray) -> float:
    """Exact sum of squares, correctly rounded to float64 (fed in 1M-value
    chunks only to bound the temporaries; the sum is exact in any order)."""
    b = np.asarray(bits, dtype=np.uint16).ravel()
    acc = SqnormAccumulator()
    for i in range(0, b.size, 1 << 20):
        acc.add(b[i:i + (1 << 20)])
    return acc.value()
