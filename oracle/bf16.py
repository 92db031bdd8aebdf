"""bfloat16 <-> float32 conversions.

[ZF] "Static Memory Allocation": parameters and gradients are held in 16-bit
floating point (BF16 is one of the two named formats), the optimizer state in
32-bit. The rounding mode is not stated; the reading taken is IEEE
round-to-nearest-even on the upper 16 bits of the float32 pattern, with no
flush of subnormals, NaN kept NaN (quiet bit set, sign and top payload bits
kept) and overflow going to infinity.
"""
import numpy as np


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening: the bf16 pattern becomes the top half of a float32."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    is_nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    # Adding 0x7FFF plus the lowest kept bit carries into the kept half exactly
    # when the dropped half is above the midpoint, or at it with an odd kept half.
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    quiet = (u >> np.uint32(16)) | np.uint32(0x0040)
    return np.where(is_nan, quiet, rounded).astype(np.uint16)
