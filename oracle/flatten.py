"""Flatten of per-tensor buffers into the padded flat buffer.

[ZF] "FSDP-1: FlatParameter and Module-Level Wrapping": a unit's tensors are
flattened into one contiguous 1-D tensor, padded to a length divisible by the
world size. Tensor t occupies [offset_t, offset_t + numel_t); the padding
[Phi, P) holds zeros.
"""
from typing import Sequence

import numpy as np

from .plan import Plan


def flatten_params(plan: Plan, tensors: Sequence[np.ndarray]) -> np.ndarray:
    if len(tensors) != len(plan.numels) or any(len(t) != n for t, n in zip(tensors, plan.numels)):
        raise ValueError("need one buffer of numel_t values per tensor")
    flat = np.zeros(plan.padded_numel, dtype=np.uint16)
    for t, off, n in zip(tensors, plan.offsets, plan.numels):
        flat[off:off + n] = np.asarray(t, dtype=np.uint16)
    return flat
