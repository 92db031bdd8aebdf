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


def flatten_params_shard0(plan, tensors: Sequence[np.ndarray]) -> np.ndarray:
    """FSDP-2 coalesced layout: rank r's buffer holds, in tensor order, rows
    [r*c_t, (r+1)*c_t) of every tensor t, each chunk padded with zeros to c_t
    rows; the N_d rank buffers side by side."""
    if len(tensors) != len(plan.numels) or any(len(t) != n for t, n in zip(tensors, plan.numels)):
        raise ValueError("need one buffer of numel_t values per tensor")
    flat = np.zeros(plan.padded_numel, dtype=np.uint16)
    for r in range(plan.n_ranks):
        base = r * plan.shard_numel
        for t, (off, n) in enumerate(zip(plan.offsets, plan.numels)):
            if n == 0:
                continue
            first = r * plan.chunk_rows[t]
            rows = min(plan.chunk_rows[t], plan.dim0[t] - first)
            if rows > 0:
                k = plan.inner[t]
                flat[base + off:base + off + rows * k] = tensors[t][first * k:(first + rows) * k]
    return flat
