"""Gather of bf16 parameter shards back into per-tensor parameters.

[ZF] "Execution Flow for ZeRO-1", step 4: an all-gather of the updated 16-bit
shards rebuilds the complete parameters on every rank. [ZF] "FSDP-1:
FlatParameter and Module-Level Wrapping": the shards are the N_d equal chunks
of one flat buffer. So the gathered flat buffer is the shards concatenated in
rank order, and tensor t is its slice [offset_t, offset_t + numel_t).
"""
from typing import List, Sequence

import numpy as np

from .plan import Plan


def gather_params(plan: Plan, shards: Sequence[np.ndarray]) -> List[np.ndarray]:
    if len(shards) != plan.n_ranks or any(len(s) != plan.shard_numel for s in shards):
        raise ValueError("need N_d shards of S elements each")
    flat = np.concatenate([np.asarray(s, dtype=np.uint16) for s in shards]) if shards else \
        np.zeros(0, dtype=np.uint16)
    return [flat[off:off + n].copy() for off, n in zip(plan.offsets, plan.numels)]


def gather_params_shard0(plan, shards: Sequence[np.ndarray]) -> List[np.ndarray]:
    """FSDP-2 all-gather output: tensor t is its rank chunks' rows stacked in
    rank order ([ZF] "FSDP-2: Per-Parameter Sharding via DTensor")."""
    if len(shards) != plan.n_ranks or any(len(s) != plan.shard_numel for s in shards):
        raise ValueError("need N_d shards of S elements each")
    out = []
    for t, (off, n) in enumerate(zip(plan.offsets, plan.numels)):
        pieces = []
        for r in range(plan.n_ranks):
            rows = min(plan.chunk_rows[t], plan.dim0[t] - r * plan.chunk_rows[t]) if n else 0
            if rows > 0:
                pieces.append(np.asarray(shards[r][off:off + rows * plan.inner[t]], np.uint16))
        out.append(np.concatenate(pieces) if pieces else np.zeros(0, np.uint16))
    return out
