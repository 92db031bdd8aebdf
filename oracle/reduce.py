"""Shard-local gradient reduction: the rank's view of a reduce-scatter.

[ZF] "Execution Flow for ZeRO-1", step 2: after backward, each rank receives
the gradient of its own partition averaged over the N_d ranks.
[ZF] "ZeRO-Stage 2": gradients are reduced into their owners' slices as soon
as they are produced, so a rank can receive them bucket by bucket.

Reading taken: the average is an fp32 sum over replicas in replica order
0..R-1 (each bf16 value widened exactly), one fp32 division by R, and one
round-to-nearest-even to bf16 (the stored gradient is 16-bit: [ZF] "Static
Memory Allocation", M_g = 2 Phi; the only code on the page sets the reduce
dtype to bfloat16).
"""
from typing import Sequence

import numpy as np

from .bf16 import bf16_to_f32, f32_to_bf16
from .plan import Plan


def reduce_shard(plan: Plan, rank: int, replicas: Sequence[np.ndarray], begin: int,
                 shard_grad: np.ndarray) -> tuple:
    """Average replicas into shard_grad where the window meets rank's shard.

    replicas[k] holds replica k's bf16 gradient for global flat elements
    [begin, begin + len(replicas[k])). shard_grad (uint16, length S) is updated
    in place on window-and-shard only. Returns (lo, hi), the global range written.
    """
    if len(replicas) < 1:
        raise ValueError("need at least one replica")
    count = len(replicas[0])
    if any(len(r) != count for r in replicas):
        raise ValueError("replicas differ in length")
    s = plan.shard_numel
    lo = max(begin, rank * s)
    hi = min(begin + count, (rank + 1) * s)
    if lo >= hi:
        return lo, lo
    acc = np.zeros(hi - lo, dtype=np.float32)
    for rep in replicas:
        acc = acc + bf16_to_f32(rep[lo - begin:hi - begin])
    avg = acc / np.float32(len(replicas))
    shard_grad[lo - rank * s:hi - rank * s] = f32_to_bf16(avg)
    return lo, hi
