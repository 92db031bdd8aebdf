"""One rank's whole optimizer step, composed from the oracle's parts.

[ZF] "Execution Flow for ZeRO-1" steps 2-4 and "ZeRO-Stage 2": reduce the
rank's slice of the gradient (averaged over the replicas), update the rank's
fp32 state, then gather every rank's bf16 shard into complete tensors. The
global norm needs one scalar from every rank; the other ranks' squared-norm
partials are inputs here (on a real cluster they arrive through a scalar
all-reduce, which the pages do not discuss).
"""
from typing import List, Sequence

import numpy as np

from .adamw import adamw_step
from .clip import clip_scale
from .gather import gather_params, gather_params_shard0
from .plan import Plan, Shard0Plan
from .reduce import reduce_shard
from .sqnorm import sqnorm


def rank_step(plan: Plan, rank: int, replicas: Sequence[np.ndarray], begin: int, state: dict,
              param_shards: List[np.ndarray], partials: Sequence[float], step: int, hp: dict,
              max_norm: float) -> dict:
    """state: dict with 'master', 'exp_avg', 'exp_avg_sq' (float32 [S]), replaced in place.

    param_shards[rank] receives the new bf16 shard (unless the step is skipped);
    partials[rank] is ignored and replaced by this rank's own partial.
    """
    shard_grad = np.zeros(plan.shard_numel, dtype=np.uint16)
    reduce_shard(plan, rank, replicas, begin, shard_grad)
    parts = [float(p) for p in partials]
    parts[rank] = sqnorm(shard_grad)
    clip = clip_scale(parts, max_norm)
    p, m, v, bits = adamw_step(state["master"], state["exp_avg"], state["exp_avg_sq"], shard_grad,
                               step, clip=clip, **hp)
    state["master"], state["exp_avg"], state["exp_avg_sq"] = p, m, v
    if bits is not None:
        param_shards[rank] = bits
    gather = gather_params_shard0 if isinstance(plan, Shard0Plan) else gather_params
    tensors = gather(plan, param_shards)
    return {"shard_grad": shard_grad, "partials": parts, "clip": clip, "tensors": tensors}
