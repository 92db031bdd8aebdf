"""CPU oracle for the partitioned mixed-precision optimizer step.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package. The product library never calls it
and it imports nothing from the product library: the two share no code.

The oracle is plain and slow on purpose: numpy array operations in the order
the method states them, float32 where the pages fix 32-bit state, float64 or
exact arithmetic elsewhere. Each function cites the passage it follows. The
cited page throughout is "Zero Redundancy Optimizer (ZeRO) and Fully Sharded
Data Parallelism (FSDP): Mathematical Foundations of Memory Partitioning,
Communication Complexity, and Overlapped Execution" (llms.blog), written [ZF]
below, with the section name after it.

Pinning status (what each function is checked against, outside itself):
  plan.py     page memory figures, closed forms, brute force on tiny lists
  bf16.py     torch's CPU float32->bfloat16 conversion, exhaustive edge sets
  reduce.py   R=1 identity, identical replicas, pure-Python brute force
  sqnorm.py   math.fsum brute force, n*c^2 closed form
  clip.py     closed form, clip-inactive equivalence
  adamw.py    step-1 closed form, constant-gradient closed form, lr=0,
              torch.optim.AdamW (CPU fp32), pure-Python brute force,
              shard invariance
  gather.py   flatten/gather round trip
  flatten.py  gather(flatten(x)) = x, padding zero, hand-worked case
  Shard(0)    torch.chunk's row cut, round trips, hand-worked case
The fp32 evaluation order inside AdamW and the clip's 1e-6 guard are readings
(the pages do not write the update out); they are pinned by the closed forms
and the torch cross-check within tolerance, not bit for bit by the pages.
"""
from .adamw import AdamWConstants, adamw_constants, adamw_step  # noqa: F401
from .bf16 import bf16_to_f32, f32_to_bf16  # noqa: F401
from .clip import clip_scale  # noqa: F401
from .flatten import flatten_params, flatten_params_shard0  # noqa: F401
from .gather import gather_params, gather_params_shard0  # noqa: F401
from .plan import Plan, Shard0Plan, memory_bytes, partition_plan, partition_plan_shard0  # noqa: F401
from .reduce import reduce_shard  # noqa: F401
from .sqnorm import SqnormAccumulator, sqnorm, sqnorm_fsum  # noqa: F401
from .step import rank_step  # noqa: F401
