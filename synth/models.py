"""Workload descriptions: model-shaped tensor lists and their training settings.

Only shapes, sizes and hyperparameters live here; nothing in this file computes
any part of the optimizer step. The tensor lists follow each model family's
definition order, row-major, as a flat parameter buffer would concatenate them
(the FlatParameter of "Zero Redundancy Optimizer (ZeRO) and Fully Sharded Data
Parallelism (FSDP): Mathematical Foundations ...", section "FSDP-1: FlatParameter
and Module-Level Wrapping", flattens a unit's tensors into one 1-D buffer; only
each tensor's element count matters for the layout).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from math import prod
from typing import List, Tuple

Shape = Tuple[int, ...]

# Input-stream kinds of the counter-based generator.
KIND_MASTER = 0    # fp32 master weights, N(0, 0.02)
KIND_GRAD = 1      # an already-averaged bf16 gradient, N(0, 1e-3)
KIND_REPLICA = 2   # one data-parallel replica's bf16 gradient, N(0, 1e-3)
KIND_PARAM = 3     # bf16 parameter shards held by other ranks (gather inputs)

MASTER_SIGMA = 0.02
GRAD_SIGMA = 1e-3


def tiny_mlp(last: int) -> List[Shape]:
    """The 'tiny' flat model: [1000,512], [512], [487,1000] and one ragged tail tensor."""
    return [(1000, 512), (512,), (487, 1000), (last,)]


def gpt2(d: int, n_layer: int, vocab: int, n_ctx: int, mlp: int) -> List[Shape]:
    shapes: List[Shape] = [(vocab, d), (n_ctx, d)]
    for _ in range(n_layer):
        shapes += [
            (d,), (d,),                 # ln_1 weight, bias
            (d, 3 * d), (3 * d,),       # fused QKV projection
            (d, d), (d,),               # attention output projection
            (d,), (d,),                 # ln_2 weight, bias
            (d, mlp), (mlp,),           # MLP up
            (mlp, d), (d,),             # MLP down
        ]
    shapes += [(d,), (d,)]              # final layer norm; the LM head is tied to the embedding
    return shapes


def llama3(d: int, n_layer: int, vocab: int, kv_dim: int, ffn: int) -> List[Shape]:
    shapes: List[Shape] = [(vocab, d)]
    for _ in range(n_layer):
        shapes += [
            (d,),                        # attention RMSNorm
            (d, d), (kv_dim, d), (kv_dim, d), (d, d),   # W_q, W_k, W_v, W_o
            (d,),                        # FFN RMSNorm
            (ffn, d), (ffn, d), (d, ffn),               # W_gate, W_up, W_down
        ]
    shapes += [(d,), (vocab, d)]         # final norm, untied LM head
    return shapes


def numels(shapes: List[Shape]) -> List[int]:
    return [int(prod(s)) for s in shapes]


@dataclass(frozen=True)
class Workload:
    name: str
    description: str
    shapes: List[Shape]
    n_ranks: int
    align: int = 128
    steps: int = 1
    max_norm: float = 0.0            # <= 0 means no clipping
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01
    seed: int = 0
    ranks: Tuple[int, ...] = ()      # ranks whose shard is stepped
    replicas: int = 0                # gradient replicas reduced per shard (0: grads arrive averaged)
    bucket: int = 0                  # flat-index bucket size of the reduce (0: whole buffer)
    extra: dict = field(default_factory=dict)

    @property
    def numels(self) -> List[int]:
        return numels(self.shapes)


WORKLOADS = {
    # 1 M-parameter flat model, 4 ranks, all shards stepped in turn, 10 steps.
    # The stated total (1,000,003) and the stated shapes (999,515 with a 3-element
    # tail) disagree; both readings are kept.
    "tiny-a": Workload("tiny-a", "tiny flat model, tail [3], N_d=4, 10 steps",
                       tiny_mlp(3), n_ranks=4, steps=10, seed=1, ranks=(0, 1, 2, 3)),
    "tiny-b": Workload("tiny-b", "tiny flat model, tail [491] (Phi=1,000,003), N_d=4, 10 steps",
                       tiny_mlp(491), n_ranks=4, steps=10, seed=1, ranks=(0, 1, 2, 3)),
    "gpt2-small": Workload("gpt2-small",
                           "GPT-2-small tensor list (124.4M), N_d=8, rank 7's shard, clip 1.0, 100 steps",
                           gpt2(768, 12, 50257, 1024, 3072), n_ranks=8, steps=100, max_norm=1.0,
                           seed=2, ranks=(7,)),
    "llama3-8b": Workload("llama3-8b",
                          "Llama-3-8B tensor list (8.03B), N_d=64, rank 63's shard, 25M-element "
                          "bucketed reduce of 64 replicas, clip 1.0, 1 step",
                          llama3(4096, 32, 128256, 1024, 14336), n_ranks=64, steps=1, max_norm=1.0,
                          seed=3, ranks=(63,), replicas=64, bucket=25_000_000),
    "llama3-70b": Workload("llama3-70b",
                           "Llama-3-70B tensor list (70.6B), N_d=8, rank 7's 8.8B-element shard, "
                           "clip 1.0, 5 steps",
                           llama3(8192, 80, 128256, 1024, 28672), n_ranks=8, steps=5, max_norm=1.0,
                           seed=4, ranks=(7,)),
    "gpt-1.3b": Workload("gpt-1.3b",
                         "1.3B GPT tensor list (d=2048, 24 layers, MLP 8192, n_ctx 2048), N_d=8, "
                         "8 replicas reduced for all 8 ranks, AdamW on every shard, gather, 1 step",
                         gpt2(2048, 24, 50257, 2048, 8192), n_ranks=8, steps=1, seed=5,
                         ranks=tuple(range(8)), replicas=8),
}
