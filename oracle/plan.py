"""Flat-buffer partition plan and static-memory accounting.

[ZF] "FSDP-1: FlatParameter and Module-Level Wrapping": the tensors of a unit
are flattened into one contiguous 1-D buffer, padded until its length divides
by the world size N_d, and cut into N_d equal chunks.
[ZF] "ZeRO-Stage 1: Optimizer State Partitioning": rank i owns a Phi/N_d slice.

Reading taken: tensors are concatenated in the given order with no gaps;
padding goes at the end only; the padded length is also a multiple of N_d*A so
that every shard holds a whole number of A-element alignment units (A = 128 in
the tiny workload, used throughout). Rank r owns flat elements [r*S, (r+1)*S).
"""
from dataclasses import dataclass
from typing import List, Tuple

Segment = Tuple[int, int, int, int]   # (tensor, offset in tensor, offset in shard, length)


@dataclass
class Plan:
    numels: List[int]
    n_ranks: int
    align: int
    offsets: List[int]
    numel: int          # Phi
    padded_numel: int   # P
    shard_numel: int    # S

    def segments(self, rank: int) -> List[Segment]:
        """Pieces of tensors that fall into rank's shard, in flat order."""
        if not 0 <= rank < self.n_ranks:
            raise ValueError("rank out of range")
        lo_r = rank * self.shard_numel
        hi_r = lo_r + self.shard_numel
        out = []
        for t, (off, n) in enumerate(zip(self.offsets, self.numels)):
            lo = max(off, lo_r)
            hi = min(off + n, hi_r)
            if lo < hi:
                out.append((t, lo - off, lo - lo_r, hi - lo))
        return out


def partition_plan(numels, n_ranks: int, align: int = 128) -> Plan:
    numels = [int(n) for n in numels]
    if n_ranks < 1 or align < 1 or any(n < 0 for n in numels):
        raise ValueError("invalid plan arguments")
    offsets = []
    total = 0
    for n in numels:
        offsets.append(total)
        total += n
    unit = n_ranks * align
    padded = -(-total // unit) * unit
    return Plan(numels, n_ranks, align, offsets, total, padded, padded // n_ranks)


def memory_bytes(plan: Plan, stage: int, padded: bool = False) -> float:
    """Static bytes per GPU for DDP (stage 0) and ZeRO stages 1-3.

    [ZF] "Static Memory Allocation": 2 (params) + 2 (grads) + 12 (fp32 master,
    m, v) bytes per parameter, 16 Phi in all. Stage formulas: [ZF] "ZeRO-Stage 1"
    (4 Phi + 12 Phi/N_d), "ZeRO-Stage 2" (2 Phi + 14 Phi/N_d), "ZeRO-Stage 3 and
    Fully Sharded Data Parallelism" (16 Phi/N_d). With padded=True the flat
    buffers are counted at their padded length P and shard length S instead.
    """
    phi, nd = plan.numel, plan.n_ranks
    if not padded:
        table = {0: 16 * phi, 1: 4 * phi + 12 * phi / nd, 2: 2 * phi + 14 * phi / nd,
                 3: 16 * phi / nd}
    else:
        p, s = plan.padded_numel, plan.shard_numel
        table = {0: 16 * phi, 1: 4 * p + 12 * s, 2: 2 * p + 14 * s, 3: 16 * s}
    if stage not in table:
        raise ValueError("stage must be 0, 1, 2 or 3")
    return float(table[stage])


@dataclass
class Shard0Plan(Plan):
    """FSDP-2 per-parameter layout.

    [ZF] "FSDP-2: Per-Parameter Sharding via DTensor (fully_shard)": each tensor
    is sharded on its own along its leading dimension (a Shard(0) placement),
    not flattened with the others; one rank's shards travel in a coalesced
    buffer. Reading taken: torch.chunk's cut, ceil(dim0 / N_d) rows per chunk,
    rank r holding rows [r*c, min((r+1)*c, dim0)) (possibly none); in a rank's
    buffer the chunks follow tensor order, each padded to c*inner elements, the
    buffer padded to a multiple of A. `offsets` are the chunk starts inside a
    rank's buffer; the flat buffer is the N_d rank buffers side by side.
    """
    dim0: List[int] = None
    chunk_rows: List[int] = None
    inner: List[int] = None

    def segments(self, rank: int) -> List[Segment]:
        if not 0 <= rank < self.n_ranks:
            raise ValueError("rank out of range")
        out = []
        for t, (off, n) in enumerate(zip(self.offsets, self.numels)):
            if n == 0:
                continue
            first = rank * self.chunk_rows[t]
            rows = min(self.chunk_rows[t], self.dim0[t] - first)
            if rows > 0:
                out.append((t, first * self.inner[t], off, rows * self.inner[t]))
        return out


def partition_plan_shard0(numels, dim0, n_ranks: int, align: int = 128) -> Shard0Plan:
    numels = [int(n) for n in numels]
    dim0 = [int(d) for d in dim0]
    if n_ranks < 1 or align < 1 or len(numels) != len(dim0):
        raise ValueError("invalid plan arguments")
    offsets, rows_l, inner_l, buf = [], [], [], 0
    for n, d in zip(numels, dim0):
        if n < 0 or (n > 0 and (d < 1 or n % d)):
            raise ValueError("dim0 must be >= 1 and divide numel")
        inner = n // d if n else 0
        rows = -(-d // n_ranks) if n else 0
        offsets.append(buf)
        rows_l.append(rows)
        inner_l.append(inner)
        buf += rows * inner
    s = -(-buf // align) * align
    return Shard0Plan(numels, n_ranks, align, offsets, sum(numels), s * n_ranks, s,
                      dim0=dim0, chunk_rows=rows_l, inner=inner_l)
