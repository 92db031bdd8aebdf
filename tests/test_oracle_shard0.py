"""Pins for the FSDP-2 per-parameter Shard(0) layout (CPU only)."""
import numpy as np
import pytest
import torch

import oracle
import synth


def _shapes(name):
    return synth.WORKLOADS[name].shapes


def test_shard0_hand_worked():
    # [10, 3] and [2] over 4 ranks, no alignment: chunks of 3 and 1 rows
    plan = oracle.partition_plan_shard0([30, 2], [10, 2], 4, 1)
    assert (plan.chunk_rows, plan.inner, plan.offsets) == ([3, 1], [3, 1], [0, 9])
    assert (plan.shard_numel, plan.padded_numel, plan.numel) == (10, 40, 32)
    assert plan.segments(0) == [(0, 0, 0, 9), (1, 0, 9, 1)]
    assert plan.segments(1) == [(0, 9, 0, 9), (1, 1, 9, 1)]
    assert plan.segments(2) == [(0, 18, 0, 9)]
    assert plan.segments(3) == [(0, 27, 0, 3)]


@pytest.mark.parametrize("seed", range(25))
def test_shard0_matches_torch_chunk(seed):
    rng = np.random.default_rng(500 + seed)
    t = int(rng.integers(1, 7))
    dim0 = [int(x) for x in rng.integers(1, 40, t)]
    inner = [int(x) for x in rng.integers(1, 9, t)]
    n_ranks = int(rng.choice([1, 2, 3, 4, 8, 16]))
    plan = oracle.partition_plan_shard0([d * k for d, k in zip(dim0, inner)], dim0, n_ranks,
                                        int(rng.choice([1, 8, 128])))
    for ti, (d, k) in enumerate(zip(dim0, inner)):
        idx = torch.arange(d * k).view(d, k)
        chunks = torch.chunk(idx, n_ranks, dim=0)
        for r in range(n_ranks):
            mine = [s for s in plan.segments(r) if s[0] == ti]
            if r < len(chunks) and chunks[r].numel():
                assert len(mine) == 1
                _, toff, soff, ln = mine[0]
                assert (toff, ln) == (int(chunks[r].flatten()[0]), chunks[r].numel())
                assert soff == plan.offsets[ti]
            else:
                assert mine == []
    assert plan.shard_numel % plan.align == 0
    assert plan.padded_numel == plan.n_ranks * plan.shard_numel


@pytest.mark.parametrize("seed", range(10))
def test_shard0_round_trip_and_coverage(seed):
    rng = np.random.default_rng(600 + seed)
    t = int(rng.integers(1, 6))
    dim0 = [int(x) for x in rng.integers(1, 30, t)]
    inner = [int(x) for x in rng.integers(1, 7, t)]
    numels = [d * k for d, k in zip(dim0, inner)]
    if seed % 3 == 0:
        numels[0], dim0[0] = 0, 0
    plan = oracle.partition_plan_shard0(numels, dim0, int(rng.choice([2, 3, 5, 8])), 4)
    tensors = [rng.integers(1, 1 << 16, n).astype(np.uint16) for n in numels]
    flat = oracle.flatten_params_shard0(plan, tensors)
    S = plan.shard_numel
    shards = [flat[r * S:(r + 1) * S] for r in range(plan.n_ranks)]
    for a, b in zip(oracle.gather_params_shard0(plan, shards), tensors):
        assert (a == b).all()
    # every tensor element appears exactly once; every other flat position is zero
    covered = np.zeros(plan.padded_numel, bool)
    seen = [np.zeros(n, int) for n in numels]
    for r in range(plan.n_ranks):
        for (ti, toff, soff, ln) in plan.segments(r):
            assert not covered[r * S + soff:r * S + soff + ln].any()
            covered[r * S + soff:r * S + soff + ln] = True
            seen[ti][toff:toff + ln] += 1
    assert all((x == 1).all() for x in seen)
    assert (flat[~covered] == 0).all()


def test_shard0_memory_per_rank():
    # FSDP-2's per-rank state is the padded coalesced buffer: 16 bytes per element
    shapes = _shapes("gpt2-small")
    numels = [int(np.prod(s)) for s in shapes]
    n_ranks, align = 8, 128
    plan = oracle.partition_plan_shard0(numels, [s[0] for s in shapes], n_ranks, align)
    assert oracle.memory_bytes(plan, 3, padded=True) == 16 * plan.shard_numel
    # padding: each tensor's rows rounded up to a multiple of N_d, then the buffer to A
    chunk_pad = sum(((d + n_ranks - 1) // n_ranks * n_ranks - d) * (n // d)
                    for n, d in zip(numels, [s[0] for s in shapes]))
    assert 0 <= plan.padded_numel - plan.numel - chunk_pad < n_ranks * align
