"""Pins for the oracle's partition plan and memory accounting (CPU only)."""
import json
import os

import numpy as np
import pytest

import oracle
from synth.models import WORKLOADS


def test_page_memory_figures(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "page_memory_figures.json")))
    one = oracle.partition_plan([1], 1, 1)
    assert oracle.memory_bytes(one, 0) == g["bytes_per_param_static"]["value"]
    f = g["ddp_70b_gb"]
    assert oracle.memory_bytes(oracle.partition_plan([f["phi"]], 1, 1), 0) / 1e9 == f["value"]
    f = g["ddp_5b_gb"]
    assert oracle.memory_bytes(oracle.partition_plan([f["phi"]], 1, 1), 0) / 1e9 == f["value"]
    f = g["zero_70b_nd64_gb"]
    plan = oracle.partition_plan([f["phi"]], f["n_d"], 1)
    for stage, printed in f["printed"].items():
        got = oracle.memory_bytes(plan, int(stage)) / 1e9
        assert round(got, f["printed_decimals"][stage]) == printed, (stage, got)
    # exact values of the printed expressions 280 + 840/64, 140 + 980/64, 1120/64
    assert oracle.memory_bytes(plan, 1) / 1e9 == 280 + 840 / 64
    assert oracle.memory_bytes(plan, 2) / 1e9 == 140 + 980 / 64
    assert oracle.memory_bytes(plan, 3) / 1e9 == 1120 / 64


def test_memory_limits_as_nd_grows(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "page_memory_figures.json")))["limits_as_nd_grows"]
    phi = 10 ** 9
    plan = oracle.partition_plan([phi], 2 ** 40, 1)
    assert oracle.memory_bytes(plan, 1) / phi == pytest.approx(g["stage1_bytes_per_param"], abs=1e-9)
    assert oracle.memory_bytes(plan, 2) / phi == pytest.approx(g["stage2_bytes_per_param"], abs=1e-9)
    assert oracle.memory_bytes(plan, 3) / phi == pytest.approx(g["stage3_bytes_per_param"], abs=1e-9)
    # the stage table at N_d = 1 collapses to DDP's 16 Phi
    plan1 = oracle.partition_plan([phi], 1, 1)
    for s in range(4):
        assert oracle.memory_bytes(plan1, s) == 16 * phi


def test_tiny_a_segments_worked_by_hand(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "tiny_a_segments.json")))
    plan = oracle.partition_plan(WORKLOADS["tiny-a"].numels, 4, 128)
    assert (plan.numel, plan.padded_numel, plan.shard_numel) == (
        g["numel"], g["padded_numel"], g["shard_numel"])
    assert plan.offsets == g["offsets"]
    for r in range(4):
        assert [list(s) for s in plan.segments(r)] == g["segments"][str(r)]


def _brute_force_owner(numels, n_ranks, align):
    """Element-by-element: flat index -> (tensor, index in tensor) and (rank, index in shard)."""
    flat = [(t, j) for t, n in enumerate(numels) for j in range(n)]
    phi = len(flat)
    p = phi
    while p % (n_ranks * align):
        p += 1
    s = p // n_ranks
    owner = [(g // s, g % s) for g in range(phi)]
    return flat, phi, p, s, owner


@pytest.mark.parametrize("seed", range(40))
def test_plan_brute_force_tiny(seed):
    rng = np.random.default_rng(seed)
    t = int(rng.integers(1, 9))
    numels = [int(x) for x in rng.integers(0, 300, size=t)]
    n_ranks = int(rng.choice([1, 2, 3, 4, 8]))
    align = int(rng.choice([1, 8, 128]))
    plan = oracle.partition_plan(numels, n_ranks, align)
    flat, phi, p, s, owner = _brute_force_owner(numels, n_ranks, align)
    assert (plan.numel, plan.padded_numel, plan.shard_numel) == (phi, p, s)
    assert p % n_ranks == 0 and s % align == 0 and p - phi < n_ranks * align
    # every element of every tensor is covered exactly once, at the right shard slot
    seen = {}
    for r in range(n_ranks):
        for (ti, toff, soff, ln) in plan.segments(r):
            assert ln > 0
            for k in range(ln):
                key = (ti, toff + k)
                assert key not in seen
                seen[key] = (r, soff + k)
    assert len(seen) == phi
    for g_idx, key in enumerate(flat):
        assert seen[key] == owner[g_idx]


# Phi, P, S and the tensor count of each workload's tensor list, from
# summing the listed shapes by hand (model definition order).
EXPECTED = {
    "tiny-a": (999_515, 999_936, 249_984, 4),
    "tiny-b": (1_000_003, 1_000_448, 250_112, 4),
    "gpt2-small": (124_439_808, 124_440_576, 15_555_072, 148),
    "llama3-8b": (8_030_261_248, 8_030_265_344, 125_472_896, 291),
    "llama3-70b": (70_553_706_496, 70_553_706_496, 8_819_213_312, 723),
    "gpt-1.3b": (1_315_723_264, 1_315_723_264, 164_465_408, 292),
}


@pytest.mark.parametrize("name", sorted(EXPECTED))
def test_workload_plans(name):
    w = WORKLOADS[name]
    plan = oracle.partition_plan(w.numels, w.n_ranks, w.align)
    assert (plan.numel, plan.padded_numel, plan.shard_numel, len(plan.numels)) == EXPECTED[name]
    total = 0
    for r in range(w.n_ranks):
        segs = plan.segments(r)
        # segments of one rank are contiguous in the shard, in flat order
        pos = 0
        for (_, _, soff, ln) in segs:
            assert soff == pos
            pos += ln
        total += pos
        assert pos == min(plan.shard_numel, max(0, plan.numel - r * plan.shard_numel))
    assert total == plan.numel


def test_plan_rejects_bad_arguments():
    with pytest.raises(ValueError):
        oracle.partition_plan([1, -1], 2, 1)
    with pytest.raises(ValueError):
        oracle.partition_plan([1], 0, 1)
    with pytest.raises(ValueError):
        oracle.partition_plan([1], 1, 0)
    empty = oracle.partition_plan([], 4, 128)
    assert (empty.numel, empty.padded_numel, empty.shard_numel) == (0, 0, 0)
    assert empty.segments(3) == []
