"""Host logic of step.py on the CPU: bucket windows and the staggered arena."""
import numpy as np
import pytest
import torch

import oracle
import synth


@pytest.fixture(scope="module")
def step():
    from zero_partitioned_mixed_partition_amd import step as s
    return s


def test_llama3_8b_rank63_bucket_windows(step):
    """Llama-3-8B at N_d = 64 with 25,000,000-element buckets: the last rank's
    shard meets buckets 316..321, in backward (descending) order; their parts
    inside the shard are 20,207,552 + 4 x 25,000,000 + 5,265,344 elements (the
    last bucket is short: it ends at P)."""
    w = synth.WORKLOADS["llama3-8b"]
    ref = oracle.partition_plan(w.numels, w.n_ranks, w.align)
    P, S = ref.padded_numel, ref.shard_numel
    assert (P, S) == (8_030_265_344, 125_472_896)
    lo, hi = 63 * S, 64 * S
    wins = step.bucket_windows(P, w.bucket, lo, hi)
    assert [b // w.bucket for b, _ in wins] == list(range(321, 315, -1))
    assert wins[0] == (321 * 25_000_000, P - 321 * 25_000_000) and wins[0][1] == 5_265_344
    parts = sorted(min(b + c, hi) - max(b, lo) for b, c in wins)
    assert parts == sorted([20_207_552] + [25_000_000] * 4 + [5_265_344])
    assert sum(parts) == S


@pytest.mark.parametrize("seed", range(20))
def test_bucket_windows_cover_the_shard_once(step, seed):
    rng = np.random.default_rng(seed)
    P = int(rng.integers(1, 10_000)) * 8
    bucket = int(rng.integers(1, 3_000))
    lo = int(rng.integers(0, P))
    hi = int(rng.integers(lo + 1, P + 1))
    wins = step.bucket_windows(P, bucket, lo, hi)
    begins = [b for b, _ in wins]
    assert begins == sorted(begins, reverse=True)            # backward order
    covered = np.zeros(P, np.int32)
    for b, c in wins:
        assert b % bucket == 0 and 0 < c <= bucket and b + c <= P
        covered[b:b + c] += 1
    assert (covered[lo:hi] == 1).all()                          # every shard element once
    assert (covered <= 1).all()
    assert step.bucket_windows(P, 0, lo, hi) == [(0, P)]       # no buckets: the whole buffer


def test_staggered_arena_layout(step):
    specs = [(1000, torch.float32), (333, torch.int16), (5, torch.float32), (4096, torch.int16)]
    views, arena = step._staggered_arena(specs, torch.device("cpu"))
    base = arena.data_ptr()
    prev_end = None
    for (n, dt), v in zip(specs, views):
        assert v.dtype == dt and v.numel() == n and v.is_contiguous()
        start = v.data_ptr() - base
        assert start % 256 == 0
        if prev_end is not None:
            assert start >= prev_end + step.STAGGER                 # no overlap, staggered
            assert start - prev_end < step.STAGGER + 256
        prev_end = start + n * v.element_size()
        assert (v == 0).all()                                       # zero-filled
    assert prev_end <= arena.numel()


def test_rank_step_chooses_the_one_pass_update_only_where_it_applies(step):
    """RankStep.step's choice between the one-pass update (reduce_update) and
    reduce, clip, AdamW, checked on the host with the device calls replaced by
    recorders: one pass only without clipping, without offload, with fusing on,
    over disjoint windows of at most FUSE_MAX_REPLICAS replicas."""
    import zero_partitioned_mixed_partition_amd as zm
    plan = zm.zero_partition_plan([1000, 37, 4096, 3, 777], 4, 128)
    reps = lambda n: [torch.zeros(700, dtype=torch.int16) for _ in range(n)]   # noqa: E731

    def taken(max_norm, windows, fuse=True):
        rs = step.RankStep(plan, 2, len(windows), step.Hyper(), max_norm, torch.device("cpu"),
                           gather=False, fuse=fuse)
        calls = []
        rs.reduce_update = lambda w, s=None: calls.append("one-pass")
        rs.reduce = lambda w, s=None: calls.append("reduce")
        rs.clip = lambda s=None: calls.append("clip")
        rs.adamw = lambda s=None: calls.append("adamw")
        rs.gather = lambda s=None: calls.append("gather")
        rs.step(windows)
        return calls

    disjoint = [(4200, 700, reps(5)), (3500, 700, reps(5)), (2800, 700, reps(5))]
    two_calls = ["reduce", "clip", "adamw", "gather"]
    assert taken(0.0, disjoint) == ["one-pass", "gather"]
    assert taken(1.0, disjoint) == two_calls                      # clipping needs the norm first
    assert taken(0.0, disjoint, fuse=False) == two_calls
    assert taken(0.0, [(3500, 700, reps(9))]) == two_calls        # more than 8 replicas
    assert taken(0.0, [(3500, 700, reps(8)), (4200, 0, reps(9))]) == two_calls
    assert taken(0.0, [(3500, 700, reps(8))]) == ["one-pass", "gather"]
    assert taken(0.0, [(3500, 700, reps(5)), (3900, 700, reps(5))]) == two_calls   # overlap

    rs = step.RankStep(plan, 2, 2, step.Hyper(), 0.0, torch.device("cpu"), gather=False)
    with pytest.raises(ValueError, match="overlap"):
        rs.reduce_update([(3500, 700, reps(5)), (3900, 700, reps(5))])
    with pytest.raises(ValueError, match="window count"):
        rs.reduce_update([(3500, 700, reps(5))])
    rs = step.RankStep(plan, 2, 1, step.Hyper(), 1.0, torch.device("cpu"), gather=False)
    with pytest.raises(ValueError, match="without"):
        rs.reduce_update([(3500, 700, reps(5))])
    assert rs.t == 0
    # per-parameter state keeps the two calls, and cannot be combined with offload
    rs = step.RankStep(plan, 2, 3, step.Hyper(), 0.0, torch.device("cpu"), gather=False,
                       per_param=True)
    calls = []
    rs.reduce_update = lambda w, s=None: calls.append("one-pass")
    rs.reduce = lambda w, s=None: calls.append("reduce")
    rs.clip = lambda s=None: calls.append("clip")
    rs.adamw = lambda s=None: calls.append("adamw")
    rs.gather = lambda s=None: calls.append("gather")
    rs.step(disjoint)
    assert calls == two_calls
    assert rs.master is None and len(rs.master_tensors) == len(plan.segments(2))
    assert [t.numel() for t in rs.master_tensors] == [ln for (_, _, _, ln) in plan.segments(2)]
    with pytest.raises(ValueError, match="separate layouts"):
        step.RankStep(plan, 2, 1, step.Hyper(), 1.0, torch.device("cpu"), offload=True, per_param=True)
    # the device-counted step takes device state (not ZeRO-Offload's), and chooses its calls
    # as the host-counted step does
    with pytest.raises(ValueError, match="not ZeRO-Offload"):
        step.RankStep(plan, 2, 1, step.Hyper(), 1.0, torch.device("cpu"), device_step=True, offload=True)
    for max_norm, want in ((0.0, ["one-pass", "gather"]), (1.0, two_calls)):
        rs = step.RankStep(plan, 2, 3, step.Hyper(), max_norm, torch.device("cpu"), gather=False)
        rs.device_step = True           # (the schedule itself needs a GPU)
        calls = []
        rs.reduce_update = lambda w, s=None: calls.append("one-pass")
        rs.reduce = lambda w, s=None: calls.append("reduce")
        rs.clip = lambda s=None: calls.append("clip")
        rs.adamw = lambda s=None: calls.append("adamw")
        rs.gather = lambda s=None: calls.append("gather")
        rs.step(disjoint)
        assert calls == want
