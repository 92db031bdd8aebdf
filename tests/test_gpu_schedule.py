"""AdamW with the step counted on the device (zero_adamw_schedule_*), on the GPU.

The schedule holds the number of updates applied and the next step's scalars
in device memory, so a step captured in a HIP graph replays successive steps.
Checked against the oracle bit for bit: a captured update-and-advance replayed
over several steps with new gradients between replays, a skipped step (NaN clip
coefficient) that is not counted, steps across the end of the schedule's table,
a learning-rate list, and several updates in one step before one advance.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_bits_equal, dev, host_f32, host_u16, needs_gpu, note, to_dev_f32, to_dev_u16

pytestmark = [pytest.mark.gpu, needs_gpu]

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


@pytest.fixture(scope="module")
def zm():
    import zero_partitioned_mixed_partition_amd as m
    torch.cuda.set_device(0)
    return m


def _inputs(n, seed):
    p = synth.normal_f32(n, seed, synth.KIND_MASTER, 0, 0, sigma=0.02)
    m = synth.normal_f32(n, seed, 10, 0, 0, sigma=1e-4)
    v = np.abs(synth.normal_f32(n, seed, 11, 0, 0, sigma=1e-7))
    return p, m, v


def _grad(n, seed, t):
    return synth.normal_bf16(n, seed, synth.KIND_GRAD, t, 0, sigma=1e-3)


def _check(dp, dm, dv, dout, p, m, v, bits, what):
    assert_bits_equal(host_f32(dp).view(np.uint32), p.view(np.uint32), f"{what} master")
    assert_bits_equal(host_f32(dm).view(np.uint32), m.view(np.uint32), f"{what} exp_avg")
    assert_bits_equal(host_f32(dv).view(np.uint32), v.view(np.uint32), f"{what} exp_avg_sq")
    assert_bits_equal(host_u16(dout), bits, f"{what} param")


def test_captured_update_replays_successive_steps_and_skips_uncounted(zm):
    """Graph: the scheduled update and the advance. Replayed 7 times; before
    each replay the gradient buffer and the clip coefficient are rewritten
    eagerly. Replay 4 carries a NaN coefficient: nothing changes and the step is
    not counted, so the replay after it applies the same step number."""
    n = 100_003
    p, m, v = _inputs(n, 5)
    dp, dm, dv = to_dev_f32(p), to_dev_f32(m), to_dev_f32(v)
    dg = torch.zeros(n, dtype=torch.int16, device=dev())
    dout = torch.zeros(n, dtype=torch.int16, device=dev())
    clip = torch.ones(1, dtype=torch.float32, device=dev())
    sched = zm.AdamWSchedule(HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["weight_decay"])
    assert sched.length == 38_797 and sched.applied() == 0
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        zm.zero_shard_adamw_step_scheduled(dp, dm, dv, dg, dout, sched, clip_scale=clip)
        sched.advance(clip_scale=clip)
    torch.cuda.synchronize()
    assert sched.applied() == 0, "capture ran nothing"
    bits = np.zeros(n, np.uint16)
    t = 0
    coefs = [1.0, 0.5, 0.75, float("nan"), 1.0, 0.25, 1.0]
    for k, coef in enumerate(coefs):
        g = _grad(n, 6, k + 1)
        dg.copy_(to_dev_u16(g))
        clip.fill_(coef)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        if math.isfinite(coef):
            t += 1
            p, m, v, bits = oracle.adamw_step(p, m, v, g, t, clip=coef, **HP)
        note(f"replay {k}: coefficient {coef}, applied {sched.applied()}")
        assert sched.applied() == t
        _check(dp, dm, dv, dout, p, m, v, bits, f"replay {k}")


def test_steps_across_the_end_of_the_table_match_the_plain_call(zm):
    """first_step three before the table's end: six eager scheduled steps (one
    advance each) against zero_shard_adamw_step with the same step numbers and
    the oracle."""
    n = 4097
    L = 38_797
    p, m, v = _inputs(n, 8)
    a = [to_dev_f32(x) for x in (p, m, v)]
    b = [to_dev_f32(x) for x in (p, m, v)]
    a_out = torch.zeros(n, dtype=torch.int16, device=dev())
    b_out = torch.zeros(n, dtype=torch.int16, device=dev())
    sched = zm.AdamWSchedule(HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["weight_decay"],
                             first_step=L - 3)
    for t in range(L - 3, L + 3):
        g = _grad(n, 9, t)
        dg = to_dev_u16(g)
        zm.zero_shard_adamw_step_scheduled(*a, dg, a_out, sched)
        sched.advance()
        zm.zero_shard_adamw_step(*b, dg, b_out, t, **HP)
        p, m, v, bits = oracle.adamw_step(p, m, v, g, t, **HP)
        torch.cuda.synchronize()
        _check(*a, a_out, p, m, v, bits, f"scheduled step {t}")
        _check(*b, b_out, p, m, v, bits, f"plain step {t}")
    assert sched.applied() == L + 2


def test_learning_rate_list_and_several_updates_per_step(zm):
    """lr = [1e-3, 2e-3, 3e-3]: steps 1..5 use 1e-3, 2e-3, 3e-3, 3e-3, 3e-3. Each
    step updates the shard as two halves with the same schedule, then advances
    once: the same bits as the oracle's whole-shard step."""
    n = 20_011
    cut = 7_000
    rates = [1e-3, 2e-3, 3e-3]
    p, m, v = _inputs(n, 12)
    dp, dm, dv = to_dev_f32(p), to_dev_f32(m), to_dev_f32(v)
    dout = torch.zeros(n, dtype=torch.int16, device=dev())
    sched = zm.AdamWSchedule(rates, HP["beta1"], HP["beta2"], HP["eps"], HP["weight_decay"])
    hp = dict(HP)
    for t in range(1, 6):
        g = _grad(n, 13, t)
        dg = to_dev_u16(g)
        for sl in (slice(0, cut), slice(cut, n)):
            zm.zero_shard_adamw_step_scheduled(dp[sl], dm[sl], dv[sl], dg[sl], dout[sl], sched)
        sched.advance()
        hp["lr"] = rates[min(t, len(rates)) - 1]
        p, m, v, bits = oracle.adamw_step(p, m, v, g, t, **hp)
        torch.cuda.synchronize()
        _check(dp, dm, dv, dout, p, m, v, bits, f"step {t}")
    assert sched.applied() == 5


def test_captured_rank_step_with_the_step_on_the_device(zm):
    """A whole RankStep(device_step=True) (reduce with its norm, clip, the
    scheduled AdamW and its advance, the gather through its copy table) captured
    in a HIP graph after one eager step on the same stream (which builds every
    table the step uses), then replayed with new replicas written between
    replays. The fourth iteration's replicas hold an infinity in the rank's
    slice: its norm is not finite, the update is skipped and not counted, and
    the next replay applies step 4. Against the oracle's rank step: the gradient
    bit for bit, the state and parameters to the bars (the device adds the norm
    partials in its own order)."""
    from gpu_util import assert_bf16_close, assert_f32_close
    from zero_partitioned_mixed_partition_amd.step import Hyper, RankStep
    numels = [1000, 37, 4096, 3, 777]
    n_ranks, rank, R = 4, 2, 3
    plan = zm.zero_partition_plan(numels, n_ranks, 128)
    ref = oracle.partition_plan(numels, n_ranks, 128)
    P, S, phi = ref.padded_numel, ref.shard_numel, ref.numel
    hyper = Hyper()
    rs = RankStep(plan, rank, 1, hyper, 1.0, dev(), gather=True, device_step=True)
    master = synth.normal_f32(S, 93, synth.KIND_MASTER, 0, 0, rank * S, phi, 0.02)
    rs.master.copy_(torch.from_numpy(master))
    shards = [synth.normal_bf16(S, 93, synth.KIND_PARAM, 0, 0, r * S, phi, 0.02) for r in range(n_ranks)]
    for r in range(n_ranks):
        if r != rank:
            rs.param_shards[r].copy_(to_dev_u16(shards[r]))
    shards[rank] = np.zeros(S, np.uint16)
    state = {"master": master.copy(), "exp_avg": np.zeros(S, np.float32),
             "exp_avg_sq": np.zeros(S, np.float32)}
    remote = [0.2, 0.1, 0.0, 0.05]
    rs.set_remote_partials(remote)
    reps = [torch.zeros(P, dtype=torch.int16, device=dev()) for _ in range(R)]
    windows = [(0, P, reps)]
    s = torch.cuda.Stream()

    def write(it):
        full = [synth.normal_bf16(P, 94, synth.KIND_REPLICA, it, k, 0, phi, 0.05) for k in range(R)]
        if it == 4:
            full[1][rank * S + 5] = 0x7F80          # +inf inside this rank's slice
        for d, h in zip(reps, full):
            d.copy_(to_dev_u16(h))
        torch.cuda.synchronize()
        return full

    graph = torch.cuda.CUDAGraph()
    applied = 0
    for it in range(1, 6):
        full = write(it)
        if it == 1:
            rs.step(windows, stream=s.cuda_stream)               # eager: builds the tables
            torch.cuda.synchronize()
            with torch.cuda.graph(graph, stream=s):
                rs.step(windows, stream=s.cuda_stream)
            torch.cuda.synchronize()
        else:
            graph.replay()
            torch.cuda.synchronize()
        want = oracle.rank_step(ref, rank, full, 0, state, shards, remote, applied + 1,
                                hyper.as_kwargs(), 1.0)
        if np.isfinite(want["clip"]):
            applied += 1
        note(f"iteration {it}: clip {want['clip']}, applied {rs.steps_applied()}")
        assert rs.steps_applied() == applied
        assert_bits_equal(host_u16(rs.grad), want["shard_grad"], f"iteration {it} gradient")
        for got, key in ((rs.master, "master"), (rs.exp_avg, "exp_avg"), (rs.exp_avg_sq, "exp_avg_sq")):
            assert_f32_close(host_f32(got), state[key], f"iteration {it} {key}")
        assert_bf16_close(host_u16(rs.param_shards[rank]), shards[rank], f"iteration {it} shard")
        for i, (a, b) in enumerate(zip(rs.tensors, want["tensors"])):
            assert_bf16_close(host_u16(a), b, f"iteration {it} tensor {i}")
    assert applied == 4


def test_scheduled_table_and_one_pass_match_their_plain_forms(zm):
    """The multi-tensor table step and the one-pass reduce and update, scheduled
    (one advance per step) against their plain forms with the host's step
    number and against the oracle, bit for bit; the table's third step carries
    a NaN coefficient and is neither applied nor counted."""
    hp = HP
    # multi-tensor table over three tensors
    lens = [5000, 37, 20_011]
    ins = [_inputs(n, 20 + i) for i, n in enumerate(lens)]
    A = [[to_dev_f32(x) for x in st] for st in ins]
    B = [[to_dev_f32(x) for x in st] for st in ins]
    gs = [torch.zeros(n, dtype=torch.int16, device=dev()) for n in lens]
    a_out = [torch.zeros(n, dtype=torch.int16, device=dev()) for n in lens]
    b_out = [torch.zeros(n, dtype=torch.int16, device=dev()) for n in lens]
    ta = zm.MultiTensorTable([a[0] for a in A], [a[1] for a in A], [a[2] for a in A], gs, a_out)
    tb = zm.MultiTensorTable([b[0] for b in B], [b[1] for b in B], [b[2] for b in B], gs, b_out)
    sched = zm.AdamWSchedule(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"])
    clip = torch.ones(1, dtype=torch.float32, device=dev())
    want = [list(st) for st in ins]
    bits = [np.zeros(n, np.uint16) for n in lens]
    t = 0
    for it, coef in enumerate([1.0, 0.5, float("nan"), 0.75]):
        host_g = [_grad(n, 30 + i, it) for i, n in enumerate(lens)]
        for d, h in zip(gs, host_g):
            d.copy_(to_dev_u16(h))
        clip.fill_(coef)
        ta.step_scheduled(sched, clip_scale=clip)
        sched.advance(clip_scale=clip)
        if math.isfinite(coef):
            t += 1
            tb.step(t, clip_scale=clip, **hp)
            for i in range(len(lens)):
                p, m, v, b = oracle.adamw_step(*want[i], host_g[i], t, clip=coef, **hp)
                want[i], bits[i] = [p, m, v], b
        torch.cuda.synchronize()
        assert sched.applied() == t
        for i in range(len(lens)):
            _check(*A[i], a_out[i], *want[i], bits[i], f"table iteration {it} tensor {i}")
            _check(*B[i], b_out[i], *want[i], bits[i], f"plain table iteration {it} tensor {i}")
    # one-pass reduce and update: rank 1 of a 2-rank plan, three replicas
    numels = [30_000, 7, 12_345]
    plan = zm.zero_partition_plan(numels, 2, 128)
    ref = oracle.partition_plan(numels, 2, 128)
    P, S, phi = ref.padded_numel, ref.shard_numel, ref.numel
    master = synth.normal_f32(S, 40, synth.KIND_MASTER, 0, 0, S, phi, 0.02)
    fa = [to_dev_f32(master), torch.zeros(S, device=dev()), torch.zeros(S, device=dev())]
    fb = [to_dev_f32(master), torch.zeros(S, device=dev()), torch.zeros(S, device=dev())]
    pa = torch.zeros(S, dtype=torch.int16, device=dev())
    pb = torch.zeros(S, dtype=torch.int16, device=dev())
    sched2 = zm.AdamWSchedule(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"])
    p, m, v = master.copy(), np.zeros(S, np.float32), np.zeros(S, np.float32)
    for t in (1, 2, 3):
        full = [synth.normal_bf16(P, 41, synth.KIND_REPLICA, t, k, 0, phi, 0.05) for k in range(3)]
        reps = [to_dev_u16(x) for x in full]
        zm.zero_reduce_adamw_step_scheduled(plan, 1, reps, 0, P, *fa, pa, sched2)
        sched2.advance()
        zm.zero_reduce_adamw_step(plan, 1, reps, 0, P, *fb, pb, t, **hp)
        g = np.zeros(S, np.uint16)
        oracle.reduce_shard(ref, 1, full, 0, g)
        p, m, v, bits1 = oracle.adamw_step(p, m, v, g, t, **hp)
        torch.cuda.synchronize()
        _check(*fa, pa, p, m, v, bits1, f"one-pass scheduled step {t}")
        _check(*fb, pb, p, m, v, bits1, f"one-pass plain step {t}")
    assert sched2.applied() == 3


@pytest.mark.parametrize("mode", ["per-parameter", "one-pass"])
def test_rank_step_device_step_equals_the_host_counted_step(zm, mode):
    """RankStep(device_step=True) against RankStep with the step counted on the
    host, on the same inputs, three steps, bit for bit: FSDP-2's per-parameter
    state (clipped, through the multi-tensor table), or the one-pass reduce and
    update over three bucket windows (no clipping)."""
    from zero_partitioned_mixed_partition_amd.step import Hyper, RankStep, rank_step_plan_windows
    numels = [1000 * 16, 37 * 16, 4096, 3 * 16, 777 * 16]
    dim0 = [1000, 37, 4096, 3, 777]
    n_ranks, rank, R = 4, 2, 3
    if mode == "per-parameter":
        plan = zm.zero_partition_plan_shard0(numels, dim0, n_ranks, 128)
        kw, max_norm, bucket = dict(per_param=True), 1.0, 0
    else:
        plan = zm.zero_partition_plan(numels, n_ranks, 128)
        kw, max_norm, bucket = dict(), 0.0, 7000
    P, S, phi = plan.padded_numel, plan.shard_numel, plan.numel
    wins = rank_step_plan_windows(plan, rank, bucket)
    steps = [RankStep(plan, rank, len(wins), Hyper(), max_norm, dev(), gather=True, device_step=d, **kw)
             for d in (True, False)]
    master = synth.normal_f32(S, 50, synth.KIND_MASTER, 0, 0, rank * S, phi, 0.02)
    for rs in steps:
        if mode == "per-parameter":
            for tt, (_, _, soff, ln) in zip(rs.master_tensors, rs.segments):
                tt.copy_(torch.from_numpy(master[soff:soff + ln]))
        else:
            rs.master.copy_(torch.from_numpy(master))
        rs.set_remote_partials([0.3, 0.1, 0.0, 0.2])
    for t in (1, 2, 3):
        full = [synth.normal_bf16(P, 51, synth.KIND_REPLICA, t, k, 0, phi, 0.05) for k in range(R)]
        dfull = [to_dev_u16(x) for x in full]
        for rs in steps:
            rs.step([(b, c, [x[b:b + c] for x in dfull]) for b, c in wins])
        torch.cuda.synchronize()
        a, b = steps
        if mode == "per-parameter":
            pairs = list(zip(a.master_tensors + a.exp_avg_tensors + a.exp_avg_sq_tensors,
                             b.master_tensors + b.exp_avg_tensors + b.exp_avg_sq_tensors))
        else:
            pairs = [(a.master, b.master), (a.exp_avg, b.exp_avg), (a.exp_avg_sq, b.exp_avg_sq)]
        for x, y in pairs:
            assert torch.equal(x.view(torch.int32), y.view(torch.int32)), f"{mode} step {t}: fp32 state"
        assert torch.equal(a.param_shards[rank], b.param_shards[rank]), f"{mode} step {t}: shard"
        for x, y in zip(a.tensors, b.tensors):
            assert torch.equal(x, y), f"{mode} step {t}: tensors"
        assert a.steps_applied() == b.steps_applied() == t
    assert ("reduce_update", 0) in steps[0]._calls if mode == "one-pass" else "adamw" in steps[0]._calls
