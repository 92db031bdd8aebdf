"""Every call runs on the stream it is given (or torch's current stream): work
queued before it on that stream comes first.

Each check queues a bounded spin on a side stream (torch.cuda._sleep, a fixed
number of cycles), then copies the call's inputs into place on that stream,
then makes the call. torch's pool streams do not wait for the null stream or
for each other, so a call issued on any other stream would read its inputs
before the copies land and differ from the oracle. The side streams keep the
default priority. Expected values come from the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import (assert_bf16_close, assert_bits_equal, assert_f32_close, dev, host_f32,
                      host_u16, needs_gpu, note, to_dev_f32, to_dev_u16)

pytestmark = [pytest.mark.gpu, needs_gpu,
              pytest.mark.skipif(not hasattr(torch.cuda, "_sleep"), reason="needs torch.cuda._sleep")]

SPIN_CYCLES = 20_000_000     # a few milliseconds of one spinning wave, then it ends

NUMELS = [1000, 37, 4096, 3, 777]
N_RANKS, RANK = 4, 2


@pytest.fixture(scope="module")
def zm():
    import zero_partitioned_mixed_partition_amd as m
    torch.cuda.set_device(0)
    return m


def _late(stream, pairs):
    """On `stream`: the spin, then dst.copy_(src) for each pair. Checks that the
    stream is still busy afterwards, so the call the caller issues next really
    is queued ahead of its inputs."""
    with torch.cuda.stream(stream):
        torch.cuda._sleep(SPIN_CYCLES)
        for dst, src in pairs:
            dst.copy_(src)
    assert not stream.query(), "the spin ended before the call was issued"


@pytest.mark.parametrize("how", ["current-stream", "explicit-handle"])
def test_rank_step_with_clip_runs_on_its_stream(zm, how):
    """RankStep's reduce, clip, AdamW and gather on a side stream, the gradient
    replicas landing on that stream just before: two steps against the oracle's
    rank step. 'current-stream' issues inside torch.cuda.stream(s) with no
    stream argument; 'explicit-handle' passes s's handle from outside it."""
    from zero_partitioned_mixed_partition_amd.step import Hyper, RankStep
    plan = zm.zero_partition_plan(NUMELS, N_RANKS, 128)
    ref = oracle.partition_plan(NUMELS, N_RANKS, 128)
    P, S, phi = ref.padded_numel, ref.shard_numel, ref.numel
    hyper, R = Hyper(), 3
    rs = RankStep(plan, RANK, 1, hyper, 1.0, dev(), gather=True)
    master = synth.normal_f32(S, 71, synth.KIND_MASTER, 0, 0, RANK * S, phi, 0.02)
    rs.master.copy_(torch.from_numpy(master))
    shards = [synth.normal_bf16(S, 71, synth.KIND_PARAM, 0, 0, r * S, phi, 0.02) for r in range(N_RANKS)]
    for r in range(N_RANKS):
        if r != RANK:
            rs.param_shards[r].copy_(to_dev_u16(shards[r]))
    shards[RANK] = np.zeros(S, np.uint16)
    state = {"master": master.copy(), "exp_avg": np.zeros(S, np.float32),
             "exp_avg_sq": np.zeros(S, np.float32)}
    remote = [0.2, 0.1, 0.0, 0.05]
    reps = [torch.zeros(P, dtype=torch.int16, device=dev()) for _ in range(R)]
    s = torch.cuda.Stream()
    for t in (1, 2):
        full = [synth.normal_bf16(P, 72, synth.KIND_REPLICA, t, k, 0, phi, 0.05) for k in range(R)]
        src = [to_dev_u16(x) for x in full]
        rs.set_remote_partials(remote)
        torch.cuda.synchronize()
        note(f"stream rank step ({how}) step {t}")
        _late(s, list(zip(reps, src)))
        if how == "current-stream":
            with torch.cuda.stream(s):
                rs.step([(0, P, reps)])
        else:
            rs.step([(0, P, reps)], stream=s.cuda_stream)
        want = oracle.rank_step(ref, RANK, full, 0, state, shards, remote, t, hyper.as_kwargs(), 1.0)
        torch.cuda.synchronize()
        assert_bits_equal(host_u16(rs.grad), want["shard_grad"], f"step {t} gradient")
        for got, key in ((rs.master, "master"), (rs.exp_avg, "exp_avg"), (rs.exp_avg_sq, "exp_avg_sq")):
            assert_f32_close(host_f32(got), state[key], f"step {t} {key}")
        assert_bf16_close(host_u16(rs.param_shards[RANK]), shards[RANK], f"step {t} shard")
        for i, (a, b) in enumerate(zip(rs.tensors, want["tensors"])):
            assert_bf16_close(host_u16(a), b, f"step {t} tensor {i}")


def test_one_pass_and_table_calls_run_on_their_stream(zm):
    """The one-pass reduce and update, the reduce from per-tensor replicas, the
    no-allocation reduce, the multi-tensor AdamW (list and table) and the
    flatten, each issued on a side stream just after its inputs land there,
    against the oracle."""
    ref = oracle.partition_plan(NUMELS, N_RANKS, 128)
    plan = zm.zero_partition_plan(NUMELS, N_RANKS, 128)
    P, S, phi = ref.padded_numel, ref.shard_numel, ref.numel
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    s = torch.cuda.Stream()
    h = s.cuda_stream
    R = 3
    full = [synth.normal_bf16(P, 81, synth.KIND_REPLICA, 1, k, 0, phi, 0.05) for k in range(R)]
    want_grad = np.zeros(S, np.uint16)
    oracle.reduce_shard(ref, RANK, full, 0, want_grad)
    src = [to_dev_u16(x) for x in full]

    # one-pass reduce and update
    master = synth.normal_f32(S, 82, synth.KIND_MASTER, 0, 0, RANK * S, phi, 0.02)
    p, m, v = to_dev_f32(master), torch.zeros(S, device=dev()), torch.zeros(S, device=dev())
    out = torch.zeros(S, dtype=torch.int16, device=dev())
    grad = torch.zeros(S, dtype=torch.int16, device=dev())
    reps = [torch.zeros(P, dtype=torch.int16, device=dev()) for _ in range(R)]
    torch.cuda.synchronize()
    note("stream: one-pass reduce and update")
    _late(s, list(zip(reps, src)))
    zm.zero_reduce_adamw_step(plan, RANK, reps, 0, P, p, m, v, out, 1, shard_grad=grad, stream=h, **hp)
    wp, wm, wv, wbits = oracle.adamw_step(master, np.zeros(S, np.float32), np.zeros(S, np.float32),
                                          want_grad, 1, **hp)
    torch.cuda.synchronize()
    assert_bits_equal(host_u16(grad), want_grad, "one-pass gradient")
    assert_bits_equal(host_f32(p).view(np.uint32), wp.view(np.uint32), "one-pass master")
    assert_bits_equal(host_u16(out), wbits, "one-pass param")

    # the no-allocation reduce, with its norm
    g2 = torch.zeros(S, dtype=torch.int16, device=dev())
    sq = torch.zeros(1, dtype=torch.float64, device=dev())
    reps2 = [torch.zeros(P, dtype=torch.int16, device=dev()) for _ in range(R)]
    torch.cuda.synchronize()
    note("stream: no-allocation reduce")
    _late(s, list(zip(reps2, src)))
    zm.zero_grad_reduce_shard_noalloc(plan, RANK, reps2, 0, P, g2, sqnorm_out=sq, stream=h)
    torch.cuda.synchronize()
    assert_bits_equal(host_u16(g2), want_grad, "no-allocation gradient")
    want_sq = oracle.sqnorm(want_grad)
    assert abs(float(sq.item()) - want_sq) <= 1e-12 * want_sq

    # the reduce from per-tensor replicas
    offs = ref.offsets
    tens = [[torch.zeros(n, dtype=torch.int16, device=dev()) for n in NUMELS] for _ in range(R)]
    pairs = [(tens[k][t], src[k][offs[t]:offs[t] + n]) for k in range(R) for t, n in enumerate(NUMELS)]
    g3 = torch.zeros(S, dtype=torch.int16, device=dev())
    table = zm.ReduceTable(plan, RANK, tens, g3)
    sq3 = torch.zeros(1, dtype=torch.float64, device=dev())
    torch.cuda.synchronize()
    note("stream: reduce table")
    _late(s, pairs)
    table.run(sq3, stream=h)
    torch.cuda.synchronize()
    assert_bits_equal(host_u16(g3), want_grad, "reduce-table gradient")
    assert abs(float(sq3.item()) - want_sq) <= 1e-12 * want_sq

    # the multi-tensor AdamW, list call and table, over three pieces of the shard
    cuts = [(0, 500), (500, 37), (537, S - 537)]
    gsrc = to_dev_u16(want_grad)
    for form in ("list", "table"):
        ms = [to_dev_f32(master[a:a + n]) for a, n in cuts]
        es = [torch.zeros(n, device=dev()) for _, n in cuts]
        vs = [torch.zeros(n, device=dev()) for _, n in cuts]
        gs = [torch.zeros(n, dtype=torch.int16, device=dev()) for _, n in cuts]
        os_ = [torch.zeros(n, dtype=torch.int16, device=dev()) for _, n in cuts]
        mt = zm.MultiTensorTable(ms, es, vs, gs, os_) if form == "table" else None
        torch.cuda.synchronize()
        note(f"stream: multi-tensor AdamW ({form})")
        _late(s, [(gd, gsrc[a:a + n]) for gd, (a, n) in zip(gs, cuts)])
        if form == "table":
            mt.step(1, stream=h, **hp)
        else:
            zm.zero_multi_tensor_adamw_step(ms, es, vs, gs, os_, 1, stream=h, **hp)
        torch.cuda.synchronize()
        for (a, n), pm, po in zip(cuts, ms, os_):
            assert_bits_equal(host_f32(pm).view(np.uint32), wp[a:a + n].view(np.uint32), f"{form} master")
            assert_bits_equal(host_u16(po), wbits[a:a + n], f"{form} param")

    # the flatten of per-tensor buffers
    tensors = [synth.normal_bf16(n, 83, synth.KIND_PARAM, 0, 0, sigma=0.1) for n in NUMELS]
    tsrc = [to_dev_u16(x) for x in tensors]
    tdst = [torch.zeros(n, dtype=torch.int16, device=dev()) for n in NUMELS]
    flat = torch.full((P,), 0x1234, dtype=torch.int16, device=dev())
    torch.cuda.synchronize()
    note("stream: flatten")
    _late(s, list(zip(tdst, tsrc)))
    zm.zero_flatten_params(plan, tdst, flat, stream=h)
    torch.cuda.synchronize()
    assert_bits_equal(host_u16(flat), oracle.flatten_params(ref, tensors), "flatten")
