"""A rank step captured in a HIP graph (torch.cuda.graph) and replayed.

The caller the no-allocation reduce is for: code under graph capture, which
cannot allocate. The captured step is zero_grad_reduce_shard_noalloc (norm
partials in the library's device array), zero_clip_scale, and AdamW with its
step number counted on the device (zero_shard_adamw_step_scheduled and
zero_adamw_schedule_advance), so replay k applies step k; the device buffers
and the schedule are allocated before capture. The graph is replayed four
times with the program's own eager work (a second, uncaptured reduce into
another buffer, host synchronisations) between the replays, and after every
replay the gradient, the fp32 state and the bf16 parameters are compared bit
for bit with an eager run of the same steps through the workspace entry points
and the host-counted AdamW, and with the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_bits_equal, dev, host_f32, host_u16, needs_gpu, note, to_dev_u16

pytestmark = [pytest.mark.gpu, needs_gpu]

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


@pytest.fixture(scope="module")
def zm():
    import zero_partitioned_mixed_partition_amd as m
    torch.cuda.set_device(0)
    return m


def test_captured_rank_step_replays_match_eager_and_oracle(zm):
    numels = [1_000_003, 4096, 3]
    n_ranks, rank, R, max_norm = 4, 2, 5, 1.0
    plan = zm.zero_partition_plan(numels, n_ranks, 128)
    ref = oracle.partition_plan(numels, n_ranks, 128)
    P, S, phi = ref.padded_numel, ref.shard_numel, ref.numel
    reps_h = [synth.normal_bf16(P, 77, synth.KIND_REPLICA, 1, k, 0, phi, 0.05) for k in range(R)]
    reps = [to_dev_u16(x) for x in reps_h]
    master0 = synth.normal_f32(S, 77, synth.KIND_MASTER, 0, 0, rank * S, phi, 0.02)
    remote = [0.5, 0.25, 0.0, 0.75]                    # the other ranks' partials (slot 2 is own)

    def state():
        return {"master": torch.from_numpy(master0.copy()).to(dev()),
                "m": torch.zeros(S, dtype=torch.float32, device=dev()),
                "v": torch.zeros(S, dtype=torch.float32, device=dev()),
                "grad": torch.zeros(S, dtype=torch.int16, device=dev()),
                "param": torch.zeros(S, dtype=torch.int16, device=dev()),
                "parts": torch.tensor(remote, dtype=torch.float64, device=dev()),
                "scale": torch.zeros(1, dtype=torch.float32, device=dev())}

    g_st, e_st = state(), state()
    sched = zm.AdamWSchedule(HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["weight_decay"])
    ws = zm.sqnorm_workspace(dev())
    # the first call on the device, outside capture: it looks up the array's address
    zm.zero_grad_reduce_shard_noalloc(plan, rank, reps, 0, P, g_st["grad"],
                                      sqnorm_out=g_st["parts"][rank:rank + 1])
    torch.cuda.synchronize()

    def step(st, noalloc, t=None):
        if noalloc:
            zm.zero_grad_reduce_shard_noalloc(plan, rank, reps, 0, P, st["grad"],
                                              sqnorm_out=st["parts"][rank:rank + 1])
        else:
            big = torch.empty(zm.ZERO_NOALLOC_SCRATCH_BYTES, dtype=torch.uint8, device=dev())
            zm.zero_grad_reduce_shard(plan, rank, reps, 0, P, st["grad"],
                                      sqnorm_out=st["parts"][rank:rank + 1], workspace=big)
        zm.zero_clip_scale(st["parts"], max_norm, st["scale"])
        if noalloc:             # the step number on the device
            zm.zero_shard_adamw_step_scheduled(st["master"], st["m"], st["v"], st["grad"], st["param"],
                                               sched, clip_scale=st["scale"])
            sched.advance(clip_scale=st["scale"])
        else:
            zm.zero_shard_adamw_step(st["master"], st["m"], st["v"], st["grad"], st["param"], t,
                                     clip_scale=st["scale"], **HP)

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):                       # recorded, not run
        step(g_st, True)
    torch.cuda.synchronize()
    assert not host_u16(g_st["param"]).any(), "capture ran nothing"

    o_state = {"master": master0.copy(), "exp_avg": np.zeros(S, np.float32),
               "exp_avg_sq": np.zeros(S, np.float32)}
    o_shards = [np.zeros(S, np.uint16) for _ in range(n_ranks)]
    other = torch.zeros(S, dtype=torch.int16, device=dev())
    for k in range(4):
        graph.replay()
        torch.cuda.synchronize()
        step(e_st, False, k + 1)                        # eager, the workspace entry point
        zm.zero_grad_reduce_shard(plan, (rank + 1) % n_ranks, reps, 0, P, other)   # unrelated eager work
        torch.cuda.synchronize()
        want = oracle.rank_step(ref, rank, reps_h, 0, o_state, o_shards, remote, k + 1, HP, max_norm)
        assert sched.applied() == k + 1
        note(f"graph replay {k}: clip {g_st['scale'].item()} (eager {e_st['scale'].item()}, "
             f"oracle {want['clip']})")
        for key in ("grad", "param"):
            assert torch.equal(g_st[key], e_st[key]), f"replay {k}: {key} differs from eager"
        for key in ("master", "m", "v"):
            assert torch.equal(g_st[key].view(torch.int32), e_st[key].view(torch.int32)), \
                f"replay {k}: {key} differs from eager"
        assert torch.equal(g_st["parts"], e_st["parts"]) and torch.equal(g_st["scale"], e_st["scale"])
        assert_bits_equal(host_u16(g_st["grad"]), want["shard_grad"], f"replay {k}: grad vs oracle")
        got_scale = np.float32(g_st["scale"].item())
        assert abs(int(got_scale.view(np.int32)) - int(np.float32(want["clip"]).view(np.int32))) <= 1
        if got_scale == np.float32(want["clip"]):
            for key, okey in (("master", "master"), ("m", "exp_avg"), ("v", "exp_avg_sq")):
                assert_bits_equal(host_f32(g_st[key]).view(np.uint32), o_state[okey].view(np.uint32),
                                  f"replay {k}: {key} vs oracle")
            assert_bits_equal(host_u16(g_st["param"]), o_shards[rank], f"replay {k}: param vs oracle")
