"""GPU parity on the model-shaped workloads, in the launch configuration the
benchmark times (the same RankStep call sequence and the same kernels).

tiny-a / tiny-b  1M-parameter flat model, N_d = 4, every shard stepped in turn,
                 gathered every step, 10 steps: full arrays against the oracle.
gpt2-small       GPT-2-small tensor list, N_d = 8, rank 7 (15.6M elements),
                 already-averaged gradients, global-norm clip 1.0, 100 steps:
                 the oracle computes every step's global norm over all 8 ranks
                 (124M values), and the full fp32 state and bf16 parameters of
                 every step, compared bit for bit through per-window digests.
bench pipeline   the benchmark's own step (8 replicas reduced for rank 7, fused
                 norm, clip, AdamW, gather of 148 tensors): full arrays for 2 steps;
                 also on the Shard(0) layout and with the AdamW offloaded to the host.
all ranks        the benchmark's own 1.3B GPT step (every rank's reduce and AdamW,
                 as two calls or in one pass, then the gather of 292 tensors): two
                 steps, windows at every rank's ends and across rank boundaries.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import (assert_bf16_close, assert_bits_equal, assert_f32_close, dev, host_f32,
                      host_u16, needs_gpu, note, to_dev_u16)

pytestmark = [pytest.mark.gpu, needs_gpu]

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


@pytest.fixture(scope="module")
def zm():
    import zero_partitioned_mixed_partition_amd as m
    torch.cuda.set_device(0)
    return m


@pytest.mark.parametrize("name", ["tiny-a", "tiny-b"])
def test_tiny_all_shards_ten_steps(zm, name):
    w = synth.WORKLOADS[name]
    ref = oracle.partition_plan(w.numels, w.n_ranks, w.align)
    plan = zm.zero_partition_plan(w.numels, w.n_ranks, w.align)
    P, S, phi = ref.padded_numel, ref.shard_numel, ref.numel
    note(f"{name}: Phi={phi} P={P} S={S} T={len(w.numels)}")
    master = synth.normal_f32(P, w.seed, synth.KIND_MASTER, 0, 0, 0, phi, synth.MASTER_SIGMA)
    states = [{"master": master[r * S:(r + 1) * S].copy(), "exp_avg": np.zeros(S, np.float32),
               "exp_avg_sq": np.zeros(S, np.float32)} for r in range(w.n_ranks)]
    shards = [np.zeros(S, np.uint16) for _ in range(w.n_ranks)]
    d_master = torch.from_numpy(master).to(dev())
    d_m = torch.zeros(P, dtype=torch.float32, device=dev())
    d_v = torch.zeros(P, dtype=torch.float32, device=dev())
    d_grad = torch.empty(P, dtype=torch.int16, device=dev())
    d_param = torch.zeros(P, dtype=torch.int16, device=dev())
    d_tensors = [torch.empty(n, dtype=torch.int16, device=dev()) for n in w.numels]
    d_shards = [d_param[r * S:(r + 1) * S] for r in range(w.n_ranks)]
    for t in range(1, w.steps + 1):
        synth.device_normal_bf16(d_grad, w.seed, synth.KIND_GRAD, t, 0, 0, phi, synth.GRAD_SIGMA)
        g = synth.normal_bf16(P, w.seed, synth.KIND_GRAD, t, 0, 0, phi, synth.GRAD_SIGMA)
        for r in range(w.n_ranks):
            sl = slice(r * S, (r + 1) * S)
            zm.zero_shard_adamw_step(d_master[sl], d_m[sl], d_v[sl], d_grad[sl], d_shards[r], t,
                                     lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                                     weight_decay=w.weight_decay)
            st = states[r]
            st["master"], st["exp_avg"], st["exp_avg_sq"], shards[r] = oracle.adamw_step(
                st["master"], st["exp_avg"], st["exp_avg_sq"], g[sl], t, **HP)
        zm.zero_gather_params(plan, d_shards, d_tensors)
        want = oracle.gather_params(ref, shards)
        torch.cuda.synchronize()
        assert_bits_equal(host_u16(d_grad), g, f"generated grad step {t}")
        for i, (a, b) in enumerate(zip(d_tensors, want)):
            assert_bits_equal(host_u16(a), b, f"step {t} tensor {i}")
    full = {k: np.concatenate([s[k] for s in states]) for k in ("master", "exp_avg", "exp_avg_sq")}
    for got, key in ((d_master, "master"), (d_m, "exp_avg"), (d_v, "exp_avg_sq")):
        exact = assert_f32_close(host_f32(got), full[key], f"{name} {key}")
        assert exact == 1.0, f"{key}: {exact:.6f} bit-identical"
    assert (host_f32(d_master)[phi:] == 0).all(), "padding must stay zero"


def _gpt2_rank_steps(zm, w, S, lo, phi, steps, chunks, scales=None):
    """Rank 7's steps on the GPU: every rank's squared norm of the generated
    gradient, the clip coefficient, AdamW. After each step the fp32 state and
    the bf16 parameters are copied back and digested chunk by chunk. With
    `scales`, each step's coefficient is overwritten with the given one before
    AdamW (the update then sees the oracle's coefficient)."""
    from oracle_workers import digest
    d_grad = torch.empty(w.n_ranks * S, dtype=torch.int16, device=dev())
    d_master = torch.empty(S, dtype=torch.float32, device=dev())
    synth.device_normal_f32(d_master, w.seed, synth.KIND_MASTER, 0, 0, lo, phi, synth.MASTER_SIGMA)
    d_m = torch.zeros(S, dtype=torch.float32, device=dev())
    d_v = torch.zeros(S, dtype=torch.float32, device=dev())
    d_param = torch.zeros(S, dtype=torch.int16, device=dev())
    d_parts = torch.zeros(w.n_ranks, dtype=torch.float64, device=dev())
    d_scale = torch.zeros(1, dtype=torch.float32, device=dev())
    got_scales, got_parts, digests = [], [], []
    for t in range(1, steps + 1):
        synth.device_normal_bf16(d_grad, w.seed, synth.KIND_GRAD, t, 0, 0, phi, synth.GRAD_SIGMA)
        for r in range(w.n_ranks):
            zm.zero_grad_sqnorm(d_grad[r * S:(r + 1) * S], d_parts[r:r + 1])
        zm.zero_clip_scale(d_parts, w.max_norm, d_scale)
        got_scales.append(np.float32(d_scale.item()))
        got_parts.append(d_parts.cpu().numpy().copy())
        if scales is not None:
            d_scale.fill_(float(scales[t - 1]))
        zm.zero_shard_adamw_step(d_master, d_m, d_v, d_grad[lo:lo + S], d_param, t,
                                 clip_scale=d_scale, **HP)
        host = (host_f32(d_master), host_f32(d_m), host_f32(d_v), host_u16(d_param))
        digests.append([tuple(digest(x[a:b]) for x in host) for a, b in chunks])
    return digests, np.array(got_scales, np.float32), np.array(got_parts)


def test_gpt2_small_rank7_hundred_steps_clip(zm):
    """Full arrays, every step: rank 7's master, exp_avg, exp_avg_sq and bf16
    parameters after each of the 100 steps, against the oracle's, bit for bit
    (the oracle runs the shard in 16 windows across a process pool and returns
    per-step digests of each array)."""
    from oracle_workers import adamw_steps_digests, grad_sqnorms
    w = synth.WORKLOADS["gpt2-small"]
    ref = oracle.partition_plan(w.numels, w.n_ranks, w.align)
    P, S, phi, rank = ref.padded_numel, ref.shard_numel, ref.numel, 7
    steps = w.steps
    lo = rank * S
    cuts = [k * S // 16 for k in range(17)]
    chunks = list(zip(cuts[:-1], cuts[1:]))
    note(f"gpt2-small: P={P} S={S}, {steps} steps on the GPU, full-array digests every step")
    gpu_digests, got_scales, got_parts = _gpt2_rank_steps(zm, w, S, lo, phi, steps, chunks)

    note("gpt2-small: oracle norms over all ranks for every step (process pool)")
    tasks = [(w.seed, synth.KIND_GRAD, t, 0, r * S, S, phi, synth.GRAD_SIGMA)
             for t in range(1, steps + 1) for r in range(w.n_ranks)]
    parts = np.array(grad_sqnorms(tasks)).reshape(steps, w.n_ranks)
    assert (np.abs(got_parts - parts) <= 1e-12 * parts).all(), "per-rank norm partials"
    scales = np.array([oracle.clip_scale(list(parts[t]), w.max_norm) for t in range(steps)],
                      dtype=np.float32)
    ulps = np.abs(got_scales.view(np.int32) - scales.view(np.int32))
    assert ulps.max() <= 1, "clip coefficients"
    same = int((ulps == 0).sum())
    note(f"gpt2-small: clip coefficients {scales.min():.6f}..{scales.max():.6f}, "
         f"{same}/{steps} bit-identical")
    if same != steps:
        # The update's parity is then checked with the oracle's coefficient as its input.
        note("gpt2-small: rerunning the GPU steps with the oracle's clip coefficients")
        gpu_digests, _, _ = _gpt2_rank_steps(zm, w, S, lo, phi, steps, chunks, scales)

    note("gpt2-small: oracle AdamW over 16 windows for every step (process pool)")
    hp = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay)
    want = adamw_steps_digests([(w.seed, lo + a, b - a, phi, [float(x) for x in scales], hp)
                                for a, b in chunks])
    names = ("master", "exp_avg", "exp_avg_sq", "param")
    for t in range(steps):
        for c, (a, b) in enumerate(chunks):
            for k, name in enumerate(names):
                assert gpu_digests[t][c][k] == want[c][t][k], \
                    f"step {t + 1}: {name} differs from the oracle in [{a}, {b})"
    note(f"gpt2-small: {steps} steps x {len(chunks)} windows x 4 arrays bit-identical")


@pytest.mark.parametrize("name", ["gpt-1.3b", "gpt-1.3b-fused"])
def test_bench_all_ranks_step_matches_oracle(zm, name):
    """The benchmark's 1.3B GPT step as bench.py times it: every rank's reduce of
    its 8 replicas (no norm: the job does not clip) and AdamW, as two calls or
    in one pass, then the gather of all 292 tensors. After two steps, on 4,096-
    element windows at both ends of every rank's shard, across every boundary
    between two ranks and at one random offset per rank: the reduced gradient
    (two calls), the fp32 master, m and v and the bf16 parameters bit for bit
    against the oracle's reduce and two AdamW steps; and every gathered tensor
    equals its span of the parameter buffer."""
    import bench
    wl = bench.make_workload(name, dev())
    try:
        P, S, phi, R = wl.P, wl.S, wl.phi, wl.replicas
        hp = wl.hyper.as_kwargs()
        note(f"bench all ranks {name}: {wl.n_ranks} ranks x {S} elements, {R} replicas, 2 steps")
        steps = 2
        for _ in range(steps):
            bench.run_step(wl)
        torch.cuda.synchronize()
        n = 4096
        rng = np.random.default_rng(5)
        starts = []
        for r in range(wl.n_ranks):
            starts += [r * S, (r + 1) * S - n, r * S + int(rng.integers(0, S - n))]
            if r:
                starts.append(r * S - n // 2)
        win = oracle.partition_plan([n], 1, 1)
        for a in starts:
            reps = [synth.normal_bf16(n, wl.seed, synth.KIND_REPLICA, 1, k, a, phi, synth.GRAD_SIGMA)
                    for k in range(R)]
            g = np.zeros(n, np.uint16)
            oracle.reduce_shard(win, 0, reps, 0, g)
            p = synth.normal_f32(n, wl.seed, synth.KIND_MASTER, 0, 0, a, phi, synth.MASTER_SIGMA)
            m, v = np.zeros(n, np.float32), np.zeros(n, np.float32)
            bits = None
            for t in range(1, steps + 1):
                p, m, v, bits = oracle.adamw_step(p, m, v, g, t, clip=1.0, **hp)
            sl = slice(a, a + n)
            if not wl.fused:
                assert_bits_equal(host_u16(wl.grad[sl]), g, f"gradient at {a}")
            for got, want, what in ((wl.master, p, "master"), (wl.m, m, "m"), (wl.v, v, "v")):
                assert_bits_equal(host_f32(got[sl]).view(np.uint32), want.view(np.uint32),
                                  f"{what} at {a}")
            assert_bits_equal(host_u16(wl.param[sl]), bits, f"parameters at {a}")
        for t, dst in enumerate(wl.tensors):
            off = wl.plan.tensor_offset(t)
            assert torch.equal(dst, wl.param[off:off + dst.numel()]), f"tensor {t}"
    finally:
        del wl
        torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["gpt2-small", "gpt2-small-fsdp2", "gpt2-small-offload",
                                  "gpt2-small-fsdp2-pertensor"])
def test_bench_pipeline_matches_oracle(zm, name):
    import bench
    setup = bench.make_workload(name, dev())
    P, S, phi, rank, R = setup.P, setup.S, setup.phi, setup.rank, setup.replicas
    w = setup.workload
    shard0 = setup.layout == "shard0"
    if shard0:
        ref = oracle.partition_plan_shard0(w.numels, [s[0] for s in w.shapes], setup.n_ranks, w.align)
    else:
        ref = oracle.partition_plan(w.numels, setup.n_ranks, w.align)
    note(f"bench pipeline {name}: reduce of {R} replicas for rank {rank} of {setup.n_ranks}, S={S}")
    steps = 2
    for _ in range(steps):
        bench.run_step(setup)
    torch.cuda.synchronize()

    # oracle: every rank's reduced gradient (for the partials), then rank 7's steps
    if shard0:
        offs = bench.model_offsets(w.numels)
        reps = [oracle.flatten_params_shard0(ref, [
            synth.normal_bf16(n, setup.seed, synth.KIND_REPLICA, 1, k, off, phi, synth.GRAD_SIGMA)
            for n, off in zip(w.numels, offs)]) for k in range(R)]
    else:
        reps = [synth.normal_bf16(P, setup.seed, synth.KIND_REPLICA, 1, k, 0, phi,
                                  synth.GRAD_SIGMA) for k in range(R)]
    partials = []
    for r in range(setup.n_ranks):
        g = np.zeros(S, np.uint16)
        oracle.reduce_shard(ref, r, reps, 0, g)
        partials.append(oracle.sqnorm(g))
    master = synth.normal_f32(S, setup.seed, synth.KIND_MASTER, 0, 0, rank * S, P if shard0 else phi,
                              synth.MASTER_SIGMA)
    if shard0:
        mask = np.zeros(S, bool)
        for (_, _, soff, ln) in ref.segments(rank):
            mask[soff:soff + ln] = True
        master[~mask] = 0.0
    state = {"master": master, "exp_avg": np.zeros(S, np.float32),
             "exp_avg_sq": np.zeros(S, np.float32)}
    shards = [synth.normal_bf16(S, setup.seed, synth.KIND_PARAM, 0, 0, r * S, phi, synth.MASTER_SIGMA)
              if r != rank else np.zeros(S, np.uint16) for r in range(setup.n_ranks)]
    out = None
    for t in range(1, steps + 1):
        out = oracle.rank_step(ref, rank, reps, 0, state, shards, partials, t, setup.hyper.as_kwargs(),
                               setup.max_norm)
    assert_bits_equal(host_u16(setup.rs.grad), out["shard_grad"], "reduced shard grad")
    got_parts = setup.rs.partials.cpu().numpy()
    want_parts = np.array(out["partials"])
    own = got_parts[setup.n_ranks]
    assert abs(own - want_parts[rank]) <= 1e-12 * want_parts[rank]
    others = np.delete(np.arange(setup.n_ranks), rank)
    assert (np.abs(got_parts[others] - want_parts[others]) <= 1e-12 * want_parts[others]).all()
    got_scale = np.float32(setup.rs.scale.item())
    assert abs(int(got_scale.view(np.int32)) - int(np.float32(out["clip"]).view(np.int32))) <= 1
    # (offload: the fp32 state is in host memory; per-tensor: one array per chunk,
    # placed back at the chunk offsets with zero padding, which the oracle keeps at zero)
    if setup.per_tensor:
        assert setup.rs.master is None and all(t.is_cuda for t in setup.rs.master_tensors)
    else:
        assert setup.rs.master.is_cuda != setup.offload
    for got, key in zip(setup.state_arrays(), ("master", "exp_avg", "exp_avg_sq")):
        exact = assert_f32_close(got, state[key], key)
        note(f"bench pipeline {name}: {key} bit-identical fraction {exact:.6f}")
    if shard0:
        assert (setup.state_arrays()[0][~mask] == 0).all(), "padding stays zero"
    for i, (a, b) in enumerate(zip(setup.rs.tensors, out["tensors"])):
        assert_bf16_close(host_u16(a), b, f"gathered tensor {i}")


def test_rank_step_fresh_replica_buffers_are_not_retained(zm):
    """A caller that hands RankStep new gradient buffers every step (as a fresh
    allocation per backward pass would) gets correct reduces, and the step keeps
    one marshalled call per window: earlier buffers are released."""
    import gc
    import weakref

    from zero_partitioned_mixed_partition_amd.step import Hyper, RankStep
    numels = [1000, 37, 4096, 3]
    plan = zm.zero_partition_plan(numels, 4, 128)
    ref = oracle.partition_plan(numels, 4, 128)
    P = ref.padded_numel
    rs = RankStep(plan, 2, 1, Hyper(), 1.0, dev(), gather=False)
    held = []
    for k in range(4):
        reps_h = [synth.normal_bf16(P, 30 + k, synth.KIND_REPLICA, 1, j, 0, ref.numel, 0.05)
                  for j in range(3)]
        reps = [to_dev_u16(r) for r in reps_h]
        held.append(weakref.ref(reps[0]))
        rs.reduce([(0, P, reps)])
        torch.cuda.synchronize()
        want = np.zeros(ref.shard_numel, np.uint16)
        oracle.reduce_shard(ref, 2, reps_h, 0, want)
        assert_bits_equal(host_u16(rs.grad), want, f"reduce call {k}")
        del reps
    gc.collect()
    assert len(rs._calls) == 1
    assert all(r() is None for r in held[:-1]), "earlier replica buffers are still referenced"


def test_rank_step_skipped_step_counts_as_an_iteration(zm):
    """A non-finite global norm (here a remote rank's partial is NaN) makes the
    clip coefficient NaN and the AdamW kernel skip the update: master, m, v and
    the bf16 shard stay as they were. RankStep's step counter counts issued
    iterations, skipped ones included, so the next step's bias correction uses
    t = 2; the oracle's rank step, run with the same inputs and step numbers,
    must match after both steps."""
    from zero_partitioned_mixed_partition_amd.step import Hyper, RankStep
    numels = [1000, 37, 4096, 3]
    n_ranks, rank, R = 4, 1, 3
    plan = zm.zero_partition_plan(numels, n_ranks, 128)
    ref = oracle.partition_plan(numels, n_ranks, 128)
    P, S, phi = ref.padded_numel, ref.shard_numel, ref.numel
    hyper = Hyper()
    rs = RankStep(plan, rank, 1, hyper, 1.0, dev(), gather=True)
    master = synth.normal_f32(S, 41, synth.KIND_MASTER, 0, 0, rank * S, phi, 0.02)
    rs.master.copy_(torch.from_numpy(master))
    shards = [synth.normal_bf16(S, 41, synth.KIND_PARAM, 0, 0, r * S, phi, 0.02) for r in range(n_ranks)]
    for r in range(n_ranks):
        if r != rank:
            rs.param_shards[r].copy_(to_dev_u16(shards[r]))
    shards[rank] = np.zeros(S, np.uint16)
    state = {"master": master.copy(), "exp_avg": np.zeros(S, np.float32),
             "exp_avg_sq": np.zeros(S, np.float32)}
    for t, remote in ((1, [0.4, 0.0, float("nan"), 0.3]), (2, [0.4, 0.0, 0.2, 0.3])):
        reps_h = [synth.normal_bf16(P, 42, synth.KIND_REPLICA, t, k, 0, phi, 0.05) for k in range(R)]
        rs.set_remote_partials(remote)
        rs.step([(0, P, [to_dev_u16(x) for x in reps_h])])
        want = oracle.rank_step(ref, rank, reps_h, 0, state, shards, remote, t, hyper.as_kwargs(), 1.0)
        torch.cuda.synchronize()
        assert rs.t == t
        if t == 1:
            assert np.isnan(want["clip"]) and np.isnan(rs.scale.item()), "the step is skipped"
            assert_bits_equal(host_f32(rs.master).view(np.uint32), master.view(np.uint32),
                              "skipped step: master untouched")
            assert not host_u16(rs.param_shards[rank]).any(), "skipped step: shard untouched"
        # (the device sums the partials in another order than the oracle, so the
        # coefficient may differ in its last bit: the bars, not bit identity)
        for got, key in ((rs.master, "master"), (rs.exp_avg, "exp_avg"), (rs.exp_avg_sq, "exp_avg_sq")):
            assert_f32_close(host_f32(got), state[key], f"step {t} {key}")
        assert_bf16_close(host_u16(rs.param_shards[rank]), shards[rank], f"step {t} shard")
        for i, (a, b) in enumerate(zip(rs.tensors, want["tensors"])):
            assert_bf16_close(host_u16(a), b, f"step {t} tensor {i}")


@pytest.mark.parametrize("fuse,R", [(True, 5), (False, 5), (True, 9)],
                         ids=["one-pass", "two-calls", "nine-replicas-two-calls"])
def test_rank_step_without_clip_over_bucket_windows(zm, fuse, R):
    """RankStep without clipping over three disjoint bucket windows of R
    replicas, 3 steps, with the gather: the one-pass path (reduce_update, one
    zero_reduce_adamw_step per window) and the reduce/AdamW calls must both give
    the oracle's rank step bit for bit (no clip, so nothing depends on the
    order of the norm partials). Windows of more than 8 replicas keep the two
    calls even when fusing is on."""
    from zero_partitioned_mixed_partition_amd.step import Hyper, RankStep, rank_step_plan_windows
    numels = [1000, 37, 4096, 3, 777]
    n_ranks, rank, bucket = 4, 2, 700
    fused = fuse and R <= RankStep.FUSE_MAX_REPLICAS
    plan = zm.zero_partition_plan(numels, n_ranks, 128)
    ref = oracle.partition_plan(numels, n_ranks, 128)
    P, S, phi = ref.padded_numel, ref.shard_numel, ref.numel
    wins = rank_step_plan_windows(plan, rank, bucket)
    assert len(wins) == 3
    hyper = Hyper()
    rs = RankStep(plan, rank, len(wins), hyper, 0.0, dev(), gather=True, fuse=fuse)
    master = synth.normal_f32(S, 51, synth.KIND_MASTER, 0, 0, rank * S, phi, 0.02)
    rs.master.copy_(torch.from_numpy(master))
    shards = [synth.normal_bf16(S, 51, synth.KIND_PARAM, 0, 0, r * S, phi, 0.02) for r in range(n_ranks)]
    for r in range(n_ranks):
        if r != rank:
            rs.param_shards[r].copy_(to_dev_u16(shards[r]))
    shards[rank] = np.zeros(S, np.uint16)
    state = {"master": master.copy(), "exp_avg": np.zeros(S, np.float32),
             "exp_avg_sq": np.zeros(S, np.float32)}
    grad_before = host_u16(rs.grad).copy()
    for t in (1, 2, 3):
        full = [synth.normal_bf16(P, 52, synth.KIND_REPLICA, t, k, 0, phi, 0.05) for k in range(R)]
        rs.step([(b, c, [to_dev_u16(x[b:b + c]) for x in full]) for b, c in wins])
        want = oracle.rank_step(ref, rank, full, 0, state, shards, [0.0] * n_ranks, t,
                                hyper.as_kwargs(), 0.0)
        torch.cuda.synchronize()
        assert want["clip"] == 1.0
        for got, key in ((rs.master, "master"), (rs.exp_avg, "exp_avg"), (rs.exp_avg_sq, "exp_avg_sq")):
            assert_bits_equal(host_f32(got).view(np.uint32), state[key].view(np.uint32),
                              f"step {t} {key}")
        assert_bits_equal(host_u16(rs.param_shards[rank]), shards[rank], f"step {t} shard")
        for i, (a, b) in enumerate(zip(rs.tensors, want["tensors"])):
            assert_bits_equal(host_u16(a), b, f"step {t} tensor {i}")
        if fused:
            assert_bits_equal(host_u16(rs.grad), grad_before, "the one-pass step stores no gradient")
        else:
            assert_bits_equal(host_u16(rs.grad), want["shard_grad"], f"step {t} gradient")
    assert rs.t == 3
    assert sorted(k[0] if isinstance(k, tuple) else k for k in rs._calls) == (
        ["gather"] + ["reduce_update"] * 3 if fused else ["adamw", "gather"] + ["reduce"] * 3)


@pytest.mark.parametrize("layout", ["flat", "shard0"])
def test_rank_step_reduce_from_per_tensor_replicas(zm, layout):
    """RankStep.reduce_tensors (a zero_reduce_table over per-tensor replicas),
    then clip and AdamW, two steps with new values in the same buffers: the
    oracle's rank step over the flattened replicas, bit for bit except the
    clip coefficient's last bit (the partials' order)."""
    from zero_partitioned_mixed_partition_amd.step import Hyper, RankStep
    numels = [1000 * 16, 37 * 16, 4096, 3 * 16, 777 * 16]
    dim0 = [1000, 37, 4096, 3, 777]
    n_ranks, rank, R = 4, 2, 3
    if layout == "flat":
        plan = zm.zero_partition_plan(numels, n_ranks, 128)
        ref = oracle.partition_plan(numels, n_ranks, 128)
        flatten = oracle.flatten_params
    else:
        plan = zm.zero_partition_plan_shard0(numels, dim0, n_ranks, 128)
        ref = oracle.partition_plan_shard0(numels, dim0, n_ranks, 128)
        flatten = oracle.flatten_params_shard0
    S = ref.shard_numel
    hyper = Hyper()
    rs = RankStep(plan, rank, 1, hyper, 1.0, dev(), gather=True)
    rng = np.random.default_rng(61)
    master = np.zeros(S, np.float32)
    covered = np.zeros(S, bool)
    for (_, _, soff, ln) in ref.segments(rank):
        covered[soff:soff + ln] = True
    master[covered] = (rng.standard_normal(int(covered.sum())) * 0.02).astype(np.float32)
    rs.master.copy_(torch.from_numpy(master))
    shards = [oracle.f32_to_bf16((rng.standard_normal(S) * 0.02).astype(np.float32)) for _ in range(n_ranks)]
    for r in range(n_ranks):
        if r != rank:
            rs.param_shards[r].copy_(to_dev_u16(shards[r]))
    shards[rank] = np.zeros(S, np.uint16)
    state = {"master": master.copy(), "exp_avg": np.zeros(S, np.float32),
             "exp_avg_sq": np.zeros(S, np.float32)}
    d_reps = [[torch.empty(n, dtype=torch.int16, device=dev()) for n in numels] for _ in range(R)]
    remote = [0.4, 0.0, 0.0, 0.3]
    for t in (1, 2):
        reps_h = [[oracle.f32_to_bf16((rng.standard_normal(n) * 0.05).astype(np.float32)) for n in numels]
                  for _ in range(R)]
        for dr, hr in zip(d_reps, reps_h):
            for d, h in zip(dr, hr):
                d.copy_(to_dev_u16(h))
        rs.set_remote_partials(remote)
        rs.reduce_tensors(d_reps)
        rs.clip()
        rs.adamw()
        rs.gather()
        flats = [flatten(ref, rep) for rep in reps_h]
        want = oracle.rank_step(ref, rank, flats, 0, state, shards, remote, t, hyper.as_kwargs(), 1.0)
        torch.cuda.synchronize()
        assert_bits_equal(host_u16(rs.grad), want["shard_grad"], f"step {t} gradient")
        got_part = float(rs.partials[n_ranks].item())
        assert abs(got_part - want["partials"][rank]) <= 1e-12 * want["partials"][rank]
        for got, key in ((rs.master, "master"), (rs.exp_avg, "exp_avg"), (rs.exp_avg_sq, "exp_avg_sq")):
            assert_f32_close(host_f32(got), state[key], f"step {t} {key}")
        assert_bf16_close(host_u16(rs.param_shards[rank]), shards[rank], f"step {t} shard")
        for i, (a, b) in enumerate(zip(rs.tensors, want["tensors"])):
            assert_bf16_close(host_u16(a), b, f"step {t} tensor {i}")
    assert list(rs._calls).count("reduce_tensors") == 1



def test_rank_step_per_parameter_state_matches_flat_state(zm):
    """RankStep(per_param=True), FSDP-2's optimizer layout (fp32 state per
    parameter chunk, the multi-tensor AdamW through its table), against the
    flat-state RankStep on the same Shard(0) plan and inputs, three clipped
    steps: every chunk's master, m and v equal the flat state's slice bit for
    bit, and so do the parameter shard and the gathered tensors; the flat
    step itself is the oracle's (checked on the last step)."""
    from zero_partitioned_mixed_partition_amd.step import Hyper, RankStep
    numels = [1000 * 16, 37 * 16, 4096, 3 * 16, 777 * 16]
    dim0 = [1000, 37, 4096, 3, 777]
    n_ranks, rank, R = 4, 1, 3
    plan = zm.zero_partition_plan_shard0(numels, dim0, n_ranks, 128)
    ref = oracle.partition_plan_shard0(numels, dim0, n_ranks, 128)
    P, S = ref.padded_numel, ref.shard_numel
    hyper = Hyper()
    flat = RankStep(plan, rank, 1, hyper, 1.0, dev(), gather=True)
    pp = RankStep(plan, rank, 1, hyper, 1.0, dev(), gather=True, per_param=True)
    rng = np.random.default_rng(71)
    segs = ref.segments(rank)
    master = np.zeros(S, np.float32)
    for (_, _, soff, ln) in segs:
        master[soff:soff + ln] = (rng.standard_normal(ln) * 0.02).astype(np.float32)
    flat.master.copy_(torch.from_numpy(master))
    for t, (_, _, soff, ln) in zip(pp.master_tensors, segs):
        t.copy_(torch.from_numpy(master[soff:soff + ln]))
    shards = [oracle.f32_to_bf16((rng.standard_normal(S) * 0.02).astype(np.float32)) for _ in range(n_ranks)]
    for r in range(n_ranks):
        if r != rank:
            flat.param_shards[r].copy_(to_dev_u16(shards[r]))
            pp.param_shards[r].copy_(to_dev_u16(shards[r]))
    shards[rank] = np.zeros(S, np.uint16)
    state = {"master": master.copy(), "exp_avg": np.zeros(S, np.float32),
             "exp_avg_sq": np.zeros(S, np.float32)}
    remote = [0.4, 0.0, 0.2, 0.3]
    for t in (1, 2, 3):
        reps_h = [synth.normal_bf16(P, 72, synth.KIND_REPLICA, t, k, 0, ref.numel, 0.05) for k in range(R)]
        reps = [to_dev_u16(x) for x in reps_h]
        for rs in (flat, pp):
            rs.set_remote_partials(remote)
            rs.step([(0, P, reps)])
        want = oracle.rank_step(ref, rank, reps_h, 0, state, shards, remote, t, hyper.as_kwargs(), 1.0)
    torch.cuda.synchronize()
    for name, flat_arr, tensors in (("master", flat.master, pp.master_tensors),
                                    ("exp_avg", flat.exp_avg, pp.exp_avg_tensors),
                                    ("exp_avg_sq", flat.exp_avg_sq, pp.exp_avg_sq_tensors)):
        fa = host_f32(flat_arr)
        for i, (x, (_, _, soff, ln)) in enumerate(zip(tensors, segs)):
            assert_bits_equal(host_f32(x).view(np.uint32), fa[soff:soff + ln].view(np.uint32),
                              f"{name} of chunk {i}")
        assert_f32_close(fa, state[name], f"flat {name} against the oracle")
    assert_bits_equal(host_u16(pp.param_shards[rank]), host_u16(flat.param_shards[rank]), "parameter shard")
    for i, (a, b) in enumerate(zip(pp.tensors, flat.tensors)):
        assert_bits_equal(host_u16(a), host_u16(b), f"tensor {i}")
    for i, (a, b) in enumerate(zip(flat.tensors, want["tensors"])):
        assert_bf16_close(host_u16(a), b, f"tensor {i} against the oracle")
