"""GPU parity on the large model-shaped workloads at their full sizes.

llama3-8b   Llama-3-8B tensor list, N_d = 64, rank 63 (125,472,896 elements):
            the shard's gradient arrives as six 25M-element flat-index buckets,
            each as 64 replica buffers, reduced into the shard in backward
            (descending) order; global-norm clip 1.0; one AdamW step. Full
            arrays against the oracle (the oracle reduces the shard in chunks
            across a process pool).
gpt-1.3b    1.3B GPT list, N_d = 8: 8 replicas reduced for every rank, AdamW on
            every shard, gather to 292 tensors. Full arrays against the oracle
            (per-window digests from a process pool), exact norm partials of
            every rank, and a full-size gather of synthetic shards.
llama3-70b  Llama-3-70B list, N_d = 8, rank 7 (8,819,213,312 elements, indices
            past 2^33): step 1 as the benchmark runs it (every rank's norm
            partial and the clip-1.0 coefficient on the device, then AdamW),
            all eight partials and the coefficient against the oracle's; four
            more steps with the oracle's coefficient; windows at the shard ends,
            around 2^31, 2^32 and 2^33 and the AdamW grid's rows, at tensor
            starts and 32 random 1M windows.
past 2^32   the one-pass reduce and AdamW over a 4,299,161,984-element shard
            (two rows of workgroups), on windows around 2^31, 2^32, the row
            boundary and the padding; the reduce table over a 4,296,020,096-
            element shard from per-tensor replicas (windows, and the whole
            squared norm against the oracle's reduce of every window).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import (assert_bf16_close, assert_bits_equal, assert_f32_close, dev, host_f32,
                      host_u16, needs_gpu, note)

pytestmark = [pytest.mark.gpu, needs_gpu]

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


@pytest.fixture(scope="module")
def zm():
    import zero_partitioned_mixed_partition_amd as m
    torch.cuda.set_device(0)
    return m


def _free_gpu():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_llama3_8b_rank63_buckets_clip_one_step(zm):
    from oracle_workers import grad_sqnorms, reduce_windows
    from zero_partitioned_mixed_partition_amd.step import Hyper, RankStep, bucket_windows
    w = synth.WORKLOADS["llama3-8b"]
    rank, R = 63, w.replicas
    plan = zm.zero_partition_plan(w.numels, w.n_ranks, w.align)
    P, S, phi = plan.padded_numel, plan.shard_numel, plan.numel
    lo = rank * S
    # the other ranks reduce on their own GPUs; their averaged gradients are drawn
    # directly, with the standard deviation of a mean of R replicas
    sigma_avg = synth.GRAD_SIGMA / math.sqrt(R)
    wins = bucket_windows(P, w.bucket, lo, lo + S)
    note(f"llama3-8b: P={P} S={S}, windows {wins}")
    assert len(wins) == 6 and wins[0] == (8_025_000_000, 5_265_344)
    rs = RankStep(plan, rank, len(wins), Hyper(), w.max_norm, dev(), gather=False)
    synth.device_normal_f32(rs.master, w.seed, synth.KIND_MASTER, 0, 0, lo, phi, synth.MASTER_SIGMA)
    scratch = torch.empty(S, dtype=torch.int16, device=dev())
    for r in range(w.n_ranks):
        if r != rank:
            synth.device_normal_bf16(scratch, w.seed, synth.KIND_GRAD, 1, 0, r * S, phi, sigma_avg)
            zm.zero_grad_sqnorm(scratch, rs.partials[r:r + 1], workspace=rs.workspace)
    del scratch
    reps = [torch.empty(w.bucket, dtype=torch.int16, device=dev()) for _ in range(R)]
    for wi, (b0, cnt) in enumerate(wins):
        for k in range(R):
            synth.device_normal_bf16(reps[k], w.seed, synth.KIND_REPLICA, 1, k, b0, phi,
                                     synth.GRAD_SIGMA, n=cnt)
        zm.zero_grad_reduce_shard(plan, rank, [x[:cnt] for x in reps], b0, cnt, rs.grad,
                                  sqnorm_out=rs.partials[w.n_ranks + wi:w.n_ranks + wi + 1],
                                  workspace=rs.workspace)
    rs.clip()
    rs.adamw()
    torch.cuda.synchronize()
    del reps
    got_parts = rs.partials.cpu().numpy()
    got_scale = np.float32(rs.scale.item())

    note("llama3-8b: oracle remote partials and the own shard's reduce (process pool)")
    remote = grad_sqnorms([(w.seed, synth.KIND_GRAD, 1, 0, r * S, S, phi, sigma_avg)
                           for r in range(w.n_ranks) if r != rank])
    chunk = 1 << 22
    tasks = [(w.numels, w.n_ranks, w.align, rank, w.seed, synth.KIND_REPLICA, 1, R, a,
              min(a + chunk, lo + S), synth.GRAD_SIGMA) for a in range(lo, lo + S, chunk)]
    res = reduce_windows(tasks)
    grad = np.concatenate([b for b, _ in res])
    acc = oracle.SqnormAccumulator()
    for _, a in res:
        acc.merge(a)
    own = acc.value()
    parts = remote[:rank] + [own]
    scale = oracle.clip_scale(parts, w.max_norm)
    note(f"llama3-8b: global norm {math.sqrt(sum(parts)):.4f}, clip {scale:.6f}")

    assert_bits_equal(host_u16(rs.grad), grad, "reduced shard gradient")
    others = np.array([i for i in range(w.n_ranks) if i != rank])
    assert (np.abs(got_parts[others] - np.array(remote)) <= 1e-12 * np.array(remote)).all()
    own_gpu = float(got_parts[w.n_ranks:].sum())
    assert abs(own_gpu - own) <= 1e-12 * own, (own_gpu, own)
    assert abs(int(got_scale.view(np.int32)) - int(np.float32(scale).view(np.int32))) <= 1
    master = synth.normal_f32(S, w.seed, synth.KIND_MASTER, 0, 0, lo, phi, synth.MASTER_SIGMA)
    z = np.zeros(S, np.float32)
    p, m, v, bits = oracle.adamw_step(master, z, z, grad, 1, clip=scale, **HP)
    for got, want, what in ((rs.master, p, "master"), (rs.exp_avg, m, "exp_avg"),
                            (rs.exp_avg_sq, v, "exp_avg_sq")):
        exact = assert_f32_close(host_f32(got), want, what)
        note(f"llama3-8b: {what} bit-identical fraction {exact:.6f}")
    assert_bf16_close(host_u16(rs.param_shards[rank]), bits, "param shard")
    del rs
    _free_gpu()


def _windows_in_shards(points, half, S, n_ranks, total):
    """Windows [c-half, c+half) around each point, clipped to [0, total) and split
    at shard boundaries, merged when they overlap."""
    spans = sorted((max(0, c - half), min(total, c + half)) for c in points)
    merged = []
    for a, b in spans:
        if merged and a <= merged[-1][1]:
            merged[-1] = (merged[-1][0], max(merged[-1][1], b))
        else:
            merged.append((a, b))
    out = []
    for a, b in merged:
        while a < b:
            end = min(b, (a // S + 1) * S)
            out.append((a, end))
            a = end
    return [(a, b) for a, b in out if b > a]


@pytest.mark.parametrize("way", ["two-calls", "one-pass"])
def test_gpt_1p3b_all_ranks_reduce_adamw_gather(zm, way):
    """Full arrays: every rank's reduced gradient, fp32 state and bf16 parameters
    against the oracle, bit for bit (the oracle runs 2^23-element windows across
    a process pool and returns digests of each array), every rank's exact
    squared-norm partial, and the gathered tensors against the parameters. The
    step runs as the reduce (one-pass kernel, fused norm) then AdamW, or as the
    one-pass reduce-and-update (zero_reduce_adamw_step, writing the gradient too;
    the norm then by zero_grad_sqnorm on it): the configuration has no clip."""
    from oracle_workers import digest, reduce_adamw_digests
    w = synth.WORKLOADS["gpt-1.3b"]
    R = w.replicas
    ref = oracle.partition_plan(w.numels, w.n_ranks, w.align)
    plan = zm.zero_partition_plan(w.numels, w.n_ranks, w.align)
    P, S, phi = ref.padded_numel, ref.shard_numel, ref.numel
    note(f"gpt-1.3b ({way}): P={P} S={S} T={len(w.numels)}, {R} replicas")
    reps = []
    for k in range(R):
        t = torch.empty(P, dtype=torch.int16, device=dev())
        synth.device_normal_bf16(t, w.seed, synth.KIND_REPLICA, 1, k, 0, phi, synth.GRAD_SIGMA)
        reps.append(t)
    master = torch.empty(P, dtype=torch.float32, device=dev())
    synth.device_normal_f32(master, w.seed, synth.KIND_MASTER, 0, 0, 0, phi, synth.MASTER_SIGMA)
    m = torch.zeros(P, dtype=torch.float32, device=dev())
    v = torch.zeros(P, dtype=torch.float32, device=dev())
    grad = torch.empty(P, dtype=torch.int16, device=dev())
    param = torch.empty(P, dtype=torch.int16, device=dev())
    parts = torch.zeros(w.n_ranks, dtype=torch.float64, device=dev())
    ws = zm.reduce_workspace(S, dev())       # the benchmark's path: the one-pass reduce
    for r in range(w.n_ranks):
        sl = slice(r * S, (r + 1) * S)
        if way == "two-calls":
            zm.zero_grad_reduce_shard(plan, r, reps, 0, P, grad[sl], sqnorm_out=parts[r:r + 1],
                                      workspace=ws)
            zm.zero_shard_adamw_step(master[sl], m[sl], v[sl], grad[sl], param[sl], 1, **HP)
        else:
            zm.zero_reduce_adamw_step(plan, r, reps, 0, P, master[sl], m[sl], v[sl], param[sl], 1,
                                      shard_grad=grad[sl], **HP)
            zm.zero_grad_sqnorm(grad[sl], parts[r:r + 1], workspace=ws)
    tensors = [torch.empty(n, dtype=torch.int16, device=dev()) for n in w.numels]
    zm.zero_gather_params(plan, [param[r * S:(r + 1) * S] for r in range(w.n_ranks)], tensors)
    torch.cuda.synchronize()
    del reps
    _free_gpu()

    # the gather: every tensor is its slice of the flat parameter buffer
    for t, (off, n) in enumerate(zip(ref.offsets, w.numels)):
        assert torch.equal(tensors[t], param[off:off + n]), f"gathered tensor {t}"
    chunk = 1 << 23
    wins = [(a, min(a + chunk, (r + 1) * S)) for r in range(w.n_ranks)
            for a in range(r * S, (r + 1) * S, chunk)]
    note(f"gpt-1.3b: oracle reduce + AdamW over all {P} elements in {len(wins)} windows "
         "(process pool), compared by digest")
    tasks = [(w.numels, w.n_ranks, w.align, a // S, w.seed, R, a, b, HP) for a, b in wins]
    accs = [oracle.SqnormAccumulator() for _ in range(w.n_ranks)]
    names = ("grad", "master", "exp_avg", "exp_avg_sq", "param")
    for (a, b), (want, acc) in zip(wins, reduce_adamw_digests(tasks, workers=16)):
        got = (host_u16(grad[a:b]), host_f32(master[a:b]), host_f32(m[a:b]), host_f32(v[a:b]),
               host_u16(param[a:b]))
        for name, x, d in zip(names, got, want):
            assert digest(x) == d, f"{name} differs from the oracle in [{a}, {b})"
        accs[a // S].merge(acc)
    for r in range(w.n_ranks):
        got, want = float(parts[r].item()), accs[r].value()
        assert abs(got - want) <= 1e-12 * want, (r, got, want)
    note(f"gpt-1.3b: {P} elements x 5 arrays bit-identical, {w.n_ranks} norm partials within 1e-12")
    del master, m, v, grad, param, tensors
    _free_gpu()


def test_gpt_1p3b_full_size_gather_of_synthetic_shards(zm):
    w = synth.WORKLOADS["gpt-1.3b"]
    ref = oracle.partition_plan(w.numels, w.n_ranks, w.align)
    plan = zm.zero_partition_plan(w.numels, w.n_ranks, w.align)
    S = ref.shard_numel
    shards = []
    for r in range(w.n_ranks):
        t = torch.empty(S, dtype=torch.int16, device=dev())
        synth.device_normal_bf16(t, w.seed, synth.KIND_PARAM, 0, 0, r * S, ref.numel, 0.02)
        shards.append(t)
    tensors = [torch.empty(n, dtype=torch.int16, device=dev()) for n in w.numels]
    zm.zero_gather_params(plan, shards, tensors)
    # the same gather through a device-resident copy table
    t_tensors = [torch.full((n,), 0x3333, dtype=torch.int16, device=dev()) for n in w.numels]
    table = zm.CopyTable.gather(plan, shards, t_tensors)
    table.run()
    torch.cuda.synchronize()
    note(f"gpt-1.3b gather: {ref.numel} parameters, {len(w.numels)} tensors, "
         f"copy table {table.blocks} workgroups")
    host_shards = [synth.normal_bf16(S, w.seed, synth.KIND_PARAM, 0, 0, r * S, ref.numel, 0.02)
                   for r in range(w.n_ranks)]
    want = oracle.gather_params(ref, host_shards)
    for i, (a, t, b) in enumerate(zip(tensors, t_tensors, want)):
        assert_bits_equal(host_u16(a), b, f"tensor {i}")
        assert_bits_equal(host_u16(t), b, f"copy table, tensor {i}")
    del shards, tensors, t_tensors, table
    _free_gpu()


def test_llama3_70b_rank7_five_steps_windows(zm):
    """The benchmark's Llama-3-70B configuration: rank 7 of 8 (S > 2^33), five
    AdamW steps. Step 1 runs the benchmark's pipeline: every rank's norm partial
    and the clip-1.0 coefficient on the device, then AdamW with that device
    coefficient; all eight partials are checked against the oracle's exact sums
    of the generated gradients, and the coefficient against the oracle's clip of
    those. Steps 2-5 take the oracle's step-1 coefficient, uploaded (the oracle's
    exact norms of all ranks for five steps would take minutes on the host). The
    fp32 state and bf16 parameters are checked after the five steps on windows at
    the shard ends, around 2^31, 2^32, 2^33, around the rows of the AdamW
    dispatch's grid, at tensor starts and 32 random 1M windows."""
    from oracle_workers import grad_sqnorms
    from zero_partitioned_mixed_partition_amd.step import Hyper, RankStep
    w = synth.WORKLOADS["llama3-70b"]
    rank = 7
    ref = oracle.partition_plan(w.numels, w.n_ranks, w.align)
    plan = zm.zero_partition_plan(w.numels, w.n_ranks, w.align)
    P, S, phi = ref.padded_numel, ref.shard_numel, ref.numel
    lo = rank * S
    assert S > 2 ** 33
    steps = w.steps
    note(f"llama3-70b: S={S} (fp32 state {12 * S / 1e9:.1f} GB); oracle norms of all "
         f"{w.n_ranks} ranks for step 1 (process pool)")
    chunk = 1 << 28
    tasks = [(w.seed, synth.KIND_GRAD, 1, 0, r * S + a, min(chunk, S - a), phi, synth.GRAD_SIGMA)
             for r in range(w.n_ranks) for a in range(0, S, chunk)]
    vals = grad_sqnorms(tasks, workers=16)
    per = len(tasks) // w.n_ranks
    # chunk values are correctly rounded, so their fp64 sum is within a few ulp
    want_parts = [math.fsum(vals[r * per:(r + 1) * per]) for r in range(w.n_ranks)]
    coef1 = np.float32(oracle.clip_scale(want_parts, 1.0))
    assert 0.0 < coef1 < 1.0

    rs = RankStep(plan, rank, 0, Hyper(), 1.0, dev(), gather=False)
    synth.device_normal_f32(rs.master, w.seed, synth.KIND_MASTER, 0, 0, lo, phi, synth.MASTER_SIGMA)
    scratch = torch.empty(S, dtype=torch.int16, device=dev())   # the other ranks' gradients
    d_parts = torch.zeros(w.n_ranks, dtype=torch.float64, device=dev())
    for r in list(range(w.n_ranks - 1)) + [rank]:                # own rank last: rs.grad keeps it
        buf = rs.grad if r == rank else scratch
        synth.device_normal_bf16(buf, w.seed, synth.KIND_GRAD, 1, 0, r * S, phi, synth.GRAD_SIGMA)
        zm.zero_grad_sqnorm(buf, d_parts[r:r + 1], workspace=rs.workspace)
    zm.zero_clip_scale(d_parts, 1.0, rs.scale)
    rs.adamw()
    torch.cuda.synchronize()
    del scratch
    got_parts = d_parts.cpu().numpy()
    for r in range(w.n_ranks):
        assert abs(got_parts[r] - want_parts[r]) <= 1e-12 * want_parts[r], (r, got_parts[r], want_parts[r])
    got_coef = np.float32(rs.scale.item())
    assert abs(int(got_coef.view(np.int32)) - int(coef1.view(np.int32))) <= 1, (got_coef, coef1)
    note(f"llama3-70b: step 1 done, clip coefficient {got_coef} (oracle {coef1})")
    coefs = [coef1] * steps
    for t in range(2, steps + 1):
        synth.device_normal_bf16(rs.grad, w.seed, synth.KIND_GRAD, t, 0, lo, phi, synth.GRAD_SIGMA)
        rs.scale.fill_(float(coef1))
        rs.adamw()
        torch.cuda.synchronize()
        note(f"llama3-70b: step {t} done")

    rng = np.random.default_rng(70)
    seg_starts = [soff for (_, _, soff, _) in ref.segments(rank)]
    per_row = -(-(-(-S // 256)) // 3) * 256        # the AdamW grid's rows (3 rows of workgroups)
    centers = [0, S, 2 ** 31, 2 ** 32, 2 ** 33, per_row, 2 * per_row] + seg_starts[1:12]
    wins = [(a, b) for a, b in _windows_in_shards([lo + c for c in centers], 2048, S, w.n_ranks, P)
            if a >= lo and b <= lo + S]
    wins += [(lo + int(x), lo + int(x) + (1 << 20)) for x in rng.integers(0, S - (1 << 20), 32)]
    note(f"llama3-70b: {len(wins)} windows, {sum(b - a for a, b in wins)} elements")
    for a, b in wins:
        n = b - a
        p = synth.normal_f32(n, w.seed, synth.KIND_MASTER, 0, 0, a, phi, synth.MASTER_SIGMA)
        m = np.zeros(n, np.float32)
        v = np.zeros(n, np.float32)
        bits = None
        for t in range(1, steps + 1):
            g = synth.normal_bf16(n, w.seed, synth.KIND_GRAD, t, 0, a, phi, synth.GRAD_SIGMA)
            p, m, v, bits = oracle.adamw_step(p, m, v, g, t, clip=coefs[t - 1], **HP)
        i0, i1 = a - lo, b - lo
        assert_f32_close(host_f32(rs.master[i0:i1]), p, f"master [{i0},{i1})")
        assert_f32_close(host_f32(rs.exp_avg[i0:i1]), m, f"exp_avg [{i0},{i1})")
        assert_f32_close(host_f32(rs.exp_avg_sq[i0:i1]), v, f"exp_avg_sq [{i0},{i1})")
        assert_bf16_close(host_u16(rs.param_shards[rank][i0:i1]), bits, f"param [{i0},{i1})")
    del rs
    _free_gpu()


def test_gpt_1p3b_full_size_flatten(zm):
    w = synth.WORKLOADS["gpt-1.3b"]
    ref = oracle.partition_plan(w.numels, w.n_ranks, w.align)
    plan = zm.zero_partition_plan(w.numels, w.n_ranks, w.align)
    tensors = []
    for n, off in zip(w.numels, ref.offsets):
        t = torch.empty(n, dtype=torch.int16, device=dev())
        synth.device_normal_bf16(t, w.seed, synth.KIND_REPLICA, 1, 3, off, ref.numel, synth.GRAD_SIGMA)
        tensors.append(t)
    flat = torch.full((ref.padded_numel,), 0x1111, dtype=torch.int16, device=dev())
    zm.zero_flatten_params(plan, tensors, flat)
    torch.cuda.synchronize()
    note(f"gpt-1.3b flatten: {ref.numel} parameters from {len(w.numels)} tensors")
    host = [synth.normal_bf16(n, w.seed, synth.KIND_REPLICA, 1, 3, off, ref.numel, synth.GRAD_SIGMA)
            for n, off in zip(w.numels, ref.offsets)]
    assert_bits_equal(host_u16(flat), oracle.flatten_params(ref, host), "flat buffer")
    del tensors, flat
    _free_gpu()


@pytest.mark.parametrize("kind", ["flat", "shard0"])
def test_pieces_longer_than_2p30_flatten_and_gather(zm, kind):
    """Segments longer than 2^30 elements are split into several kernel
    pieces, and a Shard(0) tensor of 2^31 elements or more takes the segment
    kernels instead of the tensor-major one. A full-size round trip: flatten,
    then gather, must give back every tensor bit for bit, with zero padding."""
    if kind == "flat":
        numels, dim0, n_ranks = [(1 << 30) + 4099, 3], None, 1
        plan = zm.zero_partition_plan(numels, n_ranks, 128)
    else:
        rows = (1 << 20) + 1
        numels, dim0, n_ranks = [rows * 2048, 5 * 7], [rows, 5], 2
        plan = zm.zero_partition_plan_shard0(numels, dim0, n_ranks, 128)
    note(f"long pieces ({kind}): numels={numels} P={plan.padded_numel} S={plan.shard_numel}")
    offs = [0, numels[0]]
    tensors = [torch.empty(n, dtype=torch.int16, device=dev()) for n in numels]
    for t, off in zip(tensors, offs):
        synth.device_normal_bf16(t, 95, synth.KIND_PARAM, 0, 0, off, sum(numels), 0.02)
    flat = torch.full((plan.padded_numel,), 0x1111, dtype=torch.int16, device=dev())
    zm.zero_flatten_params(plan, tensors, flat)
    S = plan.shard_numel
    back = [torch.full((n,), 0x2222, dtype=torch.int16, device=dev()) for n in numels]
    zm.zero_gather_params(plan, [flat[r * S:(r + 1) * S] for r in range(n_ranks)], back)
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(tensors, back)):
        assert torch.equal(a, b), f"tensor {i} round trip"
    # the same round trip through copy tables (pieces longer than 2^30 elements are not
    # split there: 64-bit lengths and offsets)
    flat2 = torch.full((plan.padded_numel,), 0x4444, dtype=torch.int16, device=dev())
    zm.CopyTable.flatten(plan, tensors, flat2).run()
    torch.cuda.synchronize()
    assert torch.equal(flat2, flat), "copy-table flatten"
    del flat2
    back2 = [torch.full((n,), 0x5555, dtype=torch.int16, device=dev()) for n in numels]
    zm.CopyTable.gather(plan, [flat[r * S:(r + 1) * S] for r in range(n_ranks)], back2).run()
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(tensors, back2)):
        assert torch.equal(a, b), f"tensor {i} copy-table round trip"
    del back2
    # the padding is zero and every flat element outside it holds some tensor element
    covered = torch.zeros(plan.padded_numel, dtype=torch.bool, device=dev())
    for r in range(n_ranks):
        for (t, toff, soff, ln) in plan.segments(r):
            a = r * S + soff
            assert torch.equal(flat[a:a + ln], tensors[t][toff:toff + ln]), (r, t)
            covered[a:a + ln] = True
    assert int(((flat != 0) & ~covered).sum().item()) == 0, "padding is zero"
    del tensors, back, flat, covered
    _free_gpu()


def test_shard0_flatten_waves_across_rank_buffers_past_2p31_bytes(zm):
    """The Shard(0) flatten's waves that cross a rank boundary store into two
    rank buffers S elements apart. Here S is past 2^30 elements, so those waves
    span more than 2^31 bytes: three [524294, 2056] tensors (538,974,232-element
    chunks, a multiple of 8 but not of a wave's 512 elements, so whole 16-byte
    lanes sit on both sides of the boundary) and small tensors whose chunks end
    inside waves. The whole flat buffer against oracle.flatten_params_shard0,
    then the tensor-major gather back to the tensors. [ZF] "FSDP-2: Per-Parameter
    Sharding via DTensor (fully_shard)"."""
    shapes = [(2 * 262147, 2056), (3001,), (2 * 262147, 2056), (7, 4097), (2 * 262147, 2056),
              (40001, 1234), (5,)]
    numels = [int(np.prod(s)) for s in shapes]
    dim0 = [s[0] for s in shapes]
    n_ranks = 2
    ref = oracle.partition_plan_shard0(numels, dim0, n_ranks, 128)
    plan = zm.zero_partition_plan_shard0(numels, dim0, n_ranks, 128)
    assert (plan.shard_numel, plan.padded_numel) == (ref.shard_numel, ref.padded_numel)
    S, P, phi = ref.shard_numel, ref.padded_numel, ref.numel
    assert S > 1 << 30
    note(f"shard0 flatten past 2^31-byte waves: P={P} S={S}")
    offs = np.concatenate([[0], np.cumsum(numels)[:-1]]).tolist()
    host = [synth.normal_bf16(n, 96, synth.KIND_PARAM, 0, 0, off, phi, 0.02)
            for n, off in zip(numels, offs)]
    tensors = [torch.from_numpy(h.view(np.int16)).to(dev()) for h in host]
    flat = torch.full((P,), 0x1111, dtype=torch.int16, device=dev())
    zm.zero_flatten_params(plan, tensors, flat)
    torch.cuda.synchronize()
    note("shard0 flatten past 2^31-byte waves: comparing the flat buffer with the oracle")
    want = oracle.flatten_params_shard0(ref, host)
    assert_bits_equal(host_u16(flat), want, "Shard(0) flat buffer")
    del want
    back = [torch.full((n,), 0x2222, dtype=torch.int16, device=dev()) for n in numels]
    zm.zero_gather_params(plan, [flat[r * S:(r + 1) * S] for r in range(n_ranks)], back)
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(tensors, back)):
        assert torch.equal(a, b), f"tensor {i} round trip"
    del tensors, back, flat, host
    _free_gpu()


def test_reduce_adamw_one_pass_past_2p32_elements(zm):
    """zero_reduce_adamw_step over a shard of more than 2^32 elements (one tensor
    of 2^32 + 2^22 + 333 parameters, N_d = 1, 2 replicas): the one-pass grid
    then has two rows of workgroups. Step 1 from m = v = 0, no clip, with the
    averaged gradient stored too; gradient, fp32 state and bf16 parameters
    against the oracle bit for bit on windows at both ends, around 2^31, 2^32,
    the grid's row boundary and the padding."""
    phi = 2 ** 32 + 2 ** 22 + 333
    ref = oracle.partition_plan([phi], 1, 128)
    plan = zm.zero_partition_plan([phi], 1, 128)
    P, S = ref.padded_numel, ref.shard_numel
    R, seed = 2, 77
    blocks = -(-S // 256)
    max_row = (1 << 32) // 256 - 1
    rows = -(-blocks // max_row)
    per_row = -(-blocks // rows) * 256
    assert rows == 2 and S > 2 ** 32 and P > phi
    note(f"one pass past 2^32: S={S}, {rows} rows of {per_row // 256} workgroups, R={R}")
    reps = [torch.empty(P, dtype=torch.int16, device=dev()) for _ in range(R)]
    for k, t in enumerate(reps):
        synth.device_normal_bf16(t, seed, synth.KIND_REPLICA, 1, k, 0, phi, synth.GRAD_SIGMA)
    master = torch.empty(S, dtype=torch.float32, device=dev())
    synth.device_normal_f32(master, seed, synth.KIND_MASTER, 0, 0, 0, phi, synth.MASTER_SIGMA)
    m = torch.zeros(S, dtype=torch.float32, device=dev())
    v = torch.zeros(S, dtype=torch.float32, device=dev())
    param = torch.zeros(S, dtype=torch.int16, device=dev())
    grad = torch.zeros(S, dtype=torch.int16, device=dev())
    zm.zero_reduce_adamw_step(plan, 0, reps, 0, P, master, m, v, param, 1, shard_grad=grad, **HP)
    torch.cuda.synchronize()
    del reps
    centers = [0, 2 ** 31, 2 ** 32, per_row, phi, S]
    wins = _windows_in_shards(centers, 2048, S, 1, S)
    note(f"one pass past 2^32: {len(wins)} windows, {sum(b - a for a, b in wins)} elements")
    for a, b in wins:
        n = b - a
        rh = [synth.normal_bf16(n, seed, synth.KIND_REPLICA, 1, k, a, phi, synth.GRAD_SIGMA)
              for k in range(R)]
        window_plan = oracle.partition_plan([n], 1, 1)   # the reduce is elementwise
        g = np.zeros(n, np.uint16)
        oracle.reduce_shard(window_plan, 0, rh, 0, g)
        p0 = synth.normal_f32(n, seed, synth.KIND_MASTER, 0, 0, a, phi, synth.MASTER_SIGMA)
        z = np.zeros(n, np.float32)
        p1, m1, v1, bits = oracle.adamw_step(p0, z, z, g, 1, clip=1.0, **HP)
        assert_bits_equal(host_u16(grad[a:b]), g, f"gradient [{a},{b})")
        assert_bits_equal(host_f32(master[a:b]).view(np.uint32), p1.view(np.uint32), f"master [{a},{b})")
        assert_bits_equal(host_f32(m[a:b]).view(np.uint32), m1.view(np.uint32), f"exp_avg [{a},{b})")
        assert_bits_equal(host_f32(v[a:b]).view(np.uint32), v1.view(np.uint32), f"exp_avg_sq [{a},{b})")
        assert_bits_equal(host_u16(param[a:b]), bits, f"param [{a},{b})")
    if phi < S:                                           # padding: zero gradient, state stays 0
        assert not host_u16(grad[phi:S]).any() and not host_f32(master[phi:S]).any()
    del master, m, v, param, grad
    _free_gpu()


def test_reduce_table_past_2p32_elements(zm):
    """zero_reduce_table_* over a shard of more than 2^32 elements (N_d = 1,
    one tensor of 2^32 + 2^20 + 5 parameters and a small one after it, 2
    per-tensor replicas): gradient bits on windows at both ends, around 2^31,
    2^32, the tensor boundary and the padding, and the full squared norm,
    against the oracle over the generated flat replicas."""
    big = 2 ** 32 + 2 ** 20 + 5
    numels = [big, 4099]
    ref = oracle.partition_plan(numels, 1, 128)
    plan = zm.zero_partition_plan(numels, 1, 128)
    S, phi, R, seed = ref.shard_numel, ref.numel, 2, 88
    assert S > 2 ** 32 and S > phi
    reps = []
    for k in range(R):
        rep = []
        for n, off in zip(numels, ref.offsets):
            t = torch.empty(n, dtype=torch.int16, device=dev())
            synth.device_normal_bf16(t, seed, synth.KIND_REPLICA, 1, k, off, phi, synth.GRAD_SIGMA)
            rep.append(t)
        reps.append(rep)
    grad = torch.full((S,), 0x5555, dtype=torch.int16, device=dev())
    sq = torch.zeros(1, dtype=torch.float64, device=dev())
    table = zm.ReduceTable(plan, 0, reps, grad)
    note(f"reduce table past 2^32: S={S}, {table.blocks} workgroups, R={R}")
    table.run(sqnorm_out=sq)
    torch.cuda.synchronize()
    del table, reps
    wins = _windows_in_shards([0, 2 ** 31, 2 ** 32, big, phi, S], 2048, S, 1, S)
    for a, b in wins:
        n = b - a
        flats = [synth.normal_bf16(n, seed, synth.KIND_REPLICA, 1, k, a, phi, synth.GRAD_SIGMA)
                 for k in range(R)]
        window = oracle.partition_plan([n], 1, 1)          # the reduce is elementwise
        want = np.zeros(n, np.uint16)
        oracle.reduce_shard(window, 0, flats, 0, want)
        assert_bits_equal(host_u16(grad[a:b]), want, f"gradient [{a},{b})")
    # the whole squared norm: the oracle's reduce of every window of the
    # generated replicas (process pool), its exact norm states merged in order
    from oracle_workers import reduce_window_sqnorms
    chunk = 1 << 26
    tasks = [(numels, 1, 128, 0, seed, synth.KIND_REPLICA, 1, R, a, min(a + chunk, S), synth.GRAD_SIGMA)
             for a in range(0, S, chunk)]
    note(f"reduce table past 2^32: oracle norm over {len(tasks)} windows (process pool)")
    acc = oracle.SqnormAccumulator()
    for part in reduce_window_sqnorms(tasks, workers=16):
        acc.merge(part)
    want_sq = acc.value()
    assert abs(float(sq.item()) - want_sq) <= 1e-12 * want_sq, (float(sq.item()), want_sq)
    del grad
    _free_gpu()
