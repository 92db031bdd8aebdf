"""GPU parity of each entry point against the CPU oracle, through the C ABI.

Sizes span several workgroups, a ragged tail, and unaligned (scalar-path)
pointers; edge cases cover empty inputs, single replicas, the maximum replica
count, a skipped step, and argument errors.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import (assert_bf16_close, assert_bits_equal, assert_f32_close, dev, host_f32,
                      host_u16, needs_gpu, note, to_dev_f32, to_dev_u16)

pytestmark = [pytest.mark.gpu, needs_gpu]

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


@pytest.fixture(scope="module")
def zm():
    import zero_partitioned_mixed_partition_amd as m
    torch.cuda.set_device(0)
    return m


# ----------------------------------------------------------------------------- AdamW

def _adamw_inputs(n, seed):
    p = synth.normal_f32(n, seed, synth.KIND_MASTER, 0, 0, sigma=0.02)
    m = synth.normal_f32(n, seed, 10, 0, 0, sigma=1e-4)
    v = np.abs(synth.normal_f32(n, seed, 11, 0, 0, sigma=1e-7))
    g = synth.normal_bf16(n, seed, synth.KIND_GRAD, 1, 0, sigma=1e-3)
    return p, m, v, g


@pytest.mark.parametrize("n", [1, 7, 8, 9, 4097, 256 * 8 * 37 + 5, (1 << 20) + 3])
def test_adamw_matches_oracle(zm, n):
    note(f"adamw n={n}")
    p, m, v, g = _adamw_inputs(n, 100 + n % 97)
    dp, dm, dv, dg = to_dev_f32(p), to_dev_f32(m), to_dev_f32(v), to_dev_u16(g)
    dout = torch.zeros(n, dtype=torch.int16, device=dev())
    scale = torch.tensor([0.37], dtype=torch.float32, device=dev())
    for t in (1, 2, 3):
        zm.zero_shard_adamw_step(dp, dm, dv, dg, dout, t, clip_scale=scale, **HP)
        p, m, v, bits = oracle.adamw_step(p, m, v, g, t, clip=0.37, **HP)
    torch.cuda.synchronize()
    for got, want, what in ((dp, p, "master"), (dm, m, "exp_avg"), (dv, v, "exp_avg_sq")):
        exact = assert_f32_close(host_f32(got), want, what)
        assert exact == 1.0, f"{what}: expected bit-identical fp32 ({exact:.6f})"
    assert_bits_equal(host_u16(dout), bits, "param bf16")


# Hyperparameter corners: no momentum, betas next to 1 (bias corrections of
# 1e-6), negative and large weight decay (a decay factor of 0), lr and eps of 1,
# and step counts where the bias corrections round to 1.
HP_CORNERS = {
    "betas-zero-no-decay": (dict(HP, beta1=0.0, beta2=0.0, weight_decay=0.0), (1, 2, 3)),
    "betas-near-one": (dict(HP, beta1=0.999999, beta2=0.999999), (1, 2)),
    "lr-eps-one-negative-decay": (dict(HP, lr=1.0, eps=1.0, weight_decay=-0.5), (1, 2)),
    "decay-factor-zero": (dict(HP, lr=0.01, weight_decay=100.0), (1, 2)),
    "huge-steps": (HP, (10 ** 6, 2 ** 40)),
}


@pytest.mark.parametrize("case", sorted(HP_CORNERS))
def test_adamw_hyperparameter_corners(zm, case):
    """The flat kernel and the one-pass reduce and update (one replica, whose
    average is the gradient itself) against the oracle, bit for bit, where the
    host's fp64 scalars meet their extremes."""
    hp, steps = HP_CORNERS[case]
    n = 4097
    note(f"adamw corners {case}")
    p, m, v, g = _adamw_inputs(n, 31)
    dp, dm, dv, dg = to_dev_f32(p), to_dev_f32(m), to_dev_f32(v), to_dev_u16(g)
    fp, fm, fv = to_dev_f32(p), to_dev_f32(m), to_dev_f32(v)
    dout = torch.zeros(n, dtype=torch.int16, device=dev())
    fout = torch.zeros(n, dtype=torch.int16, device=dev())
    plan = zm.zero_partition_plan([n], 1, 1)
    for t in steps:
        zm.zero_shard_adamw_step(dp, dm, dv, dg, dout, t, **hp)
        zm.zero_reduce_adamw_step(plan, 0, [dg], 0, n, fp, fm, fv, fout, t, **hp)
        p, m, v, bits = oracle.adamw_step(p, m, v, g, t, **hp)
    torch.cuda.synchronize()
    for pre, outs in (("flat", (dp, dm, dv, dout)), ("one-pass", (fp, fm, fv, fout))):
        for got, want, what in zip(outs[:3], (p, m, v), ("master", "exp_avg", "exp_avg_sq")):
            assert_bits_equal(host_f32(got).view(np.uint32), want.view(np.uint32), f"{pre} {what}")
        assert_bits_equal(host_u16(outs[3]), bits, f"{pre} param bf16")


@pytest.mark.parametrize("offset", [1, 3])
def test_adamw_unaligned_pointers_take_the_scalar_path(zm, offset):
    n = 5000
    p, m, v, g = _adamw_inputs(n + offset, 7)
    dp, dm, dv, dg = to_dev_f32(p), to_dev_f32(m), to_dev_f32(v), to_dev_u16(g)
    dout = torch.zeros(n + offset, dtype=torch.int16, device=dev())
    zm.zero_shard_adamw_step(dp[offset:], dm[offset:], dv[offset:], dg[offset:], dout[offset:], 4,
                             **HP)
    P, M, V, B = oracle.adamw_step(p[offset:], m[offset:], v[offset:], g[offset:], 4, **HP)
    torch.cuda.synchronize()
    assert_bits_equal(host_f32(dp)[offset:].view(np.uint32), P.view(np.uint32), "master")
    assert_bits_equal(host_f32(dm)[offset:].view(np.uint32), M.view(np.uint32), "exp_avg")
    assert_bits_equal(host_f32(dv)[offset:].view(np.uint32), V.view(np.uint32), "exp_avg_sq")
    assert_bits_equal(host_u16(dout)[offset:], B, "param")
    assert_bits_equal(host_f32(dp)[:offset].view(np.uint32), p[:offset].view(np.uint32), "untouched")


@pytest.mark.filterwarnings("ignore:overflow encountered:RuntimeWarning", "ignore:invalid value encountered:RuntimeWarning")
def test_adamw_special_values(zm):
    n = 64
    p = np.linspace(-3, 3, n).astype(np.float32)
    p[0], p[1], p[2] = 0.0, -0.0, 1e-40
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    g32 = np.linspace(-1e-2, 1e-2, n).astype(np.float32)
    g32[3], g32[4], g32[5], g32[6] = np.inf, -np.inf, np.nan, 0.0
    g32[7], g32[8] = 1e-38, 3e38
    g = oracle.f32_to_bf16(g32)
    dp, dm, dv, dg = to_dev_f32(p), to_dev_f32(m), to_dev_f32(v), to_dev_u16(g)
    dout = torch.zeros(n, dtype=torch.int16, device=dev())
    zm.zero_shard_adamw_step(dp, dm, dv, dg, dout, 1, **HP)
    P, M, V, B = oracle.adamw_step(p, m, v, g, 1, **HP)
    torch.cuda.synchronize()
    assert_f32_close(host_f32(dp), P, "master")
    assert_f32_close(host_f32(dm), M, "exp_avg")
    assert_f32_close(host_f32(dv), V, "exp_avg_sq")
    assert_bf16_close(host_u16(dout), B, "param")


def _bf16_rounding_cases() -> np.ndarray:
    """Every bf16 high half (2^16 patterns: both signs, zeros, subnormals,
    normals, infinities, NaNs) under the low halves that decide the rounding:
    exact (0), just above zero (1), below, at and above the tie (0x3FFF, 0x7FFF,
    0x8000, 0x8001, 0xBFFF) and the largest (0xFFFF); then 4,096 NaNs with
    random payloads of both signs."""
    hi = np.arange(1 << 16, dtype=np.uint32) << np.uint32(16)
    lows = np.array([0, 1, 0x3FFF, 0x7FFF, 0x8000, 0x8001, 0xBFFF, 0xFFFF], np.uint32)
    grid = (hi[:, None] | lows[None, :]).ravel()
    rng = np.random.default_rng(5)
    payload = rng.integers(1, 1 << 23, size=4096, dtype=np.uint32)
    sign = rng.integers(0, 2, size=4096, dtype=np.uint32) << np.uint32(31)
    nans = sign | np.uint32(0x7F800000) | payload
    return np.concatenate([grid, nans]).view(np.float32)


@pytest.mark.filterwarnings("ignore:overflow encountered:RuntimeWarning", "ignore:invalid value encountered:RuntimeWarning")
@pytest.mark.parametrize("entry", ["flat", "list", "table"])
def test_adamw_bf16_emit_every_rounding_case(zm, entry):
    """The kernels emit bf16 parameters with gfx950's packed convert. With lr = 0
    and m = v = g = 0 the update leaves the master as it is (p * 1 - 0 * 0), so the
    emitted parameter is the master rounded to bf16: compared bit for bit with the
    oracle's integer round-to-nearest-even (NaN quieted, payload's top bits and
    sign kept) on every rounding case, through each AdamW entry point. [ZF]
    "Static Memory Allocation" (16-bit parameters from fp32 masters)."""
    x = _bf16_rounding_cases()
    n = x.size
    note(f"bf16 emit ({entry}): {n} patterns")
    hp = dict(HP, lr=0.0)
    zeros = np.zeros(n, np.float32)
    P, M, V, B = oracle.adamw_step(x, zeros, zeros, np.zeros(n, np.uint16), 1, **hp)
    assert_bits_equal(B, oracle.f32_to_bf16(x), "oracle: lr = 0 emits the rounded master")
    dp, dm, dv = to_dev_f32(x), to_dev_f32(zeros), to_dev_f32(zeros)
    dg = torch.zeros(n, dtype=torch.int16, device=dev())
    dout = torch.full((n,), 0x5555, dtype=torch.int16, device=dev())
    if entry == "flat":
        zm.zero_shard_adamw_step(dp, dm, dv, dg, dout, 1, **hp)
    else:
        cuts = [0, 1, 8, 100_003, 263_000, n]          # ragged tensors, tails inside waves
        sl = [slice(a, b) for a, b in zip(cuts[:-1], cuts[1:])]
        lists = ([dp[s] for s in sl], [dm[s] for s in sl], [dv[s] for s in sl], [dg[s] for s in sl],
                 [dout[s] for s in sl])
        if entry == "list":
            zm.zero_multi_tensor_adamw_step(*lists, 1, **hp)
        else:
            zm.MultiTensorTable(*lists).step(1, **hp)
    torch.cuda.synchronize()
    assert_bits_equal(host_u16(dout), B, f"param bf16 ({entry})")
    assert_f32_close(host_f32(dp), P, f"master ({entry})")
    assert_bits_equal(host_f32(dm).view(np.uint32), M.view(np.uint32), f"exp_avg ({entry})")
    assert_bits_equal(host_f32(dv).view(np.uint32), V.view(np.uint32), f"exp_avg_sq ({entry})")


def test_adamw_nonfinite_scale_skips_and_lr0_keeps(zm):
    n = 3000
    p, m, v, g = _adamw_inputs(n, 9)
    dp, dm, dv, dg = to_dev_f32(p), to_dev_f32(m), to_dev_f32(v), to_dev_u16(g)
    dout = torch.full((n,), 77, dtype=torch.int16, device=dev())
    nan = torch.tensor([float("nan")], dtype=torch.float32, device=dev())
    zm.zero_shard_adamw_step(dp, dm, dv, dg, dout, 1, clip_scale=nan, **HP)
    torch.cuda.synchronize()
    assert_bits_equal(host_f32(dp).view(np.uint32), p.view(np.uint32), "skipped master")
    assert_bits_equal(host_f32(dv).view(np.uint32), v.view(np.uint32), "skipped v")
    assert (host_u16(dout) == 77).all()
    zm.zero_shard_adamw_step(dp, dm, dv, dg, dout, 1, **dict(HP, lr=0.0))
    torch.cuda.synchronize()
    assert_bits_equal(host_f32(dp).view(np.uint32), p.view(np.uint32), "lr=0 master")
    assert_bits_equal(host_u16(dout), oracle.f32_to_bf16(p), "lr=0 param")


def test_adamw_argument_errors(zm):
    x = torch.zeros(16, dtype=torch.float32, device=dev())
    h = torch.zeros(16, dtype=torch.int16, device=dev())
    for bad in (dict(HP, beta1=1.0), dict(HP, eps=0.0), dict(HP, lr=-1.0), dict(HP, beta2=-0.1)):
        with pytest.raises(zm.ZeroError):
            zm.zero_shard_adamw_step(x, x.clone(), x.clone(), h, h.clone(), 1, **bad)
    with pytest.raises(zm.ZeroError):
        zm.zero_shard_adamw_step(x, x.clone(), x.clone(), h, h.clone(), 0, **HP)
    with pytest.raises(zm.ZeroError):   # param_out aliasing the master weights
        zm.zero_shard_adamw_step(x, x.clone(), x.clone(), h, x.view(torch.int16)[:16], 1, **HP)
    zm.zero_shard_adamw_step(x, x, x, h, h, 1, n=0, **HP)   # empty: a no-op


# ----------------------------------------------------------------------------- reduce

@pytest.mark.parametrize("numels,n_ranks,align,rank,R,window", [
    ([1000, 37, 4096, 3], 4, 128, 2, 3, "full"),
    ([1000, 37, 4096, 3], 4, 128, 0, 1, "full"),
    ([100_000, 77_777], 8, 128, 7, 8, "full"),
    ([100_000, 77_777], 8, 128, 3, 64, "full"),
    ([100_000, 77_777], 8, 128, 5, 8, "bucket"),
    ([100_000, 77_777], 8, 128, 5, 2, "odd"),
    ([100_000, 77_777], 8, 128, 1, 8, "miss"),
    ([(1 << 20) + 13], 2, 8, 1, 5, "full"),
])
def test_reduce_matches_oracle(zm, numels, n_ranks, align, rank, R, window):
    note(f"reduce numels={numels} N_d={n_ranks} rank={rank} R={R} window={window}")
    ref = oracle.partition_plan(numels, n_ranks, align)
    plan = zm.zero_partition_plan(numels, n_ranks, align)
    P, S, phi = ref.padded_numel, ref.shard_numel, ref.numel
    begin, count = {
        "full": (0, P),
        "bucket": (rank * S - 1000, S // 3 + 1000),        # straddles the shard start
        "odd": (rank * S + 3, S - 7),                      # unaligned: scalar path
        "miss": ((rank + 2) * S, S // 2),                  # does not meet the shard
    }[window]
    reps = [synth.normal_bf16(count, 5, synth.KIND_REPLICA, 1, k, begin, phi, 1e-3) for k in range(R)]
    want = np.full(S, 0x1234, np.uint16)
    lo, hi = oracle.reduce_shard(ref, rank, reps, begin, want)
    d_out = to_dev_u16(np.full(S, 0x1234, np.uint16))
    d_sq = torch.full((1,), -1.0, dtype=torch.float64, device=dev())
    zm.zero_grad_reduce_shard(plan, rank, [to_dev_u16(r) for r in reps], begin, count, d_out,
                              sqnorm_out=d_sq)
    torch.cuda.synchronize()
    assert_bits_equal(host_u16(d_out), want, "reduced shard")
    want_sq = oracle.sqnorm(want[lo - rank * S:hi - rank * S]) if hi > lo else 0.0
    got_sq = float(d_sq.item())
    assert abs(got_sq - want_sq) <= 1e-12 * abs(want_sq), (got_sq, want_sq)


@pytest.mark.parametrize("R,n,off", [(3, 100_003, 0), (8, 100_003, 0), (64, 30_011, 0),
                                     (8, (1 << 24) + 5, 0), (5, 100_003, 1)])
def test_reduce_identical_replicas_return_the_input(zm, R, n, off):
    """A closed form, independent of the oracle: R identical bf16 replicas
    (R <= 2^16, finite values far from overflow) sum exactly in fp32 to R*x,
    and the division by R gives x back, so the averaged gradient is the
    replica itself, bit for bit, and its squared norm is the input's. Covers
    the grid-stride kernel (3, 8 and 64 replicas), the one-pass kernel (2^24 +
    5 elements, with the workspace it needs) and the scalar path (a window
    starting one element into the buffer)."""
    note(f"reduce identical replicas R={R} n={n} off={off}")
    plan = zm.zero_partition_plan([n + off], 1, 1)
    x = synth.normal_bf16(n + off, 9, synth.KIND_REPLICA, 1, 0, sigma=1.0)
    d = to_dev_u16(x)
    out = torch.full((n + off,), 0x1234, dtype=torch.int16, device=dev())
    sq = torch.zeros(1, dtype=torch.float64, device=dev())
    ws = zm.reduce_workspace(n, dev())
    zm.zero_grad_reduce_shard(plan, 0, [d[off:]] * R, off, n, out, sqnorm_out=sq, workspace=ws)
    torch.cuda.synchronize()
    got = host_u16(out)
    assert_bits_equal(got[off:], x[off:], "averaged gradient")
    assert got[:off].tolist() == [0x1234] * off, "element outside the window written"
    want = oracle.sqnorm(x[off:])
    assert abs(float(sq.item()) - want) <= 1e-12 * want


def test_reduce_argument_errors(zm):
    plan = zm.zero_partition_plan([1000], 4, 8)
    out = torch.zeros(plan.shard_numel, dtype=torch.int16, device=dev())
    rep = torch.zeros(plan.padded_numel, dtype=torch.int16, device=dev())
    with pytest.raises(zm.ZeroError):
        zm.zero_grad_reduce_shard(plan, 4, [rep], 0, plan.padded_numel, out)
    with pytest.raises(zm.ZeroError):
        zm.zero_grad_reduce_shard(plan, 0, [rep] * 65, 0, plan.padded_numel, out)
    with pytest.raises(zm.ZeroError):
        zm.zero_grad_reduce_shard(plan, 0, [rep], 10, plan.padded_numel, out)
    with pytest.raises(zm.ZeroError):   # workspace smaller than required
        zm.zero_grad_reduce_shard(plan, 0, [rep], 0, plan.padded_numel, out,
                                  sqnorm_out=torch.zeros(1, dtype=torch.float64, device=dev()),
                                  workspace=torch.zeros(8, dtype=torch.uint8, device=dev()))


# ----------------------------------------------------------------------------- sqnorm, clip

@pytest.mark.parametrize("n", [0, 1, 7, 8, 2049, (1 << 22) + 5])
def test_sqnorm_matches_oracle(zm, n):
    g = synth.normal_bf16(max(n, 1), 8, synth.KIND_GRAD, 2, 0, sigma=1e-3)[:n]
    d = to_dev_u16(g) if n else torch.zeros(1, dtype=torch.int16, device=dev())
    out = torch.full((1,), -1.0, dtype=torch.float64, device=dev())
    zm.zero_grad_sqnorm(d, out, n=n)
    torch.cuda.synchronize()
    want = oracle.sqnorm(g)
    assert abs(out.item() - want) <= 1e-12 * want, (out.item(), want)
    zm.zero_grad_sqnorm(d, out, n=n)           # repeatable bit for bit
    again = out.item()
    zm.zero_grad_sqnorm(d, out, n=n)
    torch.cuda.synchronize()
    assert again == out.item()


def test_sqnorm_constant_closed_form_and_unaligned(zm):
    c = oracle.f32_to_bf16(np.array([3.0e-3], np.float32))[0]
    cv = float(oracle.bf16_to_f32(np.array([c]))[0])
    n = 50_000_001
    d = torch.full((n + 1,), int(np.int16(np.uint16(c).view(np.int16))), dtype=torch.int16,
                   device=dev())
    out = torch.zeros(1, dtype=torch.float64, device=dev())
    zm.zero_grad_sqnorm(d[:n], out)
    torch.cuda.synchronize()
    assert out.item() == n * cv * cv
    zm.zero_grad_sqnorm(d[1:], out)          # 2-byte offset: scalar path
    torch.cuda.synchronize()
    assert out.item() == n * cv * cv


def test_norm_workspace_needs_no_initialisation(zm):
    """The workspace may hold anything before a call (here: all ones, then
    random bytes) and may be shared by calls of different grid sizes in turn;
    every result is the oracle's, and equal to a fresh workspace's."""
    nbytes = zm.zero_sqnorm_workspace_bytes()
    sizes = [(1 << 22) + 5, 2049, 9, 50_000_001, 1 << 20]
    grads = [synth.normal_bf16(n, 21, synth.KIND_GRAD, 2, 0, sigma=1e-3) for n in sizes]
    d = [to_dev_u16(g) for g in grads]
    want = [oracle.sqnorm(g) for g in grads]
    rng = np.random.default_rng(5)
    for fill in ("ones", "random"):
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev())
        if fill == "ones":
            ws.fill_(255)
        else:
            ws.copy_(torch.from_numpy(rng.integers(0, 256, nbytes, dtype=np.uint8)))
        outs = torch.full((2 * len(sizes),), -1.0, dtype=torch.float64, device=dev())
        for i, g in enumerate(d):
            zm.zero_grad_sqnorm(g, outs[i:i + 1], workspace=ws)
        for i, g in enumerate(d):            # again, in reverse: other grids before each
            j = len(sizes) - 1 - i
            zm.zero_grad_sqnorm(d[j], outs[len(sizes) + j:len(sizes) + j + 1], workspace=ws)
        torch.cuda.synchronize()
        got = outs.cpu().numpy()
        fresh = torch.zeros(len(sizes), dtype=torch.float64, device=dev())
        for i, g in enumerate(d):
            zm.zero_grad_sqnorm(g, fresh[i:i + 1])
        torch.cuda.synchronize()
        for i, w in enumerate(want):
            note(f"fill={fill} n={sizes[i]}")
            assert abs(got[i] - w) <= 1e-12 * w, (sizes[i], got[i], w)
            assert got[i] == got[len(sizes) + i] == fresh[i].item()
    # a reduce with its norm on the same workspace, between the sqnorm calls
    numels = [300_001, 17, 4096 * 1000]
    plan = zm.zero_partition_plan(numels, 4, 128)
    ref = oracle.partition_plan(numels, 4, 128)
    reps = [synth.normal_bf16(ref.padded_numel, 22, synth.KIND_REPLICA, 1, k, 0, ref.numel, 0.05)
            for k in range(3)]
    d_reps = [to_dev_u16(r) for r in reps]
    sq = torch.zeros(2, dtype=torch.float64, device=dev())
    out = torch.zeros(ref.shard_numel, dtype=torch.int16, device=dev())
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev()).fill_(255)
    zm.zero_grad_sqnorm(d[0], sq[0:1], workspace=ws)
    zm.zero_grad_reduce_shard(plan, 1, d_reps, 0, ref.padded_numel, out, sqnorm_out=sq[1:2],
                              workspace=ws)
    torch.cuda.synchronize()
    want_grad = np.zeros(ref.shard_numel, np.uint16)
    oracle.reduce_shard(ref, 1, reps, 0, want_grad)
    assert_bits_equal(host_u16(out), want_grad, "reduce on a shared workspace")
    w1 = oracle.sqnorm(want_grad)
    assert abs(sq[1].item() - w1) <= 1e-12 * w1
    assert sq[0].item() == got[0]


def test_norm_workspace_alignment_is_checked(zm):
    ws = torch.zeros(zm.zero_sqnorm_workspace_bytes() + 8, dtype=torch.uint8, device=dev())
    g = torch.zeros(64, dtype=torch.int16, device=dev())
    out = torch.zeros(1, dtype=torch.float64, device=dev())
    with pytest.raises(zm.ZeroError):
        zm.zero_grad_sqnorm(g, out, workspace=ws[4:])


@pytest.mark.parametrize("partials,max_norm", [
    ([0.25, 0.75], 0.5), ([0.25, 0.75], 2.0), ([3.0], 0.0), ([1.0, math.inf], 1.0),
    ([124.44096632917478], 1.0), ([1e-30] * 64, 1.0), ([0.0], 1.0)])
def test_clip_scale_matches_oracle(zm, partials, max_norm):
    d = torch.tensor(partials, dtype=torch.float64, device=dev())
    out = torch.zeros(1, dtype=torch.float32, device=dev())
    zm.zero_clip_scale(d, max_norm, out)
    torch.cuda.synchronize()
    want = oracle.clip_scale(partials, max_norm)
    got = np.float32(out.item())
    assert (np.isnan(want) and np.isnan(got)) or got == want, (got, want)


# ----------------------------------------------------------------------------- gather

@pytest.mark.parametrize("seed", range(6))
def test_gather_random_plans(zm, seed):
    rng = np.random.default_rng(seed)
    t = int(rng.integers(1, 9))
    numels = [int(x) for x in rng.integers(0, 40_000, t)]
    numels[0] += 1
    n_ranks = int(rng.choice([1, 2, 3, 4, 8]))
    align = int(rng.choice([1, 8, 128]))
    note(f"gather numels={numels} N_d={n_ranks} A={align}")
    ref = oracle.partition_plan(numels, n_ranks, align)
    plan = zm.zero_partition_plan(numels, n_ranks, align)
    S = ref.shard_numel
    shards = [rng.integers(0, 1 << 16, S).astype(np.uint16) for _ in range(n_ranks)]
    want = oracle.gather_params(ref, shards)
    outs = [torch.full((max(n, 1),), 0x5555, dtype=torch.int16, device=dev()) for n in numels]
    zm.zero_gather_params(plan, [to_dev_u16(s) for s in shards],
                          [o[:n] for o, n in zip(outs, numels)])
    torch.cuda.synchronize()
    for i, (o, w) in enumerate(zip(outs, want)):
        assert_bits_equal(host_u16(o)[:numels[i]], w, f"tensor {i}")


def test_gather_workload_plans_and_misaligned_destinations(zm):
    for name in ("tiny-a", "tiny-b", "gpt2-small"):
        w = synth.WORKLOADS[name]
        ref = oracle.partition_plan(w.numels, w.n_ranks, w.align)
        plan = zm.zero_partition_plan(w.numels, w.n_ranks, w.align)
        S = ref.shard_numel
        note(f"gather {name} T={len(w.numels)} S={S}")
        shards = [synth.normal_bf16(S, 30, synth.KIND_PARAM, 0, 0, r * S, ref.numel, 0.02)
                  for r in range(w.n_ranks)]
        d_shards = [to_dev_u16(s) for s in shards]
        # destinations start 1 element into their buffers: bf16 pointers off by 2 bytes
        bufs = [torch.zeros(n + 1, dtype=torch.int16, device=dev()) for n in w.numels]
        zm.zero_gather_params(plan, d_shards, [b[1:] for b in bufs])
        torch.cuda.synchronize()
        flat = np.concatenate(shards)
        for i, b in enumerate(bufs):
            off = ref.offsets[i]
            assert_bits_equal(host_u16(b)[1:], flat[off:off + w.numels[i]], f"{name} tensor {i}")


# ----------------------------------------------------------------------------- flatten

@pytest.mark.parametrize("seed", range(6))
def test_flatten_random_plans(zm, seed):
    rng = np.random.default_rng(100 + seed)
    t = int(rng.integers(1, 9))
    numels = [int(x) for x in rng.integers(0, 40_000, t)]
    numels[-1] += 1
    n_ranks = int(rng.choice([1, 2, 3, 4, 8]))
    align = int(rng.choice([1, 8, 128]))
    note(f"flatten numels={numels} N_d={n_ranks} A={align}")
    ref = oracle.partition_plan(numels, n_ranks, align)
    plan = zm.zero_partition_plan(numels, n_ranks, align)
    tensors = [rng.integers(0, 1 << 16, n).astype(np.uint16) for n in numels]
    want = oracle.flatten_params(ref, tensors)
    # odd seeds place every source one element into its buffer (2-byte misaligned)
    off = seed % 2
    bufs = [to_dev_u16(np.concatenate([np.zeros(off, np.uint16), x])) for x in tensors]
    flat = to_dev_u16(np.full(ref.padded_numel, 0x5555, np.uint16))
    zm.zero_flatten_params(plan, [b[off:] for b in bufs], flat)
    torch.cuda.synchronize()
    assert_bits_equal(host_u16(flat), want, "flat buffer")


def test_flatten_workload_plans_and_gather_round_trip(zm):
    for name in ("tiny-b", "gpt2-small"):
        w = synth.WORKLOADS[name]
        ref = oracle.partition_plan(w.numels, w.n_ranks, w.align)
        plan = zm.zero_partition_plan(w.numels, w.n_ranks, w.align)
        note(f"flatten {name} T={len(w.numels)} P={ref.padded_numel}")
        host = [synth.normal_bf16(n, 40, synth.KIND_GRAD, 1, 0, off, ref.numel, 1e-3)
                for n, off in zip(w.numels, ref.offsets)]
        d_t = [to_dev_u16(x) for x in host]
        flat = torch.full((ref.padded_numel,), 0x2222, dtype=torch.int16, device=dev())
        zm.zero_flatten_params(plan, d_t, flat)
        torch.cuda.synchronize()
        assert_bits_equal(host_u16(flat), oracle.flatten_params(ref, host), f"{name} flat")
        # the generator keys values by global index, so this flat buffer is also the
        # generator's flat gradient with zero padding
        assert_bits_equal(host_u16(flat), synth.normal_bf16(ref.padded_numel, 40, synth.KIND_GRAD,
                                                            1, 0, 0, ref.numel, 1e-3), "generator")
        S = ref.shard_numel
        outs = [torch.empty(n, dtype=torch.int16, device=dev()) for n in w.numels]
        zm.zero_gather_params(plan, [flat[r * S:(r + 1) * S] for r in range(w.n_ranks)], outs)
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, host)):
            assert_bits_equal(host_u16(a), b, f"{name} round trip tensor {i}")


# ----------------------------------------------------------------------------- FSDP-2 Shard(0)

@pytest.mark.parametrize("seed", range(6))
def test_shard0_gather_and_flatten(zm, seed):
    rng = np.random.default_rng(800 + seed)
    t = int(rng.integers(1, 8))
    dim0 = [int(x) for x in rng.integers(1, 3000, t)]
    dim0[0] = int(rng.integers(1, 4))                     # fewer rows than ranks
    numels = [d * int(k) for d, k in zip(dim0, rng.integers(1, 40, t))]
    n_ranks = int(rng.choice([2, 3, 4, 8]))
    align = int(rng.choice([1, 8, 128]))
    note(f"shard0 dim0={dim0} numels={numels} N_d={n_ranks} A={align}")
    ref = oracle.partition_plan_shard0(numels, dim0, n_ranks, align)
    plan = zm.zero_partition_plan_shard0(numels, dim0, n_ranks, align)
    tensors = [rng.integers(0, 1 << 16, n).astype(np.uint16) for n in numels]
    flat = to_dev_u16(np.full(ref.padded_numel, 0x7777, np.uint16))
    zm.zero_flatten_params(plan, [to_dev_u16(x) for x in tensors], flat)
    torch.cuda.synchronize()
    want = oracle.flatten_params_shard0(ref, tensors)
    assert_bits_equal(host_u16(flat), want, "coalesced buffers")
    S = ref.shard_numel
    shards = [rng.integers(0, 1 << 16, S).astype(np.uint16) for _ in range(n_ranks)]
    outs = [torch.full((n,), 0x1357, dtype=torch.int16, device=dev()) for n in numels]
    zm.zero_gather_params(plan, [to_dev_u16(x) for x in shards], outs)
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(outs, oracle.gather_params_shard0(ref, shards))):
        assert_bits_equal(host_u16(a), b, f"tensor {i}")


@pytest.mark.parametrize("kind,n_ranks,t", [("flat", 1, 150), ("flat", 64, 150), ("flat", 65, 150),
                                            ("flat", 100, 150), ("shard0", 3, 400), ("shard0", 8, 400),
                                            ("shard0", 9, 300), ("shard0", 64, 150), ("shard0", 97, 150)])
def test_gather_rank_counts_many_tensors_misaligned(zm, kind, n_ranks, t):
    """Up to 64 ranks the gather finds each element's rank by arithmetic (the
    compact descriptor table up to 8 ranks, the wide one above); above that it
    copies plan segments. All must agree with the oracle, over more tensors
    than one launch carries and with 2-byte-misaligned destinations."""
    rng = np.random.default_rng(900 + n_ranks)
    dim0 = [int(x) for x in rng.integers(1, 300, t)]
    numels = [d * int(k) for d, k in zip(dim0, rng.integers(1, 12, t))]
    note(f"gather {kind} N_d={n_ranks} T={t} Phi={sum(numels)}")
    if kind == "flat":
        ref = oracle.partition_plan(numels, n_ranks, 8)
        plan = zm.zero_partition_plan(numels, n_ranks, 8)
        gather = oracle.gather_params
    else:
        ref = oracle.partition_plan_shard0(numels, dim0, n_ranks, 8)
        plan = zm.zero_partition_plan_shard0(numels, dim0, n_ranks, 8)
        gather = oracle.gather_params_shard0
    S = ref.shard_numel
    shards = [rng.integers(0, 1 << 16, S).astype(np.uint16) for _ in range(n_ranks)]
    bufs = [torch.full((n + 1,), 0x3333, dtype=torch.int16, device=dev()) for n in numels]
    zm.zero_gather_params(plan, [to_dev_u16(x) for x in shards],
                          [b[1:] if i % 2 else b[:-1] for i, b in enumerate(bufs)])
    torch.cuda.synchronize()
    for i, (b, w) in enumerate(zip(bufs, gather(ref, shards))):
        got = host_u16(b)
        assert_bits_equal(got[1:] if i % 2 else got[:-1], w, f"tensor {i}")
        assert (got[0] if i % 2 else got[-1]) == 0x3333, "wrote outside the tensor"


# ----------------------------------------------------------------------------- multi-tensor AdamW

def _mt_stepper(zm, form, dp, dm, dv, dg, do):
    """The multi-tensor update of a fixed list, through the list call or the
    device-resident table."""
    if form == "table":
        tab = zm.MultiTensorTable(dp, dm, dv, dg, do)
        return lambda t, scale=None: tab.step(t, clip_scale=scale, **HP)
    return lambda t, scale=None: zm.zero_multi_tensor_adamw_step(dp, dm, dv, dg, do, t,
                                                                  clip_scale=scale, **HP)


@pytest.mark.parametrize("form", ["list", "table"])
@pytest.mark.parametrize("seed", range(3))
def test_multi_tensor_adamw_matches_oracle(zm, seed, form):
    """A ragged list (sizes around the 256-lane workgroup, empty tensors, more
    tensors than one launch carries, misaligned starts) against the oracle per
    tensor, three steps, device clip coefficient; then the NaN skip."""
    rng = np.random.default_rng(1200 + seed)
    sizes = [int(x) for x in rng.choice([0, 1, 7, 255, 256, 257, 1000, 4099, 70_001], 90)]
    note(f"multi-tensor AdamW: {len(sizes)} tensors, {sum(sizes)} elements")
    off = seed % 2                                   # odd seeds: every array starts 1 element in

    def dev_f32(a):
        return to_dev_f32(np.concatenate([np.zeros(off, np.float32), a]))[off:]

    def dev_u16(a):
        return to_dev_u16(np.concatenate([np.zeros(off, np.uint16), a]))[off:]
    P = [synth.normal_f32(n, 70 + seed, synth.KIND_MASTER, 0, 0, 0, None, 0.02) for n in sizes]
    M = [np.zeros(n, np.float32) for n in sizes]
    V = [np.zeros(n, np.float32) for n in sizes]
    dp, dm, dv = [dev_f32(x) for x in P], [dev_f32(x) for x in M], [dev_f32(x) for x in V]
    dg = [dev_u16(np.zeros(n, np.uint16)) for n in sizes]
    do = [dev_u16(np.full(n, 0x4444, np.uint16)) for n in sizes]
    scale = torch.tensor([0.8125], dtype=torch.float32, device=dev())
    bits = [None] * len(sizes)
    step = _mt_stepper(zm, form, dp, dm, dv, dg, do)
    for t in (1, 2, 3):
        G = [synth.normal_bf16(n, 70 + seed, synth.KIND_GRAD, t, i, 0, None, 1e-3)
             for i, n in enumerate(sizes)]
        for d, g in zip(dg, G):
            d.copy_(torch.from_numpy(g.view(np.int16)))
        step(t, scale)
        for i in range(len(sizes)):
            P[i], M[i], V[i], bits[i] = oracle.adamw_step(P[i], M[i], V[i], G[i], t,
                                                         clip=np.float32(0.8125), **HP)
    torch.cuda.synchronize()
    for i in range(len(sizes)):
        assert_bits_equal(host_f32(dp[i]).view(np.uint32), P[i].view(np.uint32), f"master {i}")
        assert_bits_equal(host_f32(dm[i]).view(np.uint32), M[i].view(np.uint32), f"exp_avg {i}")
        assert_bits_equal(host_f32(dv[i]).view(np.uint32), V[i].view(np.uint32), f"exp_avg_sq {i}")
        assert_bits_equal(host_u16(do[i]), bits[i], f"param {i}")
    before = [x.clone() for x in dp]
    step(4, torch.tensor([float("nan")], device=dev()))
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(before, dp))


@pytest.mark.parametrize("form", ["list", "table"])
def test_multi_tensor_adamw_equals_the_flat_kernel_on_views(zm, form):
    """Tensors that are views into one flat buffer give the flat kernel's bits."""
    sizes = [768, 768, 2304 * 768, 2304, 3, 50_000]
    n = sum(sizes)
    p0 = synth.normal_f32(n, 80, synth.KIND_MASTER, 0, 0, 0, None, 0.02)
    g = to_dev_u16(synth.normal_bf16(n, 80, synth.KIND_GRAD, 1, 0, 0, None, 1e-3))
    flat = [to_dev_f32(p0), torch.zeros(n, device=dev()), torch.zeros(n, device=dev()),
            torch.zeros(n, dtype=torch.int16, device=dev())]
    multi = [to_dev_f32(p0), torch.zeros(n, device=dev()), torch.zeros(n, device=dev()),
             torch.zeros(n, dtype=torch.int16, device=dev())]
    offs = np.cumsum([0] + sizes)

    def views(x):
        return [x[a:b] for a, b in zip(offs[:-1], offs[1:])]
    step = _mt_stepper(zm, form, views(multi[0]), views(multi[1]), views(multi[2]), views(g),
                       views(multi[3]))
    for t in (1, 2):
        zm.zero_shard_adamw_step(flat[0], flat[1], flat[2], g, flat[3], t, **HP)
        step(t)
    torch.cuda.synchronize()
    for a, b, name in zip(flat, multi, ("master", "exp_avg", "exp_avg_sq", "param")):
        assert torch.equal(a, b), name


def test_multi_tensor_table_blocks_prepared_call_and_empty_list(zm):
    """The table's workgroup count (512 elements each, empty tensors none), its
    prepared call against the list call over two steps, and an all-empty list."""
    sizes = [0, 1, 511, 512, 513, 0, 100_000]
    n = sum(sizes)
    p0 = synth.normal_f32(n, 81, synth.KIND_MASTER, 0, 0, 0, None, 0.02)
    g = to_dev_u16(synth.normal_bf16(n, 81, synth.KIND_GRAD, 1, 0, 0, None, 1e-3))
    offs = np.cumsum([0] + sizes)

    def views(x):
        return [x[a:b] for a, b in zip(offs[:-1], offs[1:])]
    bufs = [[to_dev_f32(p0), torch.zeros(n, device=dev()), torch.zeros(n, device=dev()),
             torch.zeros(n, dtype=torch.int16, device=dev())] for _ in range(2)]
    tab = zm.MultiTensorTable(views(bufs[0][0]), views(bufs[0][1]), views(bufs[0][2]), views(g),
                              views(bufs[0][3]))
    assert tab.blocks == sum((k + 511) // 512 for k in sizes)
    scale = torch.tensor([0.5], dtype=torch.float32, device=dev())
    call = tab.prepare_step(clip_scale=scale, stream=None, **HP)
    for t in (1, 2):
        call(t)
        zm.zero_multi_tensor_adamw_step(views(bufs[1][0]), views(bufs[1][1]), views(bufs[1][2]),
                                        views(g), views(bufs[1][3]), t, clip_scale=scale, **HP)
    torch.cuda.synchronize()
    for a, b, name in zip(bufs[0], bufs[1], ("master", "exp_avg", "exp_avg_sq", "param")):
        assert torch.equal(a, b), name
    e = torch.zeros(0, device=dev())
    eh = torch.zeros(0, dtype=torch.int16, device=dev())
    empty = zm.MultiTensorTable([e, e], [e, e], [e, e], [eh, eh], [eh, eh])
    assert empty.blocks == 0
    empty.step(1, **HP)
    del tab, empty


@pytest.mark.parametrize("R", [3, 8])
def test_reduce_two_groups_per_pass_full_array(zm, R):
    """Shards of 2^26 elements and more with at most 8 replicas take the
    two-groups-per-pass kernel: full array and exact norm against the oracle,
    with a ragged tail."""
    n = (1 << 26) + 4099
    plan = zm.zero_partition_plan([n], 1, 1)
    ref = oracle.partition_plan([n], 1, 1)
    note(f"reduce two groups: n={n} R={R}")
    reps = [synth.normal_bf16(n, 91, synth.KIND_REPLICA, 1, k, 0, n, 1e-3) for k in range(R)]
    want = np.zeros(n, np.uint16)
    oracle.reduce_shard(ref, 0, reps, 0, want)
    d_reps = [to_dev_u16(x) for x in reps]
    out = torch.empty(n, dtype=torch.int16, device=dev())
    sq = torch.zeros(1, dtype=torch.float64, device=dev())
    zm.zero_grad_reduce_shard(plan, 0, d_reps, 0, n, out, sqnorm_out=sq)
    torch.cuda.synchronize()
    assert_bits_equal(host_u16(out), want, "reduced")
    want_sq = oracle.sqnorm(want)
    assert abs(sq.item() - want_sq) <= 1e-12 * want_sq


@pytest.mark.parametrize("case", ["odd-window", "eight-replicas", "nine-replicas", "window-in-shard",
                                  "misaligned", "no-norm"])
def test_reduce_one_pass(zm, case):
    """Windows of 2^24 elements or more of at most 8 replicas, with a workspace
    of zero_reduce_workspace_bytes, take the one-pass kernel (a lane per element
    pair, a partial per workgroup, a two-level final sum): bits and exact norm
    against the oracle; the same bf16 output as the grid-stride kernel (fixed
    workspace); the same norm bits when repeated. Nine replicas and a
    2-byte-misaligned window fall back to the other kernels, same result."""
    big = (1 << 24) + 4097                                  # odd: the last element alone
    n_ranks, rank, R, begin, count = {
        "odd-window": (1, 0, 3, 0, big),
        "eight-replicas": (1, 0, 8, 0, big - 1),            # the one-pass maximum
        "nine-replicas": (1, 0, 9, 0, big - 1),             # grid-stride kernels
        "window-in-shard": (2, 1, 4, None, big - 3),         # 6 into rank 1's shard
        "misaligned": (1, 0, 3, 1, big),                    # odd begin: 2-byte offsets
        "no-norm": (1, 0, 5, 0, big),                       # no squared norm: no workspace
    }[case]
    numels = [2 * big + 8] if n_ranks == 2 else [big + 8]
    ref = oracle.partition_plan(numels, n_ranks, 8)
    plan = zm.zero_partition_plan(numels, n_ranks, 8)
    S, phi = ref.shard_numel, ref.numel
    if begin is None:
        begin = S + 6
    assert begin + count <= min((rank + 1) * S, ref.padded_numel)
    note(f"one-pass reduce {case}: R={R} begin={begin} count={count} S={S}")
    reps = [synth.normal_bf16(count, 93, synth.KIND_REPLICA, 1, k, begin, phi, 1e-3) for k in range(R)]
    want = np.full(S, 0x1234, np.uint16)
    lo, hi = oracle.reduce_shard(ref, rank, reps, begin, want)
    want_sq = oracle.sqnorm(want[lo - rank * S:hi - rank * S])
    d_reps = [to_dev_u16(x) for x in reps]
    if case == "no-norm":
        out = to_dev_u16(np.full(S, 0x1234, np.uint16))
        zm.zero_grad_reduce_shard(plan, rank, d_reps, begin, count, out)
        torch.cuda.synchronize()
        assert_bits_equal(host_u16(out), want, "reduced shard, no norm")
        return
    ws = zm.reduce_workspace(count, dev())
    assert ws.numel() > zm.zero_sqnorm_workspace_bytes()
    outs, sqs = [], []
    for workspace in (ws, ws, None):                       # one-pass twice, then the fixed workspace
        out = to_dev_u16(np.full(S, 0x1234, np.uint16))
        sq = torch.full((1,), -1.0, dtype=torch.float64, device=dev())
        zm.zero_grad_reduce_shard(plan, rank, d_reps, begin, count, out, sqnorm_out=sq,
                                  workspace=workspace)
        outs.append(out)
        sqs.append(sq)
    torch.cuda.synchronize()
    assert_bits_equal(host_u16(outs[0]), want, "reduced shard")
    for sq in sqs:
        assert abs(sq.item() - want_sq) <= 1e-12 * want_sq, (sq.item(), want_sq)
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
    assert sqs[0].item() == sqs[1].item()                # repeatable


@pytest.mark.parametrize("off", [0, 1])
def test_sqnorm_one_pass(zm, off):
    """2^24 elements and more, 16-byte aligned, with a workspace of
    zero_reduce_workspace_bytes: the one-pass squared norm (a ragged tail of
    n % 8 values) against the oracle's exact sum, repeatable bit for bit; the
    grid-stride kernel (fixed workspace) agrees within the same bound. A start
    2 bytes off alignment (off = 1) takes the scalar kernel."""
    n = (1 << 24) + 4099
    note(f"one-pass sqnorm n={n} offset={off}")
    g = synth.normal_bf16(n, 94, synth.KIND_GRAD, 1, 0, 0, None, 1e-3)
    want = oracle.sqnorm(g)
    buf = to_dev_u16(np.concatenate([np.zeros(off, np.uint16), g]))[off:]
    ws = zm.reduce_workspace(n, dev())
    got = []
    for workspace in (ws, ws, None):
        sq = torch.full((1,), -1.0, dtype=torch.float64, device=dev())
        zm.zero_grad_sqnorm(buf, sq, workspace=workspace)
        got.append(sq)
    torch.cuda.synchronize()
    for sq in got:
        assert abs(sq.item() - want) <= 1e-12 * want, (sq.item(), want)
    assert got[0].item() == got[1].item()


@pytest.mark.parametrize("n_ranks,t", [(3, 400), (8, 400), (9, 300), (64, 150), (97, 150)])
def test_shard0_flatten_many_tensors_misaligned(zm, n_ranks, t):
    """Shard(0) flatten over more tensors than one launch carries, from
    2-byte-misaligned sources, padding included, against the oracle (64 ranks
    and fewer: tensor-major kernel, compact table up to 8; 97: segment copies)."""
    rng = np.random.default_rng(1300 + n_ranks)
    dim0 = [int(x) for x in rng.integers(1, 400, t)]
    numels = [d * int(k) for d, k in zip(dim0, rng.integers(1, 40, t))]
    note(f"shard0 flatten N_d={n_ranks} T={t} Phi={sum(numels)}")
    ref = oracle.partition_plan_shard0(numels, dim0, n_ranks, 8)
    plan = zm.zero_partition_plan_shard0(numels, dim0, n_ranks, 8)
    tensors = [rng.integers(0, 1 << 16, n).astype(np.uint16) for n in numels]
    bufs = [to_dev_u16(np.concatenate([np.zeros(1, np.uint16), x])) for x in tensors]
    flat = to_dev_u16(np.full(ref.padded_numel, 0x6666, np.uint16))
    zm.zero_flatten_params(plan, [b[1:] for b in bufs], flat)
    torch.cuda.synchronize()
    assert_bits_equal(host_u16(flat), oracle.flatten_params_shard0(ref, tensors), "coalesced buffers")


@pytest.mark.parametrize("kind", ["flat", "shard0"])
def test_gather_skips_null_shards(zm, kind):
    """A NULL shard skips its rank's segments: gathering the other ranks first
    and the remaining rank afterwards gives the full gather."""
    rng = np.random.default_rng(1400)
    dim0 = [int(x) for x in rng.integers(1, 300, 12)]
    numels = [d * int(k) for d, k in zip(dim0, rng.integers(1, 30, 12))]
    n_ranks, rank = 4, 2
    if kind == "flat":
        ref = oracle.partition_plan(numels, n_ranks, 8)
        plan = zm.zero_partition_plan(numels, n_ranks, 8)
        gather = oracle.gather_params
    else:
        ref = oracle.partition_plan_shard0(numels, dim0, n_ranks, 8)
        plan = zm.zero_partition_plan_shard0(numels, dim0, n_ranks, 8)
        gather = oracle.gather_params_shard0
    S = ref.shard_numel
    shards = [rng.integers(0, 1 << 16, S).astype(np.uint16) for _ in range(n_ranks)]
    d = [to_dev_u16(x) for x in shards]
    outs = [torch.full((n,), 0x2468, dtype=torch.int16, device=dev()) for n in numels]
    zm.zero_gather_params(plan, [None if r == rank else x for r, x in enumerate(d)], outs)
    torch.cuda.synchronize()
    marker = [np.full(S, 0x2468, np.uint16) if r == rank else x for r, x in enumerate(shards)]
    for i, (o, w) in enumerate(zip(outs, gather(ref, marker))):
        assert_bits_equal(host_u16(o), w, f"others only, tensor {i}")   # own rank untouched
    zm.zero_gather_params(plan, [x if r == rank else None for r, x in enumerate(d)], outs)
    torch.cuda.synchronize()
    for i, (o, w) in enumerate(zip(outs, gather(ref, shards))):
        assert_bits_equal(host_u16(o), w, f"complete, tensor {i}")


# ----------------------------------------------------------------------------- copy tables

def _random_plan(zm, rng, kind):
    t = int(rng.integers(1, 9))
    dim0 = [int(x) for x in rng.integers(1, 3000, t)]
    dim0[0] = int(rng.integers(1, 4))                     # fewer rows than ranks
    numels = [d * int(k) for d, k in zip(dim0, rng.integers(1, 40, t))]
    n_ranks = int(rng.choice([1, 2, 3, 4, 8]))
    align = int(rng.choice([1, 8, 128]))
    note(f"copy table {kind} dim0={dim0} numels={numels} N_d={n_ranks} A={align}")
    if kind == "flat":
        return (oracle.partition_plan(numels, n_ranks, align), zm.zero_partition_plan(numels, n_ranks, align),
                oracle.gather_params, oracle.flatten_params, numels)
    return (oracle.partition_plan_shard0(numels, dim0, n_ranks, align),
            zm.zero_partition_plan_shard0(numels, dim0, n_ranks, align),
            oracle.gather_params_shard0, oracle.flatten_params_shard0, numels)


@pytest.mark.parametrize("kind", ["flat", "shard0"])
@pytest.mark.parametrize("seed", range(4))
def test_copy_tables_match_the_oracle(zm, seed, kind):
    """Gather and flatten through device tables on random plans, with buffers
    2 bytes off alignment on odd seeds; each table runs twice, with new data in
    its source buffers before the second run."""
    rng = np.random.default_rng(1500 + seed)
    ref, plan, gather, flatten, numels = _random_plan(zm, rng, kind)
    S = ref.shard_numel
    off = seed % 2
    d_sh = [torch.zeros(S + off, dtype=torch.int16, device=dev())[off:] for _ in range(ref.n_ranks)]
    outs = [torch.full((n + off,), 0x5555, dtype=torch.int16, device=dev())[off:] for n in numels]
    tab = zm.CopyTable.gather(plan, d_sh, outs)
    assert tab.blocks == sum((seg[3] + 2047) // 2048 for r in range(ref.n_ranks)
                             for seg in plan.segments(r) if seg[3] > 0)
    for run in range(2):
        shards = [rng.integers(0, 1 << 16, S).astype(np.uint16) for _ in range(ref.n_ranks)]
        for d, x in zip(d_sh, shards):
            d.copy_(torch.from_numpy(x.view(np.int16)))
        tab.run()
        torch.cuda.synchronize()
        for i, (o, w) in enumerate(zip(outs, gather(ref, shards))):
            assert_bits_equal(host_u16(o), w, f"gather run {run} tensor {i}")
    d_t = [torch.zeros(n + off, dtype=torch.int16, device=dev())[off:] for n in numels]
    flat = torch.full((ref.padded_numel + off,), 0x5555, dtype=torch.int16, device=dev())[off:]
    ftab = zm.CopyTable.flatten(plan, d_t, flat)
    for run in range(2):
        tensors = [rng.integers(0, 1 << 16, n).astype(np.uint16) for n in numels]
        for d, x in zip(d_t, tensors):
            d.copy_(torch.from_numpy(x.view(np.int16)))
        flat.fill_(0x3333)
        ftab.run()
        torch.cuda.synchronize()
        assert_bits_equal(host_u16(flat), flatten(ref, tensors), f"flatten run {run}")


@pytest.mark.parametrize("kind", ["flat", "shard0"])
def test_copy_tables_equal_the_calls_on_gpt2_small_and_skip_null_shards(zm, kind):
    """On the GPT-2-small list at N_d = 8, the gather table's output equals
    zero_gather_params's and the flatten table's equals zero_flatten_params's;
    a table made with a NULL shard leaves that rank's elements untouched."""
    w = synth.WORKLOADS["gpt2-small"]
    if kind == "flat":
        plan = zm.zero_partition_plan(w.numels, w.n_ranks, w.align)
    else:
        plan = zm.zero_partition_plan_shard0(w.numels, [s[0] for s in w.shapes], w.n_ranks, w.align)
    S, P = plan.shard_numel, plan.padded_numel
    flat = to_dev_u16(synth.normal_bf16(P, 31, synth.KIND_PARAM, 0, 0, 0, None, 0.02))
    shards = [flat[r * S:(r + 1) * S] for r in range(w.n_ranks)]
    a = [torch.full((n,), 0x1111, dtype=torch.int16, device=dev()) for n in w.numels]
    b = [torch.full((n,), 0x1111, dtype=torch.int16, device=dev()) for n in w.numels]
    zm.zero_gather_params(plan, shards, a)
    zm.CopyTable.gather(plan, shards, b).run()
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(a, b))
    fa = torch.full((P,), 0x2222, dtype=torch.int16, device=dev())
    fb = torch.full((P,), 0x2222, dtype=torch.int16, device=dev())
    zm.zero_flatten_params(plan, a, fa)
    zm.CopyTable.flatten(plan, a, fb).run()
    torch.cuda.synchronize()
    assert torch.equal(fa, fb)
    c = [torch.full((n,), 0x1111, dtype=torch.int16, device=dev()) for n in w.numels]
    d = [torch.full((n,), 0x1111, dtype=torch.int16, device=dev()) for n in w.numels]
    skip = [None if r == 3 else x for r, x in enumerate(shards)]
    zm.zero_gather_params(plan, skip, c)
    zm.CopyTable.gather(plan, skip, d).run()
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(c, d))


# ----------------------------------------------------------------------------- reduce + AdamW

@pytest.mark.parametrize("case", ["full-window", "nine-replicas-window", "sixty-four", "unaligned",
                                  "skip"])
def test_reduce_adamw_one_pass_matches_the_two_calls_and_the_oracle(zm, case):
    """zero_reduce_adamw_step against zero_grad_reduce_shard followed by
    zero_shard_adamw_step on the GPU, and against the oracle's reduce then AdamW,
    bit for bit, over three steps: the averaged gradient (when asked for), the
    fp32 state and the bf16 parameters; elements of the shard outside the window
    stay as they were. [ZF] "Execution Flow for ZeRO-1", steps 2-3."""
    numels, n_ranks, rank, R = [100_000, 77_777, 5], 4, 1, 3
    begin_off, count_cut, clip, with_grad = 0, 0, 0.37, True
    if case == "nine-replicas-window":
        R, begin_off, count_cut, clip, with_grad = 9, 20_001, 13_337, None, False
    elif case == "sixty-four":
        R = 64
    elif case == "unaligned":
        begin_off, count_cut = 3, 1
    elif case == "skip":
        clip = float("nan")
    ref = oracle.partition_plan(numels, n_ranks, 128)
    plan = zm.zero_partition_plan(numels, n_ranks, 128)
    P, S, phi = ref.padded_numel, ref.shard_numel, ref.numel
    lo_s = rank * S
    begin = lo_s + begin_off - 7 if begin_off else 0        # windows that start before the shard too
    count = (lo_s + S - count_cut) - begin if count_cut else P - begin
    note(f"reduce+adamw {case}: R={R} window [{begin},{begin + count}) shard [{lo_s},{lo_s + S})")
    master = synth.normal_f32(S, 31, synth.KIND_MASTER, 0, 0, lo_s, phi, 0.02)
    d = {}
    for way in ("fused", "calls"):
        d[way] = dict(p=to_dev_f32(master), m=torch.zeros(S, dtype=torch.float32, device=dev()),
                      v=torch.zeros(S, dtype=torch.float32, device=dev()),
                      o=torch.full((S,), 0x2222, dtype=torch.int16, device=dev()),
                      g=torch.full((S,), 0x1111, dtype=torch.int16, device=dev()))
    scale = None if clip is None else torch.tensor([clip], dtype=torch.float32, device=dev())
    st = {"p": master.copy(), "m": np.zeros(S, np.float32), "v": np.zeros(S, np.float32),
          "o": np.full(S, 0x2222, np.uint16), "g": np.full(S, 0x1111, np.uint16)}
    a, b = max(begin, lo_s) - lo_s, min(begin + count, lo_s + S) - lo_s
    for t in (1, 2, 3):
        reps_h = [synth.normal_bf16(count, 31, synth.KIND_REPLICA, t, k, begin, phi, 0.05)
                  for k in range(R)]
        reps = [to_dev_u16(x) for x in reps_h]
        f, c = d["fused"], d["calls"]
        zm.zero_reduce_adamw_step(plan, rank, reps, begin, count, f["p"], f["m"], f["v"], f["o"], t,
                                  clip_scale=scale, shard_grad=f["g"] if with_grad else None, **HP)
        zm.zero_grad_reduce_shard(plan, rank, reps, begin, count, c["g"])
        zm.zero_shard_adamw_step(c["p"][a:b], c["m"][a:b], c["v"][a:b], c["g"][a:b], c["o"][a:b], t,
                                 clip_scale=scale, **HP)
        g = st["g"].copy()
        oracle.reduce_shard(ref, rank, reps_h, begin, g)
        P1, M1, V1, B1 = oracle.adamw_step(st["p"][a:b], st["m"][a:b], st["v"][a:b], g[a:b], t,
                                           clip=1.0 if clip is None else clip, **HP)
        st["g"] = g
        st["p"][a:b], st["m"][a:b], st["v"][a:b] = P1, M1, V1
        if B1 is not None:
            st["o"][a:b] = B1
    torch.cuda.synchronize()
    f, c = d["fused"], d["calls"]
    for key, what in (("p", "master"), ("m", "exp_avg"), ("v", "exp_avg_sq")):
        assert_bits_equal(host_f32(f[key]).view(np.uint32), host_f32(c[key]).view(np.uint32),
                          f"{what}: one pass against the two calls")
        assert_bits_equal(host_f32(f[key]).view(np.uint32), st[key].view(np.uint32),
                          f"{what}: one pass against the oracle")
    assert_bits_equal(host_u16(f["o"]), host_u16(c["o"]), "param: one pass against the two calls")
    assert_bits_equal(host_u16(f["o"]), st["o"], "param: one pass against the oracle")
    if with_grad:
        assert_bits_equal(host_u16(f["g"]), st["g"], "averaged gradient against the oracle")
    else:
        assert (host_u16(f["g"]) == 0x1111).all(), "no gradient written when none is asked for"
    if case == "skip":
        assert_bits_equal(host_f32(f["p"]).view(np.uint32), master.view(np.uint32), "skipped: master")
        assert (host_u16(f["o"]) == 0x2222).all(), "skipped: param untouched"


# ----------------------------------------------------------------------------- reduce from per-tensor replicas

def _tensor_replicas(rng, numels, R):
    """R replicas, each a list of per-tensor bf16 arrays of finite values."""
    return [[oracle.f32_to_bf16((rng.standard_normal(n) * 0.05).astype(np.float32)) for n in numels]
            for _ in range(R)]


def _device_tensors(rep, misalign=False):
    """Device copies, each tensor in an allocation of its own; with misalign,
    every tensor starts 2 bytes into its allocation."""
    out = []
    for a in rep:
        if misalign:
            buf = torch.empty(len(a) + 1, dtype=torch.int16, device=dev())
            v = buf[1:]
            v.copy_(to_dev_u16(a))
            out.append(v)
        else:
            out.append(to_dev_u16(a))
    return out


def _oracle_reduce_from_tensors(ref, rank, reps, shard0):
    """The oracle's flatten of every replica, then its reduce of the rank's shard."""
    flatten = oracle.flatten_params_shard0 if shard0 else oracle.flatten_params
    flats = [flatten(ref, rep) for rep in reps]
    want = np.zeros(ref.shard_numel, np.uint16)
    oracle.reduce_shard(ref, rank, flats, 0, want)
    return want, oracle.sqnorm(want)


def _check_reduce_table(zm, ref, plan, reps_h, shard0, misalign=False, note_prefix=""):
    S = ref.shard_numel
    d_reps = [_device_tensors(rep, misalign) for rep in reps_h]
    for rank in range(ref.n_ranks):
        grad = torch.full((S,), 0x1234, dtype=torch.int16, device=dev())
        sq = torch.full((1,), -1.0, dtype=torch.float64, device=dev())
        table = zm.ReduceTable(plan, rank, d_reps, grad)
        table.run(sqnorm_out=sq)
        torch.cuda.synchronize()
        want, want_sq = _oracle_reduce_from_tensors(ref, rank, reps_h, shard0)
        assert_bits_equal(host_u16(grad), want, f"{note_prefix}rank {rank} gradient")
        got_sq = float(sq.item())
        assert abs(got_sq - want_sq) <= 1e-12 * want_sq, (rank, got_sq, want_sq)
        del table


@pytest.mark.parametrize("seed", range(4))
def test_reduce_table_flat_plans(zm, seed):
    """zero_reduce_table_*: every rank's averaged gradient straight from R
    per-tensor replicas, against the oracle's flatten of each replica and its
    reduce; ragged tensor sizes (16-byte and element-wise pieces), padding at
    the end, R from 1 to 9."""
    rng = np.random.default_rng(1300 + seed)
    t = int(rng.integers(1, 9))
    numels = [int(x) for x in rng.integers(1, 9000, t)]
    numels[0] = int(rng.integers(1, 5)) * 8                # an aligned small one
    n_ranks = int(rng.choice([1, 2, 4, 8]))
    align = int(rng.choice([1, 8, 128]))
    R = [1, 3, 8, 9][seed]
    ref = oracle.partition_plan(numels, n_ranks, align)
    plan = zm.zero_partition_plan(numels, n_ranks, align)
    note(f"reduce table flat: numels={numels} N_d={n_ranks} A={align} R={R}")
    _check_reduce_table(zm, ref, plan, _tensor_replicas(rng, numels, R), False)


@pytest.mark.parametrize("seed", range(4))
def test_reduce_table_shard0_plans(zm, seed):
    """The same on FSDP-2 Shard(0) plans: each rank's chunks of every tensor,
    with the rows' padding in between written as zeros."""
    rng = np.random.default_rng(1400 + seed)
    t = int(rng.integers(1, 8))
    dim0 = [int(x) for x in rng.integers(1, 3000, t)]
    dim0[0] = int(rng.integers(1, 4))                      # fewer rows than ranks
    numels = [d * int(k) for d, k in zip(dim0, rng.integers(1, 40, t))]
    n_ranks = int(rng.choice([2, 3, 4, 8]))
    align = int(rng.choice([1, 8, 128]))
    R = [2, 5, 8, 12][seed]
    ref = oracle.partition_plan_shard0(numels, dim0, n_ranks, align)
    plan = zm.zero_partition_plan_shard0(numels, dim0, n_ranks, align)
    note(f"reduce table shard0: dim0={dim0} numels={numels} N_d={n_ranks} A={align} R={R}")
    _check_reduce_table(zm, ref, plan, _tensor_replicas(rng, numels, R), True)


def test_reduce_table_misaligned_replicas_and_reruns(zm):
    """Replica tensors 2 bytes into their allocations take the element-wise
    path with the same bits; a table run again after its buffers are rewritten
    in place reduces the new contents; a run without sqnorm_out writes the same
    gradient."""
    rng = np.random.default_rng(1500)
    numels = [4096, 37, 8000, 3, 2048 * 3 + 5]
    ref = oracle.partition_plan(numels, 4, 128)
    plan = zm.zero_partition_plan(numels, 4, 128)
    reps_h = _tensor_replicas(rng, numels, 4)
    _check_reduce_table(zm, ref, plan, reps_h, False, misalign=True, note_prefix="misaligned ")
    rank, S = 2, ref.shard_numel
    d_reps = [_device_tensors(rep) for rep in reps_h]
    grad = torch.zeros(S, dtype=torch.int16, device=dev())
    table = zm.ReduceTable(plan, rank, d_reps, grad)
    assert table.blocks == sum(-(-ln // 2048) for ln in _pieces_lengths(ref, rank))
    for call in range(3):
        new_h = _tensor_replicas(rng, numels, 4)
        for dr, hr in zip(d_reps, new_h):
            for d, h in zip(dr, hr):
                d.copy_(to_dev_u16(h))
        sq = torch.zeros(1, dtype=torch.float64, device=dev())
        table.run(sqnorm_out=sq if call != 1 else None)
        torch.cuda.synchronize()
        want, want_sq = _oracle_reduce_from_tensors(ref, rank, new_h, False)
        assert_bits_equal(host_u16(grad), want, f"run {call}")
        if call != 1:
            assert abs(float(sq.item()) - want_sq) <= 1e-12 * want_sq


def _pieces_lengths(ref, rank):
    """Lengths of the rank's segments and of the padding gaps around them."""
    out, pos = [], 0
    for (_, _, soff, ln) in ref.segments(rank):
        if soff > pos:
            out.append(soff - pos)
        out.append(ln)
        pos = soff + ln
    if ref.shard_numel > pos:
        out.append(ref.shard_numel - pos)
    return out


def test_reduce_table_gpt2_small_rank7_eight_replicas(zm):
    """The GPT-2-small list, rank 7 of 8, 8 per-tensor replicas generated on
    the device (each tensor keyed by its flat offset, so a flattened replica is
    the generator's flat buffer): the table's gradient and squared norm against
    the oracle's reduce of the generated flat replicas' slice."""
    w = synth.WORKLOADS["gpt2-small"]
    rank, R, seed = 7, 8, 1600
    ref = oracle.partition_plan(w.numels, 8, w.align)
    plan = zm.zero_partition_plan(w.numels, 8, w.align)
    S, phi = ref.shard_numel, ref.numel
    reps = []
    for k in range(R):
        rep = []
        for n, off in zip(w.numels, ref.offsets):
            t = torch.empty(n, dtype=torch.int16, device=dev())
            synth.device_normal_bf16(t, seed, synth.KIND_REPLICA, 1, k, off, phi, synth.GRAD_SIGMA)
            rep.append(t)
        reps.append(rep)
    grad = torch.full((S,), 0x4321, dtype=torch.int16, device=dev())
    sq = torch.zeros(1, dtype=torch.float64, device=dev())
    table = zm.ReduceTable(plan, rank, reps, grad)
    table.run(sqnorm_out=sq)
    torch.cuda.synchronize()
    flats = [synth.normal_bf16(S, seed, synth.KIND_REPLICA, 1, k, rank * S, phi, synth.GRAD_SIGMA)
             for k in range(R)]
    window = oracle.partition_plan([S], 1, 1)              # the reduce is elementwise
    want = np.zeros(S, np.uint16)
    oracle.reduce_shard(window, 0, flats, 0, want)
    assert_bits_equal(host_u16(grad), want, "gpt2-small rank 7 gradient")
    want_sq = oracle.sqnorm(want)
    assert abs(float(sq.item()) - want_sq) <= 1e-12 * want_sq
    note(f"gpt2-small rank 7: {S} elements from {R} x {len(w.numels)} tensors, "
         f"{table.blocks} workgroups, bit-identical")


def test_reduce_table_edge_cases(zm):
    """The reduce table at R = 64 (the most replicas the ABI takes), on a plan
    whose last ranks hold only padding (written as zeros, squared norm exactly
    0), and on a one-rank plan (the whole model is the shard)."""
    rng = np.random.default_rng(1700)
    numels = [3000, 17, 500]
    ref = oracle.partition_plan(numels, 8, 512)                # P = 4096: ranks 7.. hold padding
    plan = zm.zero_partition_plan(numels, 8, 512)
    assert ref.segments(7) == [] and ref.shard_numel == 512
    _check_reduce_table(zm, ref, plan, _tensor_replicas(rng, numels, 64), False, note_prefix="R=64 ")
    ref1 = oracle.partition_plan(numels, 1, 8)
    plan1 = zm.zero_partition_plan(numels, 1, 8)
    _check_reduce_table(zm, ref1, plan1, _tensor_replicas(rng, numels, 2), False, note_prefix="one rank ")
