"""Pins for the oracle's floating-point parts (CPU only).

Each test checks the oracle against something other than itself: a library
routine, a closed form, exact rational arithmetic, or a special case.
"""
import math
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle.bf16 import bf16_to_f32, f32_to_bf16

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def _ulp32(x):
    x = np.abs(np.asarray(x, dtype=np.float32))
    return np.spacing(x).astype(np.float64)


def _close32(got, ref, rel=1e-6, ulps=4):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    tol = np.maximum(rel * np.abs(ref), ulps * _ulp32(ref))
    return np.abs(got - ref) <= tol


# ----------------------------------------------------------------------------- bf16

def _torch_bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def test_bf16_rne_matches_torch_on_every_rounding_case():
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0, 1, 0x3FFF, 0x7FFF, 0x8000, 0x8001, 0xBFFF, 0xFFFF], dtype=np.uint32)
    u = (hi[:, None] | lows[None, :]).ravel()
    x = u.view(np.float32)
    finite_or_inf = (u & 0x7FFFFFFF) <= 0x7F800000
    assert (f32_to_bf16(x[finite_or_inf]) == _torch_bf16(x[finite_or_inf])).all()


def test_bf16_nan_inf_zero_subnormal():
    x = np.array([np.nan, -np.nan, np.inf, -np.inf, 0.0, -0.0, 1e-40, -1e-40,
                  3.4e38], dtype=np.float32)
    b = f32_to_bf16(x)
    back = bf16_to_f32(b)
    assert np.isnan(back[0]) and np.isnan(back[1])
    assert (b[0] & 0x40) and (b[1] & 0x8000)        # quiet bit set, sign kept
    assert back[2] == np.inf and back[3] == -np.inf
    assert b[4] == 0 and b[5] == 0x8000
    assert back[6] != 0 and back[7] != 0             # no flush of subnormals
    assert back[8] == np.inf                          # rounds past the largest bf16
    # widening is exact: every non-NaN pattern survives the round trip
    allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ok = (allb & 0x7FFF) <= 0x7F80
    assert (f32_to_bf16(bf16_to_f32(allb[ok])) == allb[ok]).all()


# ----------------------------------------------------------------------------- sqnorm

def _random_bf16(rng, n, lo=-40, hi=40):
    mant = rng.integers(0, 128, n)
    exp = rng.integers(127 + lo, 127 + hi, n)
    sign = rng.integers(0, 2, n)
    return ((sign << 15) | (exp << 7) | mant).astype(np.uint16)


@pytest.mark.parametrize("seed", range(5))
def test_sqnorm_exact_matches_fsum(seed):
    rng = np.random.default_rng(seed)
    b = _random_bf16(rng, 20000)
    b[:50] = rng.integers(0, 128, 50).astype(np.uint16)          # subnormals and zeros
    assert oracle.sqnorm(b) == oracle.sqnorm_fsum(b)


def test_sqnorm_closed_forms():
    # n copies of c: n * c^2 exactly (c^2 has 16 significant bits)
    for c in (1.0, -0.0078125, 3.0e-3, 1.5e20):
        cb = f32_to_bf16(np.array([c], np.float32))[0]
        cv = float(bf16_to_f32(np.array([cb]))[0])
        n = 1_000_003
        assert oracle.sqnorm(np.full(n, cb, np.uint16)) == n * cv * cv
    assert oracle.sqnorm(np.zeros(0, np.uint16)) == 0.0
    inf = f32_to_bf16(np.array([np.inf], np.float32))
    assert oracle.sqnorm(np.concatenate([inf, np.ones(3, np.uint16)])) == math.inf
    nan = f32_to_bf16(np.array([np.nan], np.float32))
    assert math.isnan(oracle.sqnorm(np.concatenate([nan, inf])))


# ----------------------------------------------------------------------------- clip

def test_clip_scale_closed_form():
    assert oracle.clip_scale([0.25, 0.75], 0.5) == np.float32(0.5 / (1.0 + 1e-6))
    assert oracle.clip_scale([0.25, 0.75], 2.0) == np.float32(1.0)
    assert oracle.clip_scale([123.0], 0.0) == np.float32(1.0)
    assert np.isnan(oracle.clip_scale([1.0, math.inf], 1.0))
    assert np.isnan(oracle.clip_scale([math.nan], 1.0))
    # an expected-norm case: 124.4M N(0, 1e-3) values have norm ~ 11.155
    s = oracle.clip_scale([124_439_808 * 1e-6], 1.0)
    assert abs(float(s) - 1 / math.sqrt(124.439808)) < 1e-6


# ----------------------------------------------------------------------------- reduce

def _flat_plan(n, n_ranks=1):
    return oracle.partition_plan([n], n_ranks, 1)


def test_reduce_single_replica_is_identity():
    rng = np.random.default_rng(1)
    g = _random_bf16(rng, 1000)
    plan = _flat_plan(1000)
    out = np.zeros(1000, np.uint16)
    oracle.reduce_shard(plan, 0, [g], 0, out)
    assert (out == g).all()


@pytest.mark.parametrize("r", [2, 3, 8, 64])
def test_reduce_identical_replicas(r):
    rng = np.random.default_rng(r)
    g = _random_bf16(rng, 777, lo=-20, hi=20)
    plan = _flat_plan(777)
    out = np.zeros(777, np.uint16)
    oracle.reduce_shard(plan, 0, [g] * r, 0, out)
    assert (out == g).all()       # k*x exact for small k, so the mean is x


def _rne_bf16_of_fraction(q: Fraction) -> float:
    """Exact RNE of a rational to bf16 (normal range, q != 0)."""
    sign = -1 if q < 0 else 1
    q = abs(q)
    e = math.floor(math.log2(q))
    while Fraction(2) ** e > q:
        e -= 1
    while Fraction(2) ** (e + 1) <= q:
        e += 1
    scaled = q / Fraction(2) ** (e - 7)       # in [128, 256)
    lo = math.floor(scaled)
    rem = scaled - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return sign * float(Fraction(lo) * Fraction(2) ** (e - 7))


@pytest.mark.parametrize("r", [2, 4, 8, 16, 64])
def test_reduce_is_the_rne_of_the_exact_mean(r):
    # values k/64 with |k| < 256: every fp32 partial sum is exact, and /R is
    # exact for R a power of two, so the only rounding is the final bf16 one.
    rng = np.random.default_rng(100 + r)
    n = 400
    ks = rng.integers(-255, 256, size=(r, n))
    reps = [f32_to_bf16((k / 64.0).astype(np.float32)) for k in ks]
    plan = _flat_plan(n)
    out = np.zeros(n, np.uint16)
    oracle.reduce_shard(plan, 0, reps, 0, out)
    got = bf16_to_f32(out).astype(np.float64)
    for i in range(n):
        mean = Fraction(int(ks[:, i].sum()), 64 * r)
        want = 0.0 if mean == 0 else _rne_bf16_of_fraction(mean)
        assert got[i] == want, (i, mean)


def test_reduce_window_and_shard_intersection():
    plan = oracle.partition_plan([100, 60], 4, 8)     # Phi 160, P 160, S 40
    rng = np.random.default_rng(3)
    reps = [_random_bf16(rng, 50) for _ in range(3)]  # window [30, 80)
    out = np.full(plan.shard_numel, 0xFFFF, np.uint16)
    lo, hi = oracle.reduce_shard(plan, 1, reps, 30, out)   # shard 1 = [40, 80)
    assert (lo, hi) == (40, 80)
    full = np.zeros(40, np.uint16)
    oracle.reduce_shard(_flat_plan(40), 0, [x[10:50] for x in reps], 0, full)
    assert (out == full).all()
    out0 = np.full(plan.shard_numel, 0xFFFF, np.uint16)
    oracle.reduce_shard(plan, 0, reps, 30, out0)           # shard 0 = [0, 40): only 30..39
    assert (out0[:30] == 0xFFFF).all()
    head = np.zeros(10, np.uint16)
    oracle.reduce_shard(_flat_plan(10), 0, [x[:10] for x in reps], 0, head)
    assert (out0[30:] == head).all()


# ----------------------------------------------------------------------------- AdamW

def test_adamw_step1_closed_form():
    rng = np.random.default_rng(7)
    n = 5000
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    gb = f32_to_bf16((rng.standard_normal(n) * 1e-3).astype(np.float32))
    z = np.zeros(n, np.float32)
    p, m, v, bits = oracle.adamw_step(p0, z, z, gb, 1, **HP)
    g = bf16_to_f32(gb).astype(np.float64)
    d = 1 - HP["lr"] * HP["weight_decay"]
    want = p0.astype(np.float64) * d - HP["lr"] * g / (np.abs(g) + HP["eps"])
    # the two terms can cancel, so the error bound scales with the larger term:
    # a few fp32 roundings of quantities of size max(|p0|, lr)
    scale = np.maximum(np.abs(p0).astype(np.float64), HP["lr"])
    assert (np.abs(p - want) <= np.maximum(1e-6 * np.abs(want), 4 * _ulp32(scale))).all()
    assert _close32(m, (1 - HP["beta1"]) * g).all()
    assert _close32(v, (1 - HP["beta2"]) * g * g).all()
    assert (bits == f32_to_bf16(p)).all()


@pytest.mark.parametrize("wd", [0.01, 0.0])
def test_adamw_constant_gradient_closed_form(wd):
    # with a constant gradient the bias-corrected moments are exactly g and g^2,
    # so p_T = d^T p_0 - lr * g/(|g|+eps) * (1 + d + ... + d^(T-1)), d = 1 - lr*wd
    rng = np.random.default_rng(8)
    n, T = 3000, 20
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    p0 = p.astype(np.float64)
    gb = f32_to_bf16((rng.standard_normal(n) * 1e-3).astype(np.float32))
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    hp = dict(HP, weight_decay=wd)
    for t in range(1, T + 1):
        p, m, v, _ = oracle.adamw_step(p, m, v, gb, t, **hp)
    g = bf16_to_f32(gb).astype(np.float64)
    d = 1 - hp["lr"] * wd
    geo = T if wd == 0 else (1 - d ** T) / (1 - d)
    want = d ** T * p0 - hp["lr"] * g / (np.abs(g) + hp["eps"]) * geo
    # T steps of fp32 rounding in a value whose update is ~lr per step
    tol = np.maximum(1e-6 * np.abs(want), 3 * T * np.spacing(np.float32(0.05)))
    assert (np.abs(p - want) <= tol).all()


def test_adamw_zero_lr_keeps_master():
    rng = np.random.default_rng(9)
    n = 1000
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    gb = f32_to_bf16((rng.standard_normal(n) * 1e-3).astype(np.float32))
    z = np.zeros(n, np.float32)
    p, _, _, bits = oracle.adamw_step(p0, z, z, gb, 1, **dict(HP, lr=0.0))
    assert (p.view(np.uint32) == p0.view(np.uint32)).all()
    assert (bits == _torch_bf16(p0)).all()


def test_adamw_matches_torch_optim_adamw():
    rng = np.random.default_rng(10)
    n, T = 4096, 10
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    tp = torch.nn.Parameter(torch.from_numpy(p0.copy()))
    opt = torch.optim.AdamW([tp], lr=HP["lr"], betas=(HP["beta1"], HP["beta2"]), eps=HP["eps"],
                            weight_decay=HP["weight_decay"], foreach=False, fused=False)
    p, m, v = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    for t in range(1, T + 1):
        gb = f32_to_bf16((rng.standard_normal(n) * 1e-3).astype(np.float32))
        clip = np.float32(0.37) if t % 2 else np.float32(1.0)
        tp.grad = torch.from_numpy(bf16_to_f32(gb) * clip)
        opt.step()
        p, m, v, bits = oracle.adamw_step(p, m, v, gb, t, clip=clip, **HP)
    st = opt.state[tp]
    # torch evaluates m by lerp and v by addcmul, a different fp32 order, so the
    # two agree to rounding only; where an element's value cancels toward zero
    # the bound is taken from the array's scale (its RMS) instead of the element
    for mine, ref in ((p, tp.detach().numpy()), (m, st["exp_avg"].numpy()),
                      (v, st["exp_avg_sq"].numpy())):
        rms = float(np.sqrt(np.mean(ref.astype(np.float64) ** 2)))
        ok = _close32(mine, ref) | (np.abs(mine.astype(np.float64) - ref) <= 1e-6 * rms)
        assert ok.all()
    dist = np.abs(bits.astype(np.int32) - _torch_bf16(tp.detach().numpy()).astype(np.int32))
    assert dist.max() <= 1


def _f32(x):
    return struct.unpack("f", struct.pack("f", x))[0]


def test_adamw_brute_force_scalar_loop():
    # an independent scalar transcription with binary64 operations rounded to
    # binary32 after each step; binary64 has more than 2*24+2 bits, so each
    # rounded result equals the correctly rounded binary32 operation
    rng = np.random.default_rng(11)
    n = 64
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v = (rng.random(n) * 1e-7).astype(np.float32)
    gb = f32_to_bf16((rng.standard_normal(n) * 1e-3).astype(np.float32))
    t, clip = 7, 0.5
    P, M, V, B = oracle.adamw_step(p, m, v, gb, t, clip=clip, **HP)
    c = oracle.adamw_constants(t, **HP)
    for i in range(n):
        g = _f32(float(bf16_to_f32(gb[i:i + 1])[0]) * _f32(clip))
        mi = _f32(_f32(float(c.beta1) * float(m[i])) + _f32(float(c.one_minus_beta1) * g))
        vi = _f32(_f32(float(c.beta2) * float(v[i])) + _f32(float(c.one_minus_beta2) * _f32(g * g)))
        pi = _f32(float(p[i]) * float(c.decay))
        den = _f32(_f32(_f32(math.sqrt(vi)) / float(c.sqrt_bc2)) + float(c.eps))
        pi = _f32(pi - _f32(float(c.step_size) * _f32(mi / den)))
        assert (M[i], V[i], P[i]) == (np.float32(mi), np.float32(vi), np.float32(pi))


def test_adamw_nonfinite_clip_skips():
    rng = np.random.default_rng(12)
    p = (rng.standard_normal(10) * 0.02).astype(np.float32)
    z = np.zeros(10, np.float32)
    gb = f32_to_bf16(np.ones(10, np.float32))
    P, M, V, B = oracle.adamw_step(p, z, z, gb, 1, clip=float("nan"), **HP)
    assert B is None and (P == p).all() and (M == 0).all() and (V == 0).all()
    with pytest.raises(ValueError):
        oracle.adamw_step(p, z, z, gb, 0, **HP)


@pytest.mark.parametrize("n_ranks", [2, 4, 8, 64])
def test_shard_invariance(n_ranks):
    # partitioning keeps data-parallel semantics: N_d shard updates, each fed its
    # slice and the same global clip, concatenate to the unpartitioned update
    rng = np.random.default_rng(13)
    numels = [int(x) for x in rng.integers(1, 900, 6)]
    plan = oracle.partition_plan(numels, n_ranks, 8)
    P = plan.padded_numel
    phi = plan.numel
    p = np.zeros(P, np.float32)
    p[:phi] = rng.standard_normal(phi) * 0.02
    gb = np.zeros(P, np.uint16)
    gb[:phi] = f32_to_bf16((rng.standard_normal(phi) * 0.05).astype(np.float32))
    z = np.zeros(P, np.float32)
    full_clip = oracle.clip_scale([oracle.sqnorm(gb)], 1.0)
    Pf, Mf, Vf, Bf = oracle.adamw_step(p, z, z, gb, 3, clip=full_clip, **HP)
    S = plan.shard_numel
    parts = [oracle.sqnorm(gb[r * S:(r + 1) * S]) for r in range(n_ranks)]
    clip = oracle.clip_scale(parts, 1.0)
    assert clip == full_clip
    outs = [oracle.adamw_step(p[r * S:(r + 1) * S], z[:S], z[:S], gb[r * S:(r + 1) * S], 3,
                              clip=clip, **HP) for r in range(n_ranks)]
    assert (np.concatenate([o[0] for o in outs]).view(np.uint32) == Pf.view(np.uint32)).all()
    assert (np.concatenate([o[3] for o in outs]) == Bf).all()
    # padding stays exactly zero
    assert (Pf[phi:] == 0).all() and (Bf[phi:] == 0).all()


# ----------------------------------------------------------------------------- gather

@pytest.mark.parametrize("seed", range(10))
def test_gather_round_trip_and_segments(seed):
    rng = np.random.default_rng(seed)
    numels = [int(x) for x in rng.integers(0, 500, int(rng.integers(1, 7)))]
    n_ranks = int(rng.choice([1, 2, 3, 4, 8]))
    plan = oracle.partition_plan(numels, n_ranks, int(rng.choice([1, 8, 128])))
    tensors = [rng.integers(0, 1 << 16, n).astype(np.uint16) for n in numels]
    flat = np.zeros(plan.padded_numel, np.uint16)
    pos = 0
    for t in tensors:
        flat[pos:pos + len(t)] = t
        pos += len(t)
    S = plan.shard_numel
    shards = [flat[r * S:(r + 1) * S] for r in range(n_ranks)]
    out = oracle.gather_params(plan, shards)
    for a, b in zip(out, tensors):
        assert (a == b).all()
    # the plan's segment table describes the same copy
    seg_out = [np.full(n, 0xABCD, np.uint16) for n in numels]
    for r in range(n_ranks):
        for (t, toff, soff, ln) in plan.segments(r):
            seg_out[t][toff:toff + ln] = shards[r][soff:soff + ln]
    for a, b in zip(seg_out, tensors):
        assert (a == b).all()


def test_rank_step_composes_parts():
    rng = np.random.default_rng(14)
    plan = oracle.partition_plan([300, 41, 200], 4, 8)
    S, P = plan.shard_numel, plan.padded_numel
    reps = [np.zeros(P, np.uint16) for _ in range(4)]
    for r in reps:
        r[:plan.numel] = f32_to_bf16((rng.standard_normal(plan.numel) * 0.1).astype(np.float32))
    state = {k: np.zeros(S, np.float32) for k in ("master", "exp_avg", "exp_avg_sq")}
    state["master"][:] = rng.standard_normal(S) * 0.02
    shards = [np.zeros(S, np.uint16) for _ in range(4)]
    out = oracle.rank_step(plan, 2, reps, 0, state, shards, [0.1, 0.2, 0.0, 0.3], 1, HP, 1.0)
    g = np.zeros(S, np.uint16)
    oracle.reduce_shard(plan, 2, reps, 0, g)
    assert (out["shard_grad"] == g).all()
    assert out["partials"][2] == oracle.sqnorm(g)
    assert out["clip"] == oracle.clip_scale([0.1, 0.2, oracle.sqnorm(g), 0.3], 1.0)
    assert len(out["tensors"]) == 3


def test_sqnorm_accumulator_chunks_equal_whole():
    rng = np.random.default_rng(21)
    b = _random_bf16(rng, 50_000, lo=-60, hi=60)
    acc = oracle.SqnormAccumulator()
    for i in range(0, len(b), 7_777):
        acc.add(b[i:i + 7_777])
    assert acc.value() == oracle.sqnorm_fsum(b)


def test_sqnorm_accumulator_merge_is_exact():
    rng = np.random.default_rng(22)
    b = _random_bf16(rng, 30_000, lo=-60, hi=60)
    parts = [oracle.SqnormAccumulator().add(b[i:i + 4000]) for i in range(0, len(b), 4000)]
    acc = oracle.SqnormAccumulator()
    for p in parts:
        acc.merge(p)
    assert acc.value() == oracle.sqnorm_fsum(b)


def test_flatten_hand_worked_and_round_trips():
    # [2], [3] over 2 ranks with 2-element alignment: Phi 5, P 8, S 4
    plan = oracle.partition_plan([2, 3], 2, 2)
    flat = oracle.flatten_params(plan, [np.array([1, 2], np.uint16), np.array([3, 4, 5], np.uint16)])
    assert flat.tolist() == [1, 2, 3, 4, 5, 0, 0, 0]
    rng = np.random.default_rng(31)
    for seed in range(10):
        numels = [int(x) for x in rng.integers(0, 700, int(rng.integers(1, 6)))]
        p = oracle.partition_plan(numels, int(rng.choice([1, 2, 3, 8])), int(rng.choice([1, 8, 128])))
        tensors = [rng.integers(0, 1 << 16, n).astype(np.uint16) for n in numels]
        flat = oracle.flatten_params(p, tensors)
        assert (flat[p.numel:] == 0).all()
        S = p.shard_numel
        back = oracle.gather_params(p, [flat[r * S:(r + 1) * S] for r in range(p.n_ranks)])
        for a, b in zip(back, tensors):
            assert (a == b).all()
