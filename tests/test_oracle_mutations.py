"""Planted mistakes: each plausible slip in the oracle must fail one of its pins.

Every case below replaces one oracle function, on the CPU, with a copy that
carries a single mistake (a dropped term, a wrong sign, a swapped operand, an
off-by-one), runs the pins that cover it, and asserts that at least one pin
fails. A mutation that every pin accepts would mean the pins cannot tell the
oracle from a wrong one.
"""
import math

import numpy as np
import pytest

import oracle
import test_oracle_numerics as num
import test_oracle_plan as pln
from oracle import adamw as adamw_mod
from oracle.bf16 import bf16_to_f32, f32_to_bf16

f32 = np.float32


def _adamw_with(mistake):
    """An adamw_step carrying one mistake; the rest follows the oracle."""
    def step(master, exp_avg, exp_avg_sq, grad_bits, step, lr, beta1, beta2, eps, weight_decay,
             clip=1.0):
        c = oracle.adamw_constants(step, lr, beta1, beta2, eps, weight_decay)
        clip32 = f32(clip)
        if not np.isfinite(clip32):
            return master.copy(), exp_avg.copy(), exp_avg_sq.copy(), None
        b1, omb1, b2, omb2 = c.beta1, c.one_minus_beta1, c.beta2, c.one_minus_beta2
        ss, sbc2, dec, e = c.step_size, c.sqrt_bc2, c.decay, c.eps
        if mistake == "no_bias_correction":
            ss, sbc2 = f32(lr), f32(1.0)
        if mistake == "decay_without_lr":
            dec = f32(1.0 - weight_decay)
        if mistake == "swapped_beta1":
            b1, omb1 = omb1, b1
        if mistake == "beta1_for_v":
            b2, omb2 = b1, omb1
        g = bf16_to_f32(grad_bits) * (f32(1.0) if mistake == "clip_ignored" else clip32)
        m = b1 * exp_avg + omb1 * g
        v = b2 * exp_avg_sq + omb2 * (g * g)
        p = master * dec
        if mistake == "eps_inside_sqrt":
            denom = np.sqrt(v + e) / sbc2
        elif mistake == "no_eps":
            denom = np.sqrt(v) / sbc2
        else:
            denom = np.sqrt(v) / sbc2 + e
        if mistake == "wrong_sign":
            p = p + ss * (m / denom)
        else:
            p = p - ss * (m / denom)
        if mistake == "decay_after_update":
            p = (master - ss * (m / denom)) * dec
        return p, m, v, f32_to_bf16(p)
    return step


ADAMW_PINS = [
    num.test_adamw_step1_closed_form,
    lambda: num.test_adamw_constant_gradient_closed_form(0.01),
    num.test_adamw_matches_torch_optim_adamw,
]


def _caught(checks) -> bool:
    for check in checks:
        try:
            check()
        except AssertionError:
            return True
    return False


@pytest.mark.parametrize("mistake", ["no_bias_correction", "decay_without_lr", "swapped_beta1",
                                     "beta1_for_v", "clip_ignored", "eps_inside_sqrt", "no_eps",
                                     "wrong_sign", "decay_after_update"])
def test_adamw_mistakes_are_caught(monkeypatch, mistake):
    monkeypatch.setattr(oracle, "adamw_step", _adamw_with(mistake))
    monkeypatch.setattr(adamw_mod, "adamw_step", _adamw_with(mistake))
    assert _caught(ADAMW_PINS), mistake


def test_unmutated_adamw_passes_its_pins():
    assert not _caught(ADAMW_PINS)


def _reduce_with(mistake):
    def reduce_shard(plan, rank, replicas, begin, shard_grad):
        count = len(replicas[0])
        s = plan.shard_numel
        lo = max(begin, rank * s)
        hi = min(begin + count, (rank + 1) * s)
        if lo >= hi:
            return lo, lo
        acc = np.zeros(hi - lo, dtype=np.float32)
        for rep in replicas:
            acc = acc + bf16_to_f32(rep[lo - begin:hi - begin])
        r = len(replicas)
        if mistake == "sum_not_mean":
            avg = acc
        elif mistake == "divide_by_r_minus_1":
            avg = acc / np.float32(max(r - 1, 1))
        elif mistake == "first_replica_only":
            avg = bf16_to_f32(replicas[0][lo - begin:hi - begin])
        elif mistake == "truncate":
            avg = acc / np.float32(r)
            shard_grad[lo - rank * s:hi - rank * s] = (avg.view(np.uint32) >> 16).astype(np.uint16)
            return lo, hi
        else:
            avg = acc / np.float32(r)
        shard_grad[lo - rank * s:hi - rank * s] = f32_to_bf16(avg)
        return lo, hi
    return reduce_shard


REDUCE_PINS = [num.test_reduce_single_replica_is_identity,
               lambda: num.test_reduce_identical_replicas(8),
               lambda: num.test_reduce_is_the_rne_of_the_exact_mean(8)]


@pytest.mark.parametrize("mistake", ["sum_not_mean", "divide_by_r_minus_1", "first_replica_only",
                                     "truncate"])
def test_reduce_mistakes_are_caught(monkeypatch, mistake):
    monkeypatch.setattr(oracle, "reduce_shard", _reduce_with(mistake))
    assert _caught(REDUCE_PINS), mistake


def test_unmutated_reduce_passes_its_pins():
    assert not _caught(REDUCE_PINS)


def _sqnorm_with(mistake):
    def sqnorm(bits):
        b = np.asarray(bits, dtype=np.uint16).ravel()
        if b.size == 0:
            return 0.0
        e = ((b >> np.uint16(7)) & np.uint16(0xFF)).astype(np.int64)
        frac = (b & np.uint16(0x7F)).astype(np.float64)
        m = np.where(e > 0, frac + (127.0 if mistake == "hidden_bit" else 128.0), frac)
        per = np.bincount(e, weights=m * m, minlength=256)
        off = 133 if mistake == "exponent_bias" else 134
        terms = [math.ldexp(per[x], 2 * (x - off) if x > 0 else -266) for x in range(255) if per[x]]
        if mistake == "abs_not_square":
            terms = [math.ldexp(float(np.sum(np.where(e == x, m, 0.0))), x - off)
                     for x in range(1, 255) if per[x]]
        return math.fsum(terms)
    return sqnorm


SQNORM_PINS = [lambda: num.test_sqnorm_exact_matches_fsum(0), num.test_sqnorm_closed_forms]


@pytest.mark.parametrize("mistake", ["hidden_bit", "exponent_bias", "abs_not_square"])
def test_sqnorm_mistakes_are_caught(monkeypatch, mistake):
    monkeypatch.setattr(oracle, "sqnorm", _sqnorm_with(mistake))
    assert _caught(SQNORM_PINS), mistake


def _clip_with(mistake):
    def clip_scale(partials, max_norm):
        total = sum(float(p) for p in partials)
        if not math.isfinite(total):
            return np.float32(np.nan)
        if max_norm <= 0.0:
            return np.float32(1.0)
        norm = math.sqrt(total) if mistake != "no_sqrt" else total
        coef = max_norm / (norm + 1e-6)
        return np.float32(coef if mistake == "no_min" else min(1.0, coef))
    return clip_scale


@pytest.mark.parametrize("mistake", ["no_sqrt", "no_min"])
def test_clip_mistakes_are_caught(monkeypatch, mistake):
    monkeypatch.setattr(oracle, "clip_scale", _clip_with(mistake))
    assert _caught([num.test_clip_scale_closed_form]), mistake


def _bf16_with(mistake):
    def to_bf16(x):
        u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
        if mistake == "truncate":
            return (u >> np.uint32(16)).astype(np.uint16)
        if mistake == "ties_away":
            return ((u + np.uint32(0x8000)) >> np.uint32(16)).astype(np.uint16)
        raise AssertionError
    return to_bf16


@pytest.mark.parametrize("mistake", ["truncate", "ties_away"])
def test_bf16_mistakes_are_caught(monkeypatch, mistake):
    monkeypatch.setattr(num, "f32_to_bf16", _bf16_with(mistake))
    assert _caught([num.test_bf16_rne_matches_torch_on_every_rounding_case]), mistake


def _plan_with(mistake):
    def partition_plan(numels, n_ranks, align=128):
        numels = [int(n) for n in numels]
        if n_ranks < 1 or align < 1 or any(n < 0 for n in numels):
            raise ValueError("invalid plan arguments")
        offsets, total = [], 0
        for n in numels:
            offsets.append(total + (1 if mistake == "offset_off_by_one" and total else 0))
            total += n
        unit = n_ranks if mistake == "ignore_align" else n_ranks * align
        padded = -(-total // unit) * unit
        if mistake == "floor_not_ceil":
            padded = total // unit * unit
        return oracle.Plan(numels, n_ranks, align, offsets, total, padded, padded // n_ranks)
    return partition_plan


PLAN_PINS = [lambda: pln.test_tiny_a_segments_worked_by_hand(pln_golden()),
             lambda: pln.test_plan_brute_force_tiny(3),
             lambda: pln.test_workload_plans("gpt2-small")]


def pln_golden():
    import os
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.mark.parametrize("mistake", ["offset_off_by_one", "ignore_align", "floor_not_ceil"])
def test_plan_mistakes_are_caught(monkeypatch, mistake):
    monkeypatch.setattr(oracle, "partition_plan", _plan_with(mistake))
    assert _caught(PLAN_PINS), mistake


def test_gather_reversed_shards_is_caught(monkeypatch):
    real = oracle.gather_params

    def reversed_gather(plan, shards):
        return real(plan, list(reversed(shards)))
    monkeypatch.setattr(oracle, "gather_params", reversed_gather)
    assert _caught([lambda s=s: num.test_gather_round_trip_and_segments(s) for s in range(10)])


# ----------------------------------------------------------------------------- Shard(0), flatten

import test_oracle_shard0 as sh0  # noqa: E402
from oracle.plan import Shard0Plan  # noqa: E402


def _shard0_with(mistake):
    """partition_plan_shard0 carrying one mistake."""
    def partition_plan_shard0(numels, dim0, n_ranks, align=128):
        numels = [int(n) for n in numels]
        dim0 = [int(d) for d in dim0]
        offsets, rows_l, inner_l, buf = [], [], [], 0
        for n, d in zip(numels, dim0):
            inner = n // d if n else 0
            rows = -(-d // n_ranks) if n else 0
            if mistake == "floor_rows" and n:
                rows = max(d // n_ranks, 1)
            if mistake == "element_chunks" and n:      # cut the flattened tensor, not its rows
                rows, inner = -(-n // n_ranks), 1
            offsets.append(buf)
            rows_l.append(rows)
            inner_l.append(inner)
            buf += rows * inner
            if mistake == "chunks_unpadded" and n:     # the last rank's short chunk sets the stride
                buf -= rows * inner - max(d - (n_ranks - 1) * rows, 0) * inner
        s = buf if mistake == "ignore_align" else -(-buf // align) * align
        return Shard0Plan(numels, n_ranks, align, offsets, sum(numels), s * n_ranks, s,
                          dim0=dim0, chunk_rows=rows_l, inner=inner_l)
    return partition_plan_shard0


SHARD0_PINS = [sh0.test_shard0_hand_worked,
               *[lambda s=s: sh0.test_shard0_matches_torch_chunk(s) for s in range(25)],
               *[lambda s=s: sh0.test_shard0_round_trip_and_coverage(s) for s in range(10)]]


def _caught_any(checks) -> bool:
    """As _caught, but a mistake may also surface as an exception other than an
    assertion (an index past a buffer, a shape mismatch)."""
    for check in checks:
        try:
            check()
        except (AssertionError, ValueError, IndexError):
            return True
    return False


@pytest.mark.parametrize("mistake", ["floor_rows", "element_chunks", "chunks_unpadded",
                                     "ignore_align"])
def test_shard0_plan_mistakes_are_caught(monkeypatch, mistake):
    monkeypatch.setattr(oracle, "partition_plan_shard0", _shard0_with(mistake))
    assert _caught_any(SHARD0_PINS), mistake


def test_unmutated_shard0_passes_its_pins():
    assert not _caught_any(SHARD0_PINS)


@pytest.mark.parametrize("mistake", ["padding_not_zeroed", "ranks_reversed"])
def test_shard0_flatten_gather_mistakes_are_caught(monkeypatch, mistake):
    real_flatten, real_gather = oracle.flatten_params_shard0, oracle.gather_params_shard0
    if mistake == "padding_not_zeroed":
        def flatten(plan, tensors):
            flat = real_flatten(plan, tensors)
            covered = np.zeros(plan.padded_numel, bool)
            for r in range(plan.n_ranks):
                for (_, _, soff, ln) in plan.segments(r):
                    covered[r * plan.shard_numel + soff:r * plan.shard_numel + soff + ln] = True
            flat[~covered] = 0x3F80                  # what an uncleared buffer might hold
            return flat
        monkeypatch.setattr(oracle, "flatten_params_shard0", flatten)
    else:
        def gather(plan, shards):
            return real_gather(plan, list(reversed(shards)))
        monkeypatch.setattr(oracle, "gather_params_shard0", gather)
    assert _caught_any([lambda s=s: sh0.test_shard0_round_trip_and_coverage(s) for s in range(10)]), \
        mistake


@pytest.mark.parametrize("mistake", ["offset_off_by_one", "padding_not_zeroed"])
def test_flatten_mistakes_are_caught(monkeypatch, mistake):
    def flatten(plan, tensors):
        flat = np.zeros(plan.padded_numel, dtype=np.uint16)
        if mistake == "padding_not_zeroed":
            flat[:] = 0x3F80
        for t, off, n in zip(tensors, plan.offsets, plan.numels):
            o = off + (1 if mistake == "offset_off_by_one" and off else 0)
            flat[o:o + n] = np.asarray(t, dtype=np.uint16)[:len(flat[o:o + n])]
        return flat
    monkeypatch.setattr(oracle, "flatten_params", flatten)
    assert _caught_any([num.test_flatten_hand_worked_and_round_trips]), mistake
