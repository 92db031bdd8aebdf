"""AdamW's per-step scalars and the step schedule's host side, on the CPU.

Every AdamW entry point computes a step's eight fp32 scalars on the host
(zero_adamw_step_scalars); the device-resident schedule holds them for steps
1..L and reuses step L's for every later step. Checked here: the scalars
against the oracle's, bit for bit, over many steps and hyperparameter sets,
including steps far past the point where both bias corrections round to 1;
that the scalars stop changing at the documented step; and the schedule's
argument errors, which all come before any HIP call.
"""
import ctypes
import math

import numpy as np
import pytest

import oracle

HP_SETS = [
    dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01),
    dict(lr=3e-4, beta1=0.0, beta2=0.0, eps=1e-6, weight_decay=0.0),
    dict(lr=1.0, beta1=0.99, beta2=0.9999, eps=1.0, weight_decay=-0.5),
    dict(lr=0.02, beta1=0.5, beta2=0.95, eps=1e-12, weight_decay=100.0),
]


@pytest.fixture(scope="module")
def zm():
    import zero_partitioned_mixed_partition_amd as m
    return m


def _want(t, hp):
    c = oracle.adamw_constants(t, hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"])
    return np.array([c.beta1, c.one_minus_beta1, c.beta2, c.one_minus_beta2, c.eps, c.step_size,
                     c.sqrt_bc2, c.decay], np.float32)


@pytest.mark.parametrize("i", range(len(HP_SETS)))
def test_step_scalars_match_the_oracle(zm, i):
    hp = HP_SETS[i]
    rng = np.random.default_rng(i)
    steps = list(range(1, 200)) + [int(x) for x in rng.integers(200, 10 ** 7, 200)] + [2 ** 31, 2 ** 40, 2 ** 62]
    for t in steps:
        got = zm.zero_adamw_step_scalars(t, **hp)
        assert (got.view(np.uint32) == _want(t, hp).view(np.uint32)).all(), (t, got, _want(t, hp))


@pytest.mark.parametrize("beta1,beta2", [(0.9, 0.999), (0.0, 0.0), (0.99, 0.9999), (0.5, 0.95)])
def test_scalars_stop_changing_once_both_corrections_round_to_one(zm, beta1, beta2):
    """The documented settled step L: the first t with beta1^t and beta2^t both
    below 2^-56. From L on every scalar equals step L's, and step L - 1 differs
    only where a correction had not yet reached 1 (so the table may end at L)."""
    def below(t):
        return beta1 ** t < 2.0 ** -56 and beta2 ** t < 2.0 ** -56
    L = 1
    while not below(L):
        L += 1
    hp = dict(lr=1e-3, beta1=beta1, beta2=beta2, eps=1e-8, weight_decay=0.01)
    at_l = zm.zero_adamw_step_scalars(L, **hp)
    for t in (L, L + 1, L + 7, L + 1000, 2 * L + 3, 2 ** 31, 2 ** 40):
        assert (zm.zero_adamw_step_scalars(t, **hp).view(np.uint32) == at_l.view(np.uint32)).all(), t
    # the settled values are the limits: step size lr, sqrt(1 - beta2^t) = 1
    assert at_l[5] == np.float32(1e-3) and at_l[6] == np.float32(1.0)
    if beta2 == 0.999:
        assert L == 38_797       # the figure the header gives


def test_schedule_arguments_are_checked_before_touching_the_gpu(zm):
    lib = zm._binding
    E = lib.ZERO_EINVAL
    out = ctypes.c_void_p()
    lr = (ctypes.c_double * 2)(1e-3, 2e-3)

    def create(rates=lr, n=2, b1=0.9, b2=0.999, eps=1e-8, wd=0.01, first=1, o=ctypes.byref(out)):
        return lib._sched_create(rates, n, b1, b2, eps, wd, first, o)
    assert create(o=None) == E
    assert create(rates=None) == E and create(n=0) == E
    assert create(first=0) == E
    assert create(b1=1.0) == E and create(b2=-0.1) == E and create(eps=0.0) == E
    assert create(rates=(ctypes.c_double * 2)(1e-3, -1.0)) == E          # a negative rate
    assert create(rates=(ctypes.c_double * 2)(1e-3, math.inf)) == E
    assert create(b2=1.0 - 1e-7) == lib.ZERO_ERANGE                        # settles past 2^24 steps
    assert "settle" in zm.zero_last_error()
    assert not out.value
    assert lib._sched_length(None) == -1
    assert lib._sched_applied(None, ctypes.byref(ctypes.c_int64())) == E
    assert lib._sched_advance(None, None, None) == E
    lib._sched_free(None)
    f = (ctypes.c_float * 8)()
    assert lib._step_scalars(0, 1e-3, 0.9, 0.999, 1e-8, 0.0, f) == E     # step < 1
    assert lib._step_scalars(1, 1e-3, 0.9, 0.999, 1e-8, 0.0, None) == E
    assert lib._adamw_sched(None, None, None, None, None, 1, None, None, None) == E   # NULL schedule
    assert lib._mt_step_sched(None, None, None, None) == E                           # NULL table
    plan = zm.zero_partition_plan([1000], 2, 1)
    reps = (ctypes.c_void_p * 2)(0x10000, 0x20000)
    state = [ctypes.c_void_p(0x100000 * (k + 1)) for k in range(4)]
    assert lib._reduce_adamw_sched(plan.handle, 1, reps, 2, 0, 1000, *state, None, None, None, None) == E
    assert "NULL schedule" in zm.zero_last_error()
