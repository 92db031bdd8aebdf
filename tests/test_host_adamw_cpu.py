"""ZeRO-Offload's host update (zero_host_adamw_step) against the oracle, on the CPU.

It runs the device kernel's exact per-element arithmetic on the host, so the
bar is bit-identical fp32 state and bf16 parameters."""
import numpy as np
import pytest

import oracle
import synth

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


@pytest.fixture(scope="module")
def zm():
    import zero_partitioned_mixed_partition_amd as m
    return m


def _inputs(n, seed):
    p = synth.normal_f32(n, seed, synth.KIND_MASTER, 0, 0, sigma=0.02)
    m = synth.normal_f32(n, seed, 10, 0, 0, sigma=1e-4)
    v = np.abs(synth.normal_f32(n, seed, 11, 0, 0, sigma=1e-7))
    g = synth.normal_bf16(n, seed, synth.KIND_GRAD, 1, 0, sigma=1e-3)
    return p, m, v, g


@pytest.mark.parametrize("n,threads", [(1, 1), (7, 4), (65_537, 3), ((1 << 20) + 3, 0),
                                       ((1 << 20) + 3, 1)])
def test_host_adamw_matches_oracle_bit_for_bit(zm, n, threads):
    p, m, v, g = _inputs(n, 40 + n % 13)
    out = np.zeros(n, np.uint16)
    for t in (1, 2, 3):
        zm.zero_host_adamw_step(p, m, v, g, out, t, clip_scale=0.37, n_threads=threads, **HP)
    P, M, V = _inputs(n, 40 + n % 13)[:3]
    for t in (1, 2, 3):
        P, M, V, B = oracle.adamw_step(P, M, V, g, t, clip=0.37, **HP)
    assert (p.view(np.uint32) == P.view(np.uint32)).all()
    assert (m.view(np.uint32) == M.view(np.uint32)).all()
    assert (v.view(np.uint32) == V.view(np.uint32)).all()
    assert (out == B).all()


@pytest.mark.parametrize("case", ["betas-zero-no-decay", "betas-near-one", "lr-eps-one-negative-decay",
                                  "decay-factor-zero", "huge-steps"])
def test_host_adamw_hyperparameter_corners(zm, case):
    """The host update's own fp64 scalars at their extremes, against the oracle
    bit for bit (no momentum, betas next to 1, negative and large weight decay,
    lr and eps of 1, bias corrections that round to 1)."""
    hp, steps = {
        "betas-zero-no-decay": (dict(HP, beta1=0.0, beta2=0.0, weight_decay=0.0), (1, 2, 3)),
        "betas-near-one": (dict(HP, beta1=0.999999, beta2=0.999999), (1, 2)),
        "lr-eps-one-negative-decay": (dict(HP, lr=1.0, eps=1.0, weight_decay=-0.5), (1, 2)),
        "decay-factor-zero": (dict(HP, lr=0.01, weight_decay=100.0), (1, 2)),
        "huge-steps": (HP, (10 ** 6, 2 ** 40)),
    }[case]
    n = 4097
    p, m, v, g = _inputs(n, 31)
    out = np.zeros(n, np.uint16)
    P, M, V = p.copy(), m.copy(), v.copy()
    for t in steps:
        zm.zero_host_adamw_step(p, m, v, g, out, t, n_threads=2, **hp)
        P, M, V, B = oracle.adamw_step(P, M, V, g, t, **hp)
    assert (p.view(np.uint32) == P.view(np.uint32)).all()
    assert (m.view(np.uint32) == M.view(np.uint32)).all()
    assert (v.view(np.uint32) == V.view(np.uint32)).all()
    assert (out == B).all()


@pytest.mark.filterwarnings("ignore:overflow encountered:RuntimeWarning", "ignore:invalid value encountered:RuntimeWarning")
def test_host_adamw_special_values_and_skip(zm):
    n = 64
    p = np.linspace(-3, 3, n).astype(np.float32)
    p[0], p[1], p[2] = 0.0, -0.0, 1e-40
    g32 = np.linspace(-1e-2, 1e-2, n).astype(np.float32)
    g32[3], g32[4], g32[5], g32[7], g32[8] = np.inf, -np.inf, np.nan, 1e-38, 3e38
    g = oracle.f32_to_bf16(g32)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    out = np.zeros(n, np.uint16)
    P, M, V, B = oracle.adamw_step(p, m, v, g, 1, **HP)
    q = p.copy()
    zm.zero_host_adamw_step(q, m, v, g, out, 1, **HP)
    same = (q.view(np.uint32) == P.view(np.uint32)) | (np.isnan(q) & np.isnan(P))
    assert same.all()
    nan_b = (B & 0x7FFF) > 0x7F80
    assert ((out == B) | (nan_b & ((out & 0x7FFF) > 0x7F80))).all()
    # a non-finite clip coefficient skips the update
    r = p.copy()
    z = np.zeros(n, np.float32)
    out2 = np.full(n, 9, np.uint16)
    zm.zero_host_adamw_step(r, z, z.copy(), g, out2, 1, clip_scale=float("nan"), **HP)
    assert (r.view(np.uint32) == p.view(np.uint32)).all() and (out2 == 9).all()


def test_host_adamw_argument_errors(zm):
    x = np.zeros(4, np.float32)
    h = np.zeros(4, np.uint16)
    with pytest.raises(zm.ZeroError):
        zm.zero_host_adamw_step(x, x.copy(), x.copy(), h, h.copy(), 0, **HP)
    with pytest.raises(zm.ZeroError):
        zm.zero_host_adamw_step(x, x.copy(), x.copy(), h, h.copy(), 1, **dict(HP, beta2=1.0))
    with pytest.raises(ValueError):
        zm.zero_host_adamw_step(x, x.copy(), x.copy(), h[:2], h.copy(), 1, **HP)
    # arrays that share memory: the pool's slices would race
    with pytest.raises(zm.ZeroError, match="master overlaps exp_avg"):
        zm.zero_host_adamw_step(x, x, x.copy(), h, h.copy(), 1, **HP)
    with pytest.raises(zm.ZeroError, match="param_out overlaps grad"):
        zm.zero_host_adamw_step(x, x.copy(), x.copy(), h, h, 1, **HP)
    y = np.zeros(8, np.float32)
    with pytest.raises(zm.ZeroError, match="exp_avg overlaps exp_avg_sq"):
        zm.zero_host_adamw_step(x, y[:4], y[3:7], h, h.copy(), 1, **HP)


def test_host_pool_repeated_and_concurrent_runs_agree(zm):
    """Many back-to-back runs of the worker pool, with varying task counts and
    from two caller threads at once, give the single-threaded bits."""
    import threading
    n = 300_007
    p0, m0, v0, g = _inputs(n, 77)
    ref = [p0.copy(), m0.copy(), v0.copy(), np.zeros(n, np.uint16)]
    for t in range(1, 6):
        zm.zero_host_adamw_step(*ref[:3], g, ref[3], t, n_threads=1, **HP)

    def run(threads_seq, out):
        st = [p0.copy(), m0.copy(), v0.copy(), np.zeros(n, np.uint16)]
        for t, th in zip(range(1, 6), threads_seq):
            zm.zero_host_adamw_step(*st[:3], g, st[3], t, n_threads=th, **HP)
        out.append(st)

    outs = []
    for seq in ([2, 3, 5, 8, 64], [7, 4, 1, 16, 3]):
        run(seq, outs)
    th = [threading.Thread(target=run, args=([5, 6, 7, 8, 9], outs)) for _ in range(2)]
    for x in th:
        x.start()
    for x in th:
        x.join()
    assert len(outs) == 4
    for st in outs:
        for a, b in zip(st, ref):
            assert (a.view(a.dtype) == b).all() if a.dtype == np.uint16 else \
                (a.view(np.uint32) == b.view(np.uint32)).all()
