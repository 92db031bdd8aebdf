"""Process-pool helpers that run oracle computations over generated inputs.

Imported by spawned worker processes: numpy, the generator and the oracle only.
Each task regenerates its own inputs from the seeded generator, so nothing
large crosses process boundaries except results.
"""
import multiprocessing as mp
import os
from concurrent.futures import ProcessPoolExecutor


def _init(threads: int) -> None:
    os.environ["OMP_NUM_THREADS"] = str(threads)


def _pool(workers):
    workers = workers or max(1, min(8, (os.cpu_count() or 2) // 2))
    return ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn"),
                               initializer=_init, initargs=(2,))


def _grad_slice_sqnorm(args):
    import oracle
    import synth
    seed, kind, step, replica, g0, n, phi, sigma = args
    acc = oracle.SqnormAccumulator()
    for off in range(0, n, 1 << 22):
        m = min(1 << 22, n - off)
        acc.add(synth.normal_bf16(m, seed, kind, step, replica, g0 + off, phi, sigma))
    return acc.value()


def grad_sqnorms(tasks, workers=None):
    """tasks: (seed, kind, step, replica, g0, n, phi, sigma) per generated gradient
    slice; returns the oracle's exact squared norm of each, in task order."""
    with _pool(workers) as ex:
        return list(ex.map(_grad_slice_sqnorm, tasks, chunksize=1))


def _reduce_window(args):
    """The oracle's reduce of R generated replicas over global window [w0, w1),
    which must lie inside rank's shard; returns (bf16 bits, exact sqnorm state)."""
    import numpy as np
    import oracle
    import synth
    numels, n_ranks, align, rank, seed, kind, step, n_rep, w0, w1, sigma = args
    plan = oracle.partition_plan(numels, n_ranks, align)
    s = plan.shard_numel
    assert rank * s <= w0 < w1 <= (rank + 1) * s
    reps = [synth.normal_bf16(w1 - w0, seed, kind, step, k, w0, plan.numel, sigma)
            for k in range(n_rep)]
    # the reduce is elementwise: the window, seen as a one-rank flat buffer of its own
    window = oracle.partition_plan([w1 - w0], 1, 1)
    bits = np.zeros(w1 - w0, np.uint16)
    oracle.reduce_shard(window, 0, reps, 0, bits)
    return bits, oracle.SqnormAccumulator().add(bits)


def reduce_windows(tasks, workers=None):
    with _pool(workers) as ex:
        return list(ex.map(_reduce_window, tasks, chunksize=1))


def _reduce_window_sqnorm(args):
    """The exact squared-norm state of the oracle's reduce over one window
    (as _reduce_window, without returning the bits)."""
    return _reduce_window(args)[1]


def reduce_window_sqnorms(tasks, workers=None):
    """Per task (as reduce_windows), the exact squared-norm state of the
    oracle's reduced gradient over that window, in task order."""
    with _pool(workers) as ex:
        return list(ex.map(_reduce_window_sqnorm, tasks, chunksize=1))


def digest(a) -> str:
    """128-bit digest of an array's bytes: two arrays agree bit for bit exactly
    when their digests do (up to a 2^-128 collision)."""
    import numpy as np
    import xxhash
    return xxhash.xxh3_128_hexdigest(np.ascontiguousarray(a).view(np.uint8))


def _adamw_steps_digests(args):
    """The oracle's AdamW over one window of a shard for steps 1..T, with the
    generated gradient of each step and the given clip coefficients; returns,
    per step, the digests of (master, exp_avg, exp_avg_sq, param bits)."""
    import numpy as np
    import oracle
    import synth
    seed, g0, n, phi, scales, hp = args
    p = synth.normal_f32(n, seed, synth.KIND_MASTER, 0, 0, g0, phi, synth.MASTER_SIGMA)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    out = []
    for t, clip in enumerate(scales, start=1):
        g = synth.normal_bf16(n, seed, synth.KIND_GRAD, t, 0, g0, phi, synth.GRAD_SIGMA)
        p, m, v, bits = oracle.adamw_step(p, m, v, g, t, clip=clip, **hp)
        out.append((digest(p), digest(m), digest(v), digest(bits)))
    return out


def adamw_steps_digests(tasks, workers=None):
    with _pool(workers) as ex:
        return list(ex.map(_adamw_steps_digests, tasks, chunksize=1))


def _reduce_adamw_digests(args):
    """One step of a window of a rank's shard, from R generated replicas: the
    oracle's reduce, then AdamW step 1 from master ~ N(0, 0.02) and zero moments.
    Returns the digests of (grad bits, master, exp_avg, exp_avg_sq, param bits)
    and the exact squared-norm state of the reduced gradient."""
    import numpy as np
    import oracle
    import synth
    numels, n_ranks, align, rank, seed, n_rep, w0, w1, hp = args
    bits, acc = _reduce_window((numels, n_ranks, align, rank, seed, synth.KIND_REPLICA, 1, n_rep,
                                w0, w1, synth.GRAD_SIGMA))
    phi = sum(numels)
    p0 = synth.normal_f32(w1 - w0, seed, synth.KIND_MASTER, 0, 0, w0, phi, synth.MASTER_SIGMA)
    z = np.zeros(w1 - w0, np.float32)
    P1, M1, V1, B1 = oracle.adamw_step(p0, z, z, bits, 1, **hp)
    return (digest(bits), digest(P1), digest(M1), digest(V1), digest(B1)), acc


def reduce_adamw_digests(tasks, workers=None):
    with _pool(workers) as ex:
        for r in ex.map(_reduce_adamw_digests, tasks, chunksize=1):
            yield r


def canonical_nan_f32(a):
    """float32 bits with every NaN replaced by one quiet NaN (0x7FC00000): NaN
    signs and payloads that IEEE leaves open (the sign of sqrt of a negative
    number) compare equal."""
    import numpy as np
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).copy()
    u[(u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)] = np.uint32(0x7FC00000)
    return u


def canonical_nan_bf16(a):
    import numpy as np
    u = np.ascontiguousarray(a, dtype=np.uint16).copy()
    u[(u & np.uint16(0x7FFF)) > np.uint16(0x7F80)] = np.uint16(0x7FC0)
    return u


def _adamw_sweep_digests(args):
    """The oracle's AdamW step on n elements whose second moment runs over the
    float32 bit patterns [lo, lo + n) (mod 2^32), with master p0, first moment m0
    and a zero gradient; digests of (master, exp_avg, exp_avg_sq, param) after
    NaN canonicalisation."""
    import numpy as np
    import oracle
    lo, n, p0, m0, step, hp = args
    v = (np.arange(lo, lo + n, dtype=np.uint64) & np.uint64(0xFFFFFFFF)).astype(np.uint32).view(np.float32)
    p = np.full(n, p0, np.float32)
    m = np.full(n, m0, np.float32)
    with np.errstate(all="ignore"):
        P, M, V, B = oracle.adamw_step(p, m, v, np.zeros(n, np.uint16), step, **hp)
    return (digest(canonical_nan_f32(P)), digest(canonical_nan_f32(M)), digest(canonical_nan_f32(V)),
            digest(canonical_nan_bf16(B)))


def adamw_sweep_digests(tasks, workers=None):
    with _pool(workers) as ex:
        for r in ex.map(_adamw_sweep_digests, tasks, chunksize=1):
            yield r
