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
