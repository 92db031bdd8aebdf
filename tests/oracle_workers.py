"""Process-pool helpers that run oracle computations over generated inputs.

Imported by spawned worker processes: numpy, the generator and the oracle only.
"""
import os
from concurrent.futures import ProcessPoolExecutor
import multiprocessing as mp


def _init(threads: int) -> None:
    os.environ["OMP_NUM_THREADS"] = str(threads)


def _grad_slice_sqnorm(args):
    import oracle
    import synth
    seed, kind, step, replica, g0, n, phi, sigma = args
    bits = synth.normal_bf16(n, seed, kind, step, replica, g0, phi, sigma)
    return oracle.sqnorm(bits)


def grad_sqnorms(tasks, workers=None):
    """tasks: (seed, kind, step, replica, g0, n, phi, sigma) per generated gradient
    slice; returns the oracle's exact squared norm of each, in task order."""
    workers = workers or max(1, min(8, (os.cpu_count() or 2) // 2))
    ctx = mp.get_context("spawn")
    with ProcessPoolExecutor(max_workers=workers, mp_context=ctx, initializer=_init,
                             initargs=(2,)) as ex:
        return list(ex.map(_grad_slice_sqnorm, tasks, chunksize=1))
