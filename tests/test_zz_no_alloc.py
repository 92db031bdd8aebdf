"""The reduce that allocates nothing (zero_grad_reduce_shard_noalloc) against
zero_grad_reduce_shard given a caller workspace of the same size as the
library's device array: calls in a row on one device, each smaller than the
one before, the bf16 output and the fp64 norm compared bit for bit; the
smallest also against the oracle, and one call without the norm. The array
keeps the previous call's partials, so each call must overwrite what it reads.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_bits_equal, dev, host_u16, needs_gpu, note

pytestmark = [pytest.mark.gpu, needs_gpu]


@pytest.fixture(scope="module")
def zm():
    import zero_partitioned_mixed_partition_amd as m
    torch.cuda.set_device(0)
    return m


def _replicas(n, R, seed, phi):
    reps = []
    for k in range(R):
        t = torch.empty(n, dtype=torch.int16, device=dev())
        synth.device_normal_bf16(t, seed, synth.KIND_REPLICA, 1, k, 0, phi, synth.GRAD_SIGMA)
        reps.append(t)
    return reps


def test_noalloc_reduce_equals_the_workspace_call(zm):
    ws = torch.empty(zm.ZERO_NOALLOC_SCRATCH_BYTES, dtype=torch.uint8, device=dev())
    # (numels, N_d, rank, replicas): the first window is past the array's
    # one-pass limit (the grid-stride kernel, 2,048 partials), the second takes
    # the one-pass kernel (about 45,000 partials), the third the grid-stride
    # kernel on a small window.
    cases = [([300_000_000, 5], 1, 0, 2),
             ([23_000_000, 777], 1, 0, 8),
             ([1_000_003, 4096, 3], 4, 3, 5)]
    for i, (numels, nd, rank, R) in enumerate(cases):
        plan = zm.zero_partition_plan(numels, nd, 128)
        P, S, phi = plan.padded_numel, plan.shard_numel, plan.numel
        note(f"noalloc reduce call {i}: P={P} S={S} rank={rank} R={R}")
        reps = _replicas(P, R, 60 + i, phi)
        out_a = torch.full((S,), 0x1111, dtype=torch.int16, device=dev())
        out_b = torch.full((S,), 0x2222, dtype=torch.int16, device=dev())
        sq = torch.full((2,), -1.0, dtype=torch.float64, device=dev())
        zm.zero_grad_reduce_shard(plan, rank, reps, 0, P, out_a, sqnorm_out=sq[0:1], workspace=ws)
        zm.zero_grad_reduce_shard_noalloc(plan, rank, reps, 0, P, out_b, sqnorm_out=sq[1:2])
        torch.cuda.synchronize()
        assert torch.equal(out_a, out_b), f"call {i}: bf16 output"
        a, b = sq.cpu().numpy()
        assert a == b and a > 0, f"call {i}: norm {a!r} against {b!r}"
        if i == len(cases) - 1:
            host = [synth.normal_bf16(P, 60 + i, synth.KIND_REPLICA, 1, k, 0, phi, synth.GRAD_SIGMA)
                    for k in range(R)]
            ref = oracle.partition_plan(numels, nd, 128)
            want = np.zeros(S, np.uint16)
            oracle.reduce_shard(ref, rank, host, 0, want)
            assert_bits_equal(host_u16(out_b), want, "small window against the oracle")
            exact = oracle.sqnorm(want)
            assert abs(b - exact) <= 1e-12 * exact, (b, exact)
            # without the norm: the output only, no scratch needed
            out_c = torch.full((S,), 0x3333, dtype=torch.int16, device=dev())
            zm.zero_grad_reduce_shard_noalloc(plan, rank, reps, 0, P, out_c)
            torch.cuda.synchronize()
            assert torch.equal(out_c, out_a), "no norm: bf16 output"
        del reps, out_a, out_b
        torch.cuda.empty_cache()
