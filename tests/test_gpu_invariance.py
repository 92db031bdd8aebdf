"""Shard invariance and degenerate inputs on the GPU path.

The model's flat buffer split over N_d ranks must give the same bits on
[0, Phi) whatever N_d is: every element's reduce and update depend only on
that element and the global clip coefficient ("ZeRO-Stage 1": each rank
updates its own slice with the same rule). Checked at N_d = 1, 2, 3, 8 and 64
through the C ABI, two steps with a device clip coefficient, then gathered.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_util import assert_bits_equal, dev, host_f32, host_u16, needs_gpu, note

pytestmark = [pytest.mark.gpu, needs_gpu]

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
NUMELS = [70_001, 3, 128 * 1024, 999, 50_000]


@pytest.fixture(scope="module")
def zm():
    import zero_partitioned_mixed_partition_amd as m
    torch.cuda.set_device(0)
    return m


def _run(zm, n_ranks, order=None):
    plan = zm.zero_partition_plan(NUMELS, n_ranks, 128)
    P, S, phi = plan.padded_numel, plan.shard_numel, plan.numel
    master = torch.empty(P, dtype=torch.float32, device=dev())
    synth.device_normal_f32(master, 7, synth.KIND_MASTER, 0, 0, 0, phi, 0.02)
    m = torch.zeros(P, dtype=torch.float32, device=dev())
    v = torch.zeros(P, dtype=torch.float32, device=dev())
    grad = torch.empty(P, dtype=torch.int16, device=dev())
    param = torch.empty(P, dtype=torch.int16, device=dev())
    scale = torch.tensor([0.375], dtype=torch.float32, device=dev())
    reps = [torch.empty(P, dtype=torch.int16, device=dev()) for _ in range(4)]
    for t in (1, 2):
        for k, r in enumerate(reps):
            synth.device_normal_bf16(r, 7, synth.KIND_REPLICA, t, k, 0, phi, 1e-3)
        for rank in (order if order is not None else range(n_ranks)):
            sl = slice(rank * S, (rank + 1) * S)
            zm.zero_grad_reduce_shard(plan, rank, reps, 0, P, grad[sl])
            zm.zero_shard_adamw_step(master[sl], m[sl], v[sl], grad[sl], param[sl], t,
                                     clip_scale=scale, **HP)
    tensors = [torch.empty(n, dtype=torch.int16, device=dev()) for n in NUMELS]
    zm.zero_gather_params(plan, [param[r * S:(r + 1) * S] for r in range(n_ranks)], tensors)
    torch.cuda.synchronize()
    return (host_f32(master)[:phi], host_f32(m)[:phi], host_f32(v)[:phi], host_u16(grad)[:phi],
            [host_u16(x) for x in tensors], host_f32(master)[phi:])


def test_shard_invariance_over_rank_counts(zm):
    base = _run(zm, 1)
    for n_ranks in (2, 3, 8, 64):
        note(f"invariance N_d={n_ranks}")
        got = _run(zm, n_ranks)
        for name, a, b in zip(("master", "exp_avg", "exp_avg_sq", "grad"), got[:4], base[:4]):
            assert_bits_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                              b.view(np.uint32) if b.dtype == np.float32 else b, f"{name} N_d={n_ranks}")
        for i, (a, b) in enumerate(zip(got[4], base[4])):
            assert_bits_equal(a, b, f"tensor {i} N_d={n_ranks}")
        assert (got[5] == 0).all(), "padding stays zero"


def test_empty_window_and_empty_tensors(zm):
    plan = zm.zero_partition_plan([1000, 0, 24], 4, 8)
    S = plan.shard_numel
    out = torch.full((S,), 77, dtype=torch.int16, device=dev())
    sq = torch.full((1,), -1.0, dtype=torch.float64, device=dev())
    rep = torch.ones(plan.padded_numel, dtype=torch.int16, device=dev())
    zm.zero_grad_reduce_shard(plan, 2, [rep], 0, 0, out, sqnorm_out=sq)   # empty window
    torch.cuda.synchronize()
    assert sq.item() == 0.0 and (out == 77).all()
    shards = [torch.full((S,), r + 1, dtype=torch.int16, device=dev()) for r in range(4)]
    tens = [torch.full((n,), -1, dtype=torch.int16, device=dev()) for n in (1000, 0, 24)]
    zm.zero_gather_params(plan, shards, tens)
    torch.cuda.synchronize()
    flat = np.concatenate([np.full(S, r + 1, np.uint16) for r in range(4)])
    assert_bits_equal(host_u16(tens[0]), flat[:1000], "tensor 0")
    assert_bits_equal(host_u16(tens[2]), flat[1000:1024], "tensor 2")
    empty = zm.zero_partition_plan([0, 0], 3, 128)
    assert empty.padded_numel == 0
    zm.zero_gather_params(empty, [torch.empty(0, dtype=torch.int16, device=dev())] * 3,
                          [torch.empty(0, dtype=torch.int16, device=dev())] * 2)
    zm.zero_flatten_params(empty, [torch.empty(0, dtype=torch.int16, device=dev())] * 2,
                           torch.empty(0, dtype=torch.int16, device=dev()))
    torch.cuda.synchronize()


def test_rank_results_do_not_depend_on_update_order(zm):
    """The emulated ranks share one device: each rank's reduce and update must
    depend only on its own slice, not on which ranks ran before it. Eight ranks
    updated in reverse and in a shuffled order give the bits of rank order."""
    base = _run(zm, 8)
    for order in (list(range(7, -1, -1)), [3, 6, 0, 5, 1, 7, 2, 4]):
        note(f"update order {order}")
        got = _run(zm, 8, order)
        for name, a, b in zip(("master", "exp_avg", "exp_avg_sq", "grad"), got[:4], base[:4]):
            assert_bits_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                              b.view(np.uint32) if b.dtype == np.float32 else b, f"{order} {name}")
        for i, (a, b) in enumerate(zip(got[4], base[4])):
            assert_bits_equal(a, b, f"{order} tensor {i}")
