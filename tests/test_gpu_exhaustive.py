"""AdamW's fp32 square root and divisions over every float32 second moment.

The kernel's per-element arithmetic includes sqrt(v), a division by
sqrt(1 - beta2^t) and the ratio m / denom, each an IEEE correctly rounded fp32
operation (no fast-math, no contraction). With a zero gradient the update gives
v = beta2 * v_old; beta2 = 0.5 makes that v_old / 2, exact except where the
halving rounds a subnormal. Running the fused AdamW step on all 2^32 float32
bit patterns of v_old (in 2^26-element chunks) therefore feeds the square root
and both divisions essentially every float32 input, and the bf16 emit the
resulting parameters; the master, both moments and the bf16 parameters are
compared with the oracle (numpy's correctly rounded float32 operations) bit for
bit, by digest per chunk, with NaNs canonicalised (IEEE leaves the sign of
sqrt of a negative number open). [ZF] "Static Memory Allocation" (fp32 m_t,
v_t); the update's reading is the oracle's.
"""
import numpy as np
import pytest
import torch

from gpu_util import dev, host_f32, host_u16, needs_gpu, note

pytestmark = [pytest.mark.gpu, needs_gpu]

HP = dict(lr=1e-3, beta1=0.9, beta2=0.5, eps=1e-8, weight_decay=0.01)
CHUNK = 1 << 26
P0, M0 = 1.0, 1.0


@pytest.fixture(scope="module")
def zm():
    import zero_partitioned_mixed_partition_amd as m
    torch.cuda.set_device(0)
    return m


def test_adamw_over_every_float32_second_moment(zm):
    from oracle_workers import (adamw_sweep_digests, canonical_nan_bf16, canonical_nan_f32,
                                digest)
    total = 1 << 32
    starts = list(range(0, total, CHUNK))
    note(f"adamw sweep: {total} second moments in {len(starts)} chunks; oracle in a process pool")
    want = adamw_sweep_digests([(lo, CHUNK, P0, M0, 1, HP) for lo in starts], workers=12)
    base = torch.arange(CHUNK, dtype=torch.int64, device=dev())
    p = torch.empty(CHUNK, dtype=torch.float32, device=dev())
    m = torch.empty(CHUNK, dtype=torch.float32, device=dev())
    g = torch.zeros(CHUNK, dtype=torch.int16, device=dev())
    out = torch.empty(CHUNK, dtype=torch.int16, device=dev())
    names = ("master", "exp_avg", "exp_avg_sq", "param")
    for i, (lo, w) in enumerate(zip(starts, want)):
        x = (base + lo) & 0xFFFFFFFF                  # bit patterns lo .. lo + CHUNK - 1
        v = torch.where(x >= 1 << 31, x - (1 << 32), x).to(torch.int32).view(torch.float32)
        p.fill_(P0)
        m.fill_(M0)
        zm.zero_shard_adamw_step(p, m, v, g, out, 1, **HP)
        torch.cuda.synchronize()
        got = (digest(canonical_nan_f32(host_f32(p))), digest(canonical_nan_f32(host_f32(m))),
               digest(canonical_nan_f32(host_f32(v))), digest(canonical_nan_bf16(host_u16(out))))
        for name, a, b in zip(names, got, w):
            assert a == b, f"{name} differs from the oracle for bit patterns [{lo:#x}, {lo + CHUNK:#x})"
        if i % 16 == 15:
            note(f"adamw sweep: {i + 1} of {len(starts)} chunks bit-identical")
