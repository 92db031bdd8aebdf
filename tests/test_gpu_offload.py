"""GPU parity of the ZeRO-Offload step: device gradients to the host, the
host update, parameters back to the device, in overlapped chunks."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_bits_equal, dev, host_u16, needs_gpu, note, to_dev_u16

pytestmark = [pytest.mark.gpu, needs_gpu]

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


@pytest.fixture(scope="module")
def zm():
    import zero_partitioned_mixed_partition_amd as m
    torch.cuda.set_device(0)
    return m


@pytest.mark.parametrize("n,chunk", [(5_000_003, 1 << 20), (1000, 257), (4096, 1 << 20)])
def test_offload_matches_oracle(zm, n, chunk):
    note(f"offload n={n} chunk={chunk}")
    p = synth.normal_f32(n, 61, synth.KIND_MASTER, 0, 0, sigma=0.02)
    hp = torch.from_numpy(p.copy())
    hm = torch.zeros(n, dtype=torch.float32)
    hv = torch.zeros(n, dtype=torch.float32)
    staging = torch.empty(4 * chunk, dtype=torch.int16).pin_memory()
    d_grad = torch.empty(n, dtype=torch.int16, device=dev())
    d_param = torch.zeros(n, dtype=torch.int16, device=dev())
    d_scale = torch.tensor([0.61], dtype=torch.float32, device=dev())
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    bits = None
    for t in (1, 2, 3):
        synth.device_normal_bf16(d_grad, 61, synth.KIND_GRAD, t, 0, 0, n, 1e-3)
        zm.zero_offload_adamw_step(hp, hm, hv, d_grad, d_param, staging, t, clip_scale=d_scale, **HP)
        g = synth.normal_bf16(n, 61, synth.KIND_GRAD, t, 0, 0, n, 1e-3)
        p, m, v, bits = oracle.adamw_step(p, m, v, g, t, clip=np.float32(0.61), **HP)
    torch.cuda.synchronize()
    assert_bits_equal(hp.numpy().view(np.uint32), p.view(np.uint32), "host master")
    assert_bits_equal(hm.numpy().view(np.uint32), m.view(np.uint32), "host exp_avg")
    assert_bits_equal(hv.numpy().view(np.uint32), v.view(np.uint32), "host exp_avg_sq")
    assert_bits_equal(host_u16(d_param), bits, "device params")


def test_offload_orders_with_the_stream_and_skips_nonfinite(zm):
    n = 300_000
    p = synth.normal_f32(n, 62, synth.KIND_MASTER, 0, 0, sigma=0.02)
    hp = torch.from_numpy(p.copy())
    hm = torch.zeros(n, dtype=torch.float32)
    hv = torch.zeros(n, dtype=torch.float32)
    staging = torch.empty(4 * 65536, dtype=torch.int16).pin_memory()
    g = synth.normal_bf16(n, 62, synth.KIND_GRAD, 1, 0, 0, n, 1e-3)
    d_grad = torch.zeros(n, dtype=torch.int16, device=dev())
    d_param = torch.zeros(n, dtype=torch.int16, device=dev())
    # the gradient lands on the stream right before the step: the step must see it
    d_grad.copy_(to_dev_u16(g), non_blocking=True)
    zm.zero_offload_adamw_step(hp, hm, hv, d_grad, d_param, staging, 1, **HP)
    after = d_param.clone()              # ordered after the parameter copies on the stream
    torch.cuda.synchronize()
    P, M, V, B = oracle.adamw_step(p, np.zeros(n, np.float32), np.zeros(n, np.float32), g, 1, **HP)
    assert_bits_equal(hp.numpy().view(np.uint32), P.view(np.uint32), "master")
    assert_bits_equal(host_u16(after), B, "params seen by later stream work")
    nan = torch.tensor([float("nan")], dtype=torch.float32, device=dev())
    before = hp.clone()
    zm.zero_offload_adamw_step(hp, hm, hv, d_grad, d_param, staging, 2, clip_scale=nan, **HP)
    assert torch.equal(before, hp)
