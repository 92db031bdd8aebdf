"""Every kernel's per-wave store addresses, modelled on the CPU.

The kernels' streaming stores are buffer stores: a 64-bit base that is the
same for every lane of a wave, plus a 32-bit offset per lane. The common form
(st_stream) takes the first active lane's address less 2 GiB as the base, so
every lane of a wave must store within 2 GiB of that lane; the Shard(0)
flatten, whose waves can store into two rank buffers S elements apart, passes
each rank's own base instead (st_stream_at). tests/host_store_span.cpp runs the
tensor-major copy's real index map and routing (tensor_major.hpp) on plans from
the real planner (plan.cpp), and the contiguous kernels' index formulas, and
checks each store form's contract, wave by wave, on:
  - the five workload lists, flat (FSDP-1 / ZeRO) at their N_d and Shard(0)
    (FSDP-2, "FSDP-2: Per-Parameter Sharding via DTensor (fully_shard)"),
  - a 13B-class GPT list (d = 5120, 40 layers) under Shard(0) at N_d = 8,
    whose shards hold 1.6e9 elements, and the Llama-3-70B list under Shard(0)
    at N_d = 64.
It also reports the span the flatten's waves would have had under the common
form: on the 13B list that span passes 2^31 bytes, which is the case the
per-rank base exists for, so the model would catch a return to it.
"""
import os
import re
import shutil
import subprocess

import pytest

import synth
from synth import models

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "zero_partitioned_mixed_partition_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

GPT_13B = models.gpt2(5120, 40, 50257, 2048, 20480)
# Large chunks whose length is a multiple of 8 elements (so lanes on both sides
# of a boundary take whole 16-byte accesses) but not of a wave's 512, so waves
# cross the boundaries of large chunks too: at N_d = 2 the three big tensors'
# chunks hold 538,974,232 elements each, so the per-rank offsets pass 2^30
# bytes, and a wave across one big tensor's boundary spans the other chunks of
# the rank buffer, 2^31 bytes or more.
RAGGED = [(2 * 262147, 2056), (3001,), (2 * 262147, 2056), (7, 4097), (2 * 262147, 2056),
          (40001, 1234), (5,)]


def _spec(kind: int, shapes, n_ranks: int, align: int = 128) -> str:
    lines = [f"plan {kind} {n_ranks} {align} {len(shapes)}"]
    for s in shapes:
        n = 1
        for d in s:
            n *= d
        lines.append(f"{n} {s[0] if s else 1}")
    return "\n".join(lines)


def _cases():
    cases = []
    for name in ("tiny-a", "tiny-b", "gpt2-small", "llama3-8b", "llama3-70b", "gpt-1.3b"):
        w = synth.WORKLOADS[name]
        cases.append((f"{name} flat", _spec(0, w.shapes, w.n_ranks, w.align)))
        cases.append((f"{name} shard0", _spec(1, w.shapes, w.n_ranks, w.align)))
    cases.append(("gpt-13b shard0 N_d=8", _spec(1, GPT_13B, 8)))
    cases.append(("gpt-13b flat N_d=8", _spec(0, GPT_13B, 8)))
    cases.append(("llama3-70b shard0 N_d=64", _spec(1, synth.WORKLOADS["llama3-70b"].shapes, 64)))
    cases.append(("ragged shard0 N_d=2", _spec(1, RAGGED, 2)))
    cases.append(("ragged shard0 N_d=8", _spec(1, [RAGGED[1], RAGGED[3]] + RAGGED[5:], 8)))
    return cases


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    if shutil.which("g++") is None or not os.path.exists(f"{ROCM}/include/hip"):
        pytest.skip("needs g++ and the HIP headers")
    exe = str(tmp_path_factory.mktemp("span") / "store_span")
    cmd = ["g++", "-O2", "-std=c++17", f"-I{ROCM}/include", "-D__HIP_PLATFORM_AMD__", f"-I{CSRC}",
           f"-I{os.path.join(ROOT, 'include')}", os.path.join(ROOT, "tests", "host_store_span.cpp"),
           os.path.join(CSRC, "plan.cpp"), os.path.join(CSRC, "status.cpp"), "-o", exe,
           f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib"]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert b.returncode == 0, b.stderr[-3000:]
    return exe


def test_every_wave_keeps_its_store_form_contract(harness):
    cases = _cases()
    r = subprocess.run([harness], input="\n".join(s for _, s in cases) + "\n", capture_output=True,
                       text=True, timeout=900)
    out = r.stdout.strip().splitlines()
    assert r.returncode == 0 and out and out[-1] == "ok", (r.stdout[-3000:], r.stderr[-2000:])
    rows = {}
    for (label, _), line in zip(cases, out[:-1]):
        kv = dict(re.findall(r"(\w+)=(\S+)", line))
        rows[label] = kv
        assert int(kv["first_lane_span"]) <= 1024, (label, line)   # one run of <= 64 x 16 bytes
        assert int(kv["at_max_end"]) < 1 << 32, (label, line)
    # The Shard(0) lists take the tensor-major kernel (their tensors are < 2^31
    # elements, at most 64 ranks), and its flatten's waves do cross rank buffers.
    for label in ("gpt2-small shard0", "gpt-13b shard0 N_d=8", "llama3-70b shard0 N_d=64",
                  "ragged shard0 N_d=2", "ragged shard0 N_d=8"):
        assert rows[label]["route"].startswith("tensor-major"), (label, rows[label])
        assert int(rows[label]["elems"]) > 0
    # 13B-class under Shard(0) at N_d = 8: S = 1,606,677,760 elements, and a wave
    # crossing a [5120] norm's 640-element chunk boundary spans about 2 S bytes, past
    # what the first-lane form can address.
    big = rows["gpt-13b shard0 N_d=8"]
    assert int(big["S"]) == 1_606_677_760
    assert int(big["old_form_span"]) > 1 << 31
    assert int(rows["llama3-70b shard0 N_d=64"]["old_form_span"]) > 1 << 31
    # ragged rows: waves cross large chunks' boundaries, at per-rank offsets past 2^30 bytes
    assert int(rows["ragged shard0 N_d=2"]["at_max_end"]) > 1 << 30
    assert int(rows["ragged shard0 N_d=2"]["old_form_span"]) > 1 << 31
