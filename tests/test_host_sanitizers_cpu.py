"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/host_sanitize.cpp is built with g++ together with plan.cpp, pieces.cpp,
schedule.cpp and status.cpp, with -fsanitize=address,undefined and no recovery, and run on the
workload lists (flat and Shard(0), the large ones checked through the ABI's
segment queries, the small ones element by element), 800 random lists, empty
and zero-sized tensors, argument errors and sizes that overflow int64. Any
sanitizer report or failed check ends the run with a non-zero status.
"""
import os
import shutil
import subprocess

import pytest

import synth
from test_store_span_cpu import GPT_13B, RAGGED, _spec

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "zero_partitioned_mixed_partition_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(f"{ROCM}/include/hip"),
                    reason="needs g++ and the HIP headers")
def test_host_code_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "host_sanitize")
    cmd = ["g++", "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", f"-I{ROCM}/include",
           "-D__HIP_PLATFORM_AMD__", f"-I{CSRC}", f"-I{os.path.join(ROOT, 'include')}",
           os.path.join(ROOT, "tests", "host_sanitize.cpp"), os.path.join(CSRC, "plan.cpp"),
           os.path.join(CSRC, "pieces.cpp"), os.path.join(CSRC, "schedule.cpp"),
           os.path.join(CSRC, "status.cpp"), "-o", exe,
           f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib"]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert b.returncode == 0, b.stderr[-3000:]
    specs = []
    for name in ("tiny-a", "tiny-b", "gpt2-small", "llama3-8b", "llama3-70b", "gpt-1.3b"):
        w = synth.WORKLOADS[name]
        specs += [_spec(0, w.shapes, w.n_ranks, w.align), _spec(1, w.shapes, w.n_ranks, w.align)]
    specs += [_spec(1, GPT_13B, 8), _spec(1, synth.WORKLOADS["llama3-70b"].shapes, 64),
              _spec(1, RAGGED, 2)]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], input="\n".join(specs) + "\n", capture_output=True, text=True,
                       timeout=900, env=env)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), (r.stdout[-3000:], r.stderr[-4000:])
