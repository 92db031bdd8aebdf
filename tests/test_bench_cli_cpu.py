"""bench.py's command-line contract on the CPU: one GPU only, the workloads it
names, and the traffic record's lookup (no GPU needed for any of these)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, cwd=ROOT)


@pytest.mark.parametrize("n", ["2", "8"])
def test_more_than_one_gpu_is_refused_with_a_message(n):
    r = _run("--gpus", n)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_unknown_workload_is_refused():
    r = _run("--workload", "no-such-model")
    assert r.returncode != 0 and "invalid choice" in r.stderr


def test_every_workload_has_default_steps_and_a_description_path():
    sys.path.insert(0, ROOT)
    import bench
    assert set(bench.DEFAULT_STEPS) == set(bench.WORKLOAD_NAMES)
    assert bench.parse_args([]).workload == "llama3-70b"
    assert bench.parse_args([]).device_step is False           # the benchmark's line: host step
    assert bench.parse_args(["--device-step"]).device_step is True
    for name in bench.WORKLOAD_NAMES:
        steps, warmup = bench.DEFAULT_STEPS[name]
        assert steps >= 1 and 0 <= warmup <= steps


def test_traffic_record_matches_sources_and_sizes():
    """Each committed traffic entry names its kernel, its element count and the
    digest of the AdamW sources it was taken with; measured_traffic returns an
    entry only for the current sources, so a changed kernel reads as null."""
    sys.path.insert(0, ROOT)
    import bench
    d = json.load(open(bench.TRAFFIC_FILE))
    digest = bench.kernel_source_digest()
    for e in d["runs"]:
        assert {"kernel", "elems", "bytes_per_launch", "algorithmic_bytes", "source_sha256"} <= set(e)
        assert 0.99 < e["bytes_per_launch"] / e["algorithmic_bytes"] < 1.01
        got = bench.measured_traffic(e["elems"], e["kernel"])
        assert got == (e["bytes_per_launch"] if e["source_sha256"] == digest else None)
    assert bench.measured_traffic(12345) is None


@pytest.mark.parametrize("replicas,max_norm", [(0, 1.0), (8, 1.0), (8, 0.0)])
def test_cpu_baseline_reports_its_sample_and_core_count(replicas, max_norm):
    """The cpu_baseline leg on a small stand-in workload (the attributes it
    reads, no device): one pass at least, a readable sample naming the count and
    the work (the norm and clip only where the workload clips), one core."""
    import types
    sys.path.insert(0, ROOT)
    import bench
    import synth
    from zero_partitioned_mixed_partition_amd.step import Hyper
    w = synth.WORKLOADS["tiny-a"]
    wl = types.SimpleNamespace(name="stand-in", hyper=Hyper(), S=4096, rank=1, seed=7,
                               phi=w.numel if hasattr(w, "numel") else sum(w.numels),
                               replicas=replicas, max_norm=max_norm)
    r = bench.cpu_baseline(wl, 0.0)
    assert r["kind"] == "oracle" and r["unit"] == "params/s" and r["cores"] == 1
    assert r["value"] > 0 and r["seconds"] > 0
    count, rest = r["sample"].split(" ", 1)
    assert int(count) >= 1 and rest.startswith("passes of the per-element work")
    assert ("reduce of 8 replica windows" in rest) == (replicas == 8)
    assert ("clip" in rest) == (max_norm > 0)
