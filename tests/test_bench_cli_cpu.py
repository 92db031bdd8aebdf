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


def _counter_csv(folder, counter, rows):
    """A rocprofv3-style counter_collection.csv: (dispatch, kernel, KiB) rows,
    each dispatch split over two channel rows as the real files are."""
    import csv
    folder.mkdir(parents=True)
    with open(folder / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for d, name, kib in rows:
            w.writerow([d, name, counter, kib / 2])
            w.writerow([d, name, counter, kib / 2])


@pytest.mark.parametrize("workload,steps,launches", [("gpt-1.3b", 1, 8), ("gpt2-small", 2, 1)])
def test_write_traffic_takes_bytes_per_launch(tmp_path, monkeypatch, workload, steps, launches):
    """--write-traffic on synthetic counter files: reads scaled by the 1 GiB
    copy's FETCH_SIZE (which reads it as half), writes by its WRITE_SIZE, and
    the entry's bytes are per AdamW launch (the mean over the profiled
    dispatches), whatever the launches per step."""
    sys.path.insert(0, ROOT)
    import bench
    import synth
    import zero_partitioned_mixed_partition_amd as zm
    w = synth.WORKLOADS[workload]
    S = zm.zero_partition_plan(w.numels, w.n_ranks, w.align).shard_numel
    kib = 28 * S / 1024 / 2          # each direction, before scaling
    copy = "__amd_rocclr_copyBuffer"
    n = steps * launches
    fetch = [(0, copy, float(1 << 19))] + [(1 + i, "adamw_kernel(float*)", kib / 2) for i in range(n)]
    write = [(0, copy, float(1 << 20))] + [(1 + i, "adamw_kernel(float*)", kib) for i in range(n)]
    _counter_csv(tmp_path / "fetch", "FETCH_SIZE", fetch)
    _counter_csv(tmp_path / "write", "WRITE_SIZE", write)
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    args = bench.parse_args(["--workload", workload, "--profile-steps", str(steps), "--write-traffic",
                             str(tmp_path / "fetch"), str(tmp_path / "write")])
    assert bench.write_traffic(args) == 0
    (e,) = json.load(open(out))["runs"]
    assert e["elems"] == S and e["dispatches_per_call"] == launches
    assert e["fetch_scale"] == 2.0 and e["write_scale"] == 1.0
    assert e["bytes_per_launch"] == pytest.approx(28 * S, rel=1e-12)
    assert e["algorithmic_bytes"] == 28 * S
