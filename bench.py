"""Benchmark: one data-parallel rank's partitioned optimizer step on one MI355X.

Default workload: the GPT-2-small tensor list (148 tensors, 124,439,808
parameters) split over N_d = 8 ranks with 128-element alignment; the timed
rank is rank 7 (15,555,072-element shard). One step is the whole hot path:

  reduce   rank 7's slice of 8 bf16 gradient replicas (full flat buffers in
           HBM), averaged, with its squared-norm partial fused in
  clip     global-norm coefficient (max norm 1.0) from 8 partials on device
  adamw    fp32 master/m/v update of the shard, bf16 parameters emitted
  gather   8 bf16 parameter shards -> 148 per-tensor parameters

All inputs are seeded synthetic data resident in HBM before timing starts.
The other ranks' norm partials and parameter shards are inputs (computed
once, untimed, before the timed region): on a cluster they arrive through a
scalar all-reduce and the parameter all-gather.

Prints one JSON line. Only rank 0 at N = 1 exists: larger N is refused.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak
METRIC = "shard AdamW step: params/sec and achieved HBM GB/s (% of MI355X peak)"


def parse_args(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="gpt2-small",
                    choices=["gpt2-small", "gpt-1.3b-rank", "llama3-8b-rank"])
    ap.add_argument("--cpu-baseline-seconds", type=float, default=15.0,
                    help="rough budget for the oracle's host timing (0 disables it)")
    ap.add_argument("--profile-steps", type=int, default=0,
                    help="run only this many steps, untimed, for a profiler (no JSON)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="with --profile-steps: first copy 1 GiB once (a plain copy kernel of known "
                         "size, to scale hardware byte counters)")
    return ap.parse_args(argv)


class Setup:
    """Device buffers and inputs of one rank's step for a workload."""

    def __init__(self, name: str, device):
        import torch

        import synth
        import zero_partitioned_mixed_partition_amd as zm
        from zero_partitioned_mixed_partition_amd.step import Hyper, RankStep

        spec = {
            # name: (tensor list, N_d, rank, replicas, max_norm)
            "gpt2-small": ("gpt2-small", 8, 7, 8, 1.0),
            "gpt-1.3b-rank": ("gpt-1.3b", 8, 7, 8, 1.0),
            "llama3-8b-rank": ("llama3-8b", 64, 63, 8, 1.0),
        }[name]
        w = synth.WORKLOADS[spec[0]]
        self.name, self.workload = name, w
        self.n_ranks, self.rank, self.replicas, self.max_norm = spec[1], spec[2], spec[3], spec[4]
        self.seed = 1000 + w.seed
        self.device = device
        self.plan = zm.zero_partition_plan(w.numels, self.n_ranks, w.align)
        P, S, phi = self.plan.padded_numel, self.plan.shard_numel, self.plan.numel
        self.P, self.S, self.phi = P, S, phi
        self.hyper = Hyper(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                           weight_decay=w.weight_decay)
        self.rs = RankStep(self.plan, self.rank, 1, self.hyper, self.max_norm, device)

        # gradient replicas: full padded flat buffers, one per data-parallel replica
        self.reps = []
        for k in range(self.replicas):
            t = torch.empty(P, dtype=torch.int16, device=device)
            synth.device_normal_bf16(t, self.seed, synth.KIND_REPLICA, 1, k, 0, phi, synth.GRAD_SIGMA)
            self.reps.append(t)
        synth.device_normal_f32(self.rs.master, self.seed, synth.KIND_MASTER, 0, 0, self.rank * S, phi,
                                synth.MASTER_SIGMA)
        for r in range(self.n_ranks):
            if r != self.rank:
                synth.device_normal_bf16(self.rs.param_shards[r], self.seed, synth.KIND_PARAM, 0, 0,
                                         r * S, phi, synth.MASTER_SIGMA)
        # other ranks' squared-norm partials: their reduce, run once here
        tmp = torch.empty(S, dtype=torch.int16, device=device)
        parts = torch.zeros(self.n_ranks, dtype=torch.float64, device=device)
        for r in range(self.n_ranks):
            if r != self.rank:
                zm.zero_grad_reduce_shard(self.plan, r, self.reps, 0, P, tmp,
                                          sqnorm_out=parts[r:r + 1], workspace=self.rs.workspace)
        self.rs.partials[:self.n_ranks].copy_(parts)
        torch.cuda.synchronize()
        self.windows = [(0, P, self.reps)]

    def step(self):
        self.rs.step(self.windows)

    # algorithmic bytes per step of each kernel (what the method must move)
    def bytes_per_kernel(self):
        S, R = self.S, self.replicas
        return {"reduce": (2 * R + 2) * S, "clip": 8 * (self.n_ranks + 1) + 4,
                "adamw": 28 * S, "gather": 4 * self.phi}


def time_kernels(setup: "Setup", steps: int):
    """Per-kernel mean duration (ms) from HIP events on the launch stream."""
    import torch
    names = ["reduce", "clip", "adamw", "gather"]
    calls = {"reduce": lambda: setup.rs.reduce(setup.windows), "clip": setup.rs.clip,
             "adamw": setup.rs.adamw, "gather": setup.rs.gather}
    ev = {n: [] for n in names}
    for _ in range(steps):
        for n in names:
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            calls[n]()
            b.record()
            ev[n].append((a, b))
    torch.cuda.synchronize()
    return {n: sum(a.elapsed_time(b) for a, b in ev[n]) / len(ev[n]) for n in names}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "adamw_traffic.json")
ADAMW_SOURCES = [os.path.join(ROOT, "zero_partitioned_mixed_partition_amd", "csrc", f)
                 for f in ("adamw.hip", "device_common.hpp")]


def kernel_source_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in ADAMW_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def measured_traffic(setup: "Setup"):
    """HBM bytes per AdamW launch from the committed counter runs (FETCH_SIZE and
    WRITE_SIZE, scaled by a 1 GiB copy), or None when the kernel sources have
    changed since they were taken or they cover another shard size."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    d = json.load(open(TRAFFIC_FILE))
    if d.get("source_sha256") != kernel_source_digest() or d.get("elems") != setup.S:
        return None
    return d["bytes_per_launch"]


def cpu_baseline(setup: "Setup", budget_s: float):
    """The oracle's rank step on the host for the same workload, bounded in time."""
    import numpy as np

    import oracle
    import synth
    P, S, phi, rank = setup.P, setup.S, setup.phi, setup.rank
    ref = oracle.partition_plan(setup.workload.numels, setup.n_ranks, setup.workload.align)
    lo = rank * S
    # the oracle needs only the rank's window of each replica for its reduce
    reps = [synth.normal_bf16(S, setup.seed, synth.KIND_REPLICA, 1, k, lo, phi, synth.GRAD_SIGMA)
            for k in range(setup.replicas)]
    state = {"master": synth.normal_f32(S, setup.seed, synth.KIND_MASTER, 0, 0, lo, phi,
                                        synth.MASTER_SIGMA),
             "exp_avg": np.zeros(S, np.float32), "exp_avg_sq": np.zeros(S, np.float32)}
    shards = [synth.normal_bf16(S, setup.seed, synth.KIND_PARAM, 0, 0, r * S, phi, synth.MASTER_SIGMA)
              for r in range(setup.n_ranks)]
    partials = [1.0] * setup.n_ranks
    hp = dict(lr=setup.hyper.lr, beta1=setup.hyper.beta1, beta2=setup.hyper.beta2,
              eps=setup.hyper.eps, weight_decay=setup.hyper.weight_decay)
    # one untimed step first: the first touch of fresh host pages is not oracle work
    oracle.rank_step(ref, rank, reps, lo, state, shards, partials, 1, hp, setup.max_norm)
    t0 = time.perf_counter()
    n = 0
    while True:
        n += 1
        oracle.rank_step(ref, rank, reps, lo, state, shards, partials, 1 + n, hp, setup.max_norm)
        el = time.perf_counter() - t0
        if el >= budget_s or n >= 50:
            break
    return {"value": S * n / el, "unit": "params/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} full rank-{rank} steps of the same workload (reduce of "
                      f"{setup.replicas} replica windows, exact norm, clip, AdamW on "
                      f"{S} elements, gather of {phi} parameters), single-threaded numpy",
            "seconds": el, "host_cpus": len(os.sched_getaffinity(0))}


def main(argv=None):
    args = parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(the per-rank step is measured on one GPU's share)", file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 2
    device = torch.device("cuda:0")
    torch.cuda.set_device(device)
    print(f"[bench] setting up {args.workload}", file=sys.stderr, flush=True)
    setup = Setup(args.workload, device)
    if args.profile_steps:
        if args.calibrate_copy:
            src = torch.ones(1 << 28, dtype=torch.float32, device=device)
            dst = torch.empty_like(src)
            torch.cuda.synchronize()
            dst.copy_(src)                      # reads 1 GiB, writes 1 GiB
            torch.cuda.synchronize()
            del src, dst
        for _ in range(args.profile_steps):
            setup.step()
        torch.cuda.synchronize()
        print(f"[bench] ran {args.profile_steps} steps for profiling", file=sys.stderr, flush=True)
        return 0

    for _ in range(args.warmup):
        setup.step()
    torch.cuda.synchronize()
    # Timed region: whole steps; AdamW is bracketed by events on the stream it is
    # launched on (torch's current stream, which every call here uses).
    adamw_ev = []
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        setup.rs.reduce(setup.windows)
        setup.rs.clip()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        setup.rs.adamw()
        b.record()
        adamw_ev.append((a, b))
        setup.rs.gather()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = start.elapsed_time(end) / args.steps
    adamw_ms = sum(a.elapsed_time(b) for a, b in adamw_ev) / len(adamw_ev)
    print(f"[bench] {args.steps} steps: {ms_per_step:.4f} ms/step (wall {wall:.3f} s), "
          f"adamw {adamw_ms * 1e3:.1f} us", file=sys.stderr, flush=True)

    kernel_ms = time_kernels(setup, max(20, min(args.steps, 200)))
    kernel_ms["adamw"] = adamw_ms
    bpk = setup.bytes_per_kernel()
    kernels = {n: {"ms": kernel_ms[n], "bytes": bpk[n],
                   "gbs": bpk[n] / (kernel_ms[n] * 1e-3) / 1e9,
                   "frac_of_hbm_peak": bpk[n] / (kernel_ms[n] * 1e-3) / 1e9 / HBM_PEAK_GBS}
               for n in kernel_ms}
    step_bytes = sum(bpk.values())
    adamw_gbs = kernels["adamw"]["gbs"]
    value = setup.S / (ms_per_step * 1e-3)
    traffic = measured_traffic(setup)

    cpu = None
    if args.cpu_baseline_seconds > 0:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        cpu = cpu_baseline(setup, args.cpu_baseline_seconds)

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{setup.workload.name} tensor list, N_d={setup.n_ranks}, "
                               f"rank {setup.rank} shard of {setup.S} elements; step = reduce of "
                               f"{setup.replicas} bf16 replicas + sqnorm + clip {setup.max_norm} + "
                               f"AdamW + gather of {len(setup.workload.numels)} tensors",
                   "params": setup.phi, "shard_elems": setup.S, "n_ranks": setup.n_ranks,
                   "replicas": setup.replicas, "parallelism": "one rank of dp8 (one GPU)"},
        "adamw_params_per_s": setup.S / (kernels["adamw"]["ms"] * 1e-3),
        "adamw_hbm_gbs": adamw_gbs,
        "adamw_frac_of_hbm_peak": adamw_gbs / HBM_PEAK_GBS,
        "step_hbm_gbs": step_bytes / (ms_per_step * 1e-3) / 1e9,
        "kernels": kernels,
        "roofline": {"bound": "hbm", "kernel": "adamw_kernel", "achieved": adamw_gbs,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": adamw_gbs / HBM_PEAK_GBS,
                     "traffic": traffic},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
