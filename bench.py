"""Benchmark: the data-parallel rank's partitioned optimizer step on one MI355X.

Default workload (`llama3-70b`): the Llama-3-70B tensor list (723 tensors,
70,553,706,496 parameters) split over N_d = 8 ranks with 128-element alignment;
the timed rank is rank 7 (8,819,213,312-element shard, its fp32 state and bf16
gradient and parameters resident in HBM, about 141 GB). The gradients arrive
already averaged (the configuration's stated form), so one step is:

  sqnorm   the shard's squared-norm partial (fp64, one pass)
  clip     global-norm coefficient (max norm 1.0) from every rank's partial
  adamw    fp32 master/m/v update of the shard, bf16 parameters emitted

Other workloads (`--workload`), each timed as its own configuration states:
  gpt2-small  rank 7 of 8 of the GPT-2-small list (148 tensors, 124,439,808
              parameters, 15,555,072-element shard): reduce of 8 bf16 replicas
              (full flat buffers in HBM) with the fused squared norm, clip 1.0,
              AdamW, gather of the 8 shards to 148 tensors through a
              device-resident copy table (the call-based gather timed beside it)
  llama3-8b   rank 63 of 64: six 25M-element buckets of 64 replicas reduced
              into the 125,472,896-element shard, clip 1.0, AdamW
  gpt-1.3b    all 8 ranks of the 1.3B GPT list: 8 replicas reduced for every
              rank, AdamW on every shard, gather to 292 tensors (the job does
              not clip, so no squared norm is computed)
  gpt-1.3b-fused  the same with each rank's reduce and AdamW in one pass
              (zero_reduce_adamw_step)
  gpt2-small-fsdp2  the gpt2-small step on FSDP-2's per-parameter Shard(0) layout
              (every tensor cut along dim 0; a rank's chunks in one coalesced
              buffer); the replicas are per-tensor gradients flattened into it
              (one replica's flatten is also timed, outside the step)
  gpt2-small-fsdp2-pertensor  the Shard(0) step with per-parameter optimizer
              state: every local chunk has its own fp32 tensors, updated by the
              multi-tensor AdamW over the ragged list (its device-resident
              table in the step; the list call timed beside it)
  gpt2-small-offload  the gpt2-small step with ZeRO-Offload's update: the fp32
              master/m/v live in host DRAM; the shard's bf16 gradients go to
              the host, the host runs AdamW, the bf16 parameters come back, in
              overlapped chunks (reduce, clip and gather stay on the GPU)

`--also W ...` measures further workloads after the line's and reports them
under the line's "also" key (summaries: step, AdamW events, kernels, traffic).

All inputs are seeded synthetic data resident in HBM before timing starts. The
other ranks' norm partials and parameter shards are inputs computed once,
untimed (on a cluster they arrive through a scalar all-reduce and the
parameter all-gather). Prints one JSON line. One GPU only: --gpus > 1 is refused.
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak
METRIC = "shard AdamW step: params/sec and achieved HBM GB/s (% of MI355X peak)"
WORKLOAD_NAMES = ["gpt2-small", "llama3-8b", "llama3-70b", "gpt-1.3b", "gpt-1.3b-fused",
                  "gpt2-small-fsdp2", "gpt2-small-offload", "gpt2-small-fsdp2-pertensor"]
PCIE_PEAK_GBS = 128.0          # PCIe 5.0 x16, both directions together (64 GB/s each way)
OFFLOAD_CHUNK = 1 << 21        # elements per staging slot of the offload pipeline


def parse_args(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: 200, or fewer for the large workloads)")
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="llama3-70b", choices=WORKLOAD_NAMES)
    ap.add_argument("--cpu-baseline-seconds", type=float, default=15.0,
                    help="rough budget for the oracle's host timing (0 disables it)")
    ap.add_argument("--profile-steps", type=int, default=0,
                    help="run only this many steps, untimed, for a profiler (no JSON)")
    ap.add_argument("--device-step", action="store_true",
                    help="count AdamW's step on the device (RankStep(device_step=True)): the "
                         "scheduled update kernels, the AdamW phase including the one-lane "
                         "advance; a comparison run, not the benchmark's line")
    ap.add_argument("--profile-extra", action="store_true",
                    help="with --profile-steps: first run each phase timed outside the step once "
                         "(the step's dispatches stay the run's last ones)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="with --profile-steps: first copy 1 GiB once (a plain copy kernel of known "
                         "size, to scale hardware byte counters)")
    ap.add_argument("--also", nargs="*", default=None, choices=WORKLOAD_NAMES, metavar="WORKLOAD",
                    help="after the line's workload, measure these too (their figures go under "
                         "'also')")
    ap.add_argument("--stagger", type=int, default=None, metavar="BYTES",
                    help="gap between consecutive arrays of an arena and between replica buffers "
                         "(default: the step module's STAGGER; 0 packs them end to end at "
                         "256-byte-aligned starts)")
    ap.add_argument("--separate-arrays", action="store_true",
                    help="give every state array and replica buffer an allocation of its own "
                         "instead of one staggered arena (a layout comparison)")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU: read two rocprofv3 --pmc output folders (FETCH_SIZE, WRITE_SIZE) "
                         "of a '--profile-steps N --calibrate-copy' run of this workload, and record "
                         "the AdamW call's HBM bytes in profiles/adamw_traffic.json")
    return ap.parse_args(argv)


DEFAULT_STEPS = {"gpt2-small": (200, 20), "llama3-8b": (20, 3), "llama3-70b": (5, 1),
                 "gpt-1.3b": (10, 2), "gpt-1.3b-fused": (10, 2), "gpt2-small-fsdp2": (200, 20),
                 "gpt2-small-offload": (30, 3), "gpt2-small-fsdp2-pertensor": (200, 20)}


class RankWorkload:
    """One rank's step: reduce (or plain squared norm), clip, AdamW, optional gather."""

    SPECS = {
        # name: tensor list, N_d, rank, replicas (0: gradients arrive averaged), bucket, gather,
        # layout (flat: FSDP-1 / ZeRO; shard0: FSDP-2 per-parameter)
        "gpt2-small": ("gpt2-small", 8, 7, 8, 0, True, "flat"),
        "llama3-8b": ("llama3-8b", 64, 63, 64, 25_000_000, False, "flat"),
        "llama3-70b": ("llama3-70b", 8, 7, 0, 0, False, "flat"),
        "gpt2-small-fsdp2": ("gpt2-small", 8, 7, 8, 0, True, "shard0"),
        "gpt2-small-offload": ("gpt2-small", 8, 7, 8, 0, True, "flat"),
        "gpt2-small-fsdp2-pertensor": ("gpt2-small", 8, 7, 8, 0, True, "shard0"),
    }

    def __init__(self, name: str, device, device_step: bool = False):
        import torch

        import synth
        import zero_partitioned_mixed_partition_amd as zm
        from zero_partitioned_mixed_partition_amd.step import (Hyper, RankStep, bucket_windows,
                                                               staggered_replicas)

        lst, nd, rank, reps, bucket, gather, layout = self.SPECS[name]
        w = synth.WORKLOADS[lst]
        self.name, self.workload, self.device, self.layout = name, w, device, layout
        self.n_ranks, self.rank, self.replicas, self.bucket = nd, rank, reps, bucket
        self.max_norm = w.max_norm if w.max_norm > 0 else 1.0
        self.seed = 1000 + w.seed
        if layout == "shard0":
            self.plan = zm.zero_partition_plan_shard0(w.numels, [s[0] for s in w.shapes], nd,
                                                      w.align)
        else:
            self.plan = zm.zero_partition_plan(w.numels, nd, w.align)
        P, S, phi = self.plan.padded_numel, self.plan.shard_numel, self.plan.numel
        self.P, self.S, self.phi = P, S, phi
        lo = rank * S
        self.hyper = Hyper(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                           weight_decay=w.weight_decay)
        spans = bucket_windows(P, bucket, lo, lo + S) if reps else []
        self.offload = name.endswith("-offload")
        self.n_threads = len(os.sched_getaffinity(0))
        self.per_tensor = name.endswith("-pertensor")
        if device_step and self.offload:
            raise SystemExit("bench.py: --device-step takes device state; not with the offload workload")
        self.rs = RankStep(self.plan, rank, len(spans), self.hyper, self.max_norm, device,
                           gather=gather, offload=self.offload, offload_chunk=OFFLOAD_CHUNK,
                           host_threads=self.n_threads, per_param=self.per_tensor,
                           device_step=device_step)
        rs = self.rs
        if self.offload:         # the fp32 master lives in host memory
            rs.master.copy_(torch.from_numpy(synth.normal_f32(S, self.seed, synth.KIND_MASTER, 0, 0,
                                                              lo, phi, synth.MASTER_SIGMA)))
        else:
            master = rs.master if not self.per_tensor else torch.empty(S, dtype=torch.float32,
                                                                       device=device)
            synth.device_normal_f32(master, self.seed, synth.KIND_MASTER, 0, 0, lo,
                                    phi if layout == "flat" else P, synth.MASTER_SIGMA)
            if layout == "shard0":   # padding inside the coalesced buffer starts at zero
                master.mul_(padding_mask(self.plan, rank).to(device))
            if self.per_tensor:      # each parameter chunk's own fp32 tensor
                for t, (_, _, soff, ln) in zip(rs.master_tensors, rs.segments):
                    t.copy_(master[soff:soff + ln])
                del master
        if gather:
            for r in range(nd):
                if r != rank:
                    synth.device_normal_bf16(rs.param_shards[r], self.seed, synth.KIND_PARAM, 0, 0,
                                             r * S, phi, synth.MASTER_SIGMA)
        # gradient inputs
        self.windows = []
        if reps and not bucket and layout == "shard0":
            # each replica's per-tensor gradients, flattened into the coalesced layout
            full = staggered_replicas(reps, P, device)
            offs = model_offsets(w.numels)
            for k, t in enumerate(full):
                per_tensor = []
                for n, off in zip(w.numels, offs):
                    g = torch.empty(n, dtype=torch.int16, device=device)
                    synth.device_normal_bf16(g, self.seed, synth.KIND_REPLICA, 1, k, off, phi,
                                             synth.GRAD_SIGMA)
                    per_tensor.append(g)
                zm.zero_flatten_params(self.plan, per_tensor, t)
                if k == 0:          # kept: replica 0's flatten is timed outside the step
                    self.flatten_in = per_tensor
                del per_tensor
            self.windows = [(0, P, full)]
            self.flatten_out = torch.empty(P, dtype=torch.int16, device=device)
            self._ft = zm.CopyTable.flatten(self.plan, self.flatten_in, self.flatten_out)
            st0 = torch.cuda.current_stream(device).cuda_stream
            self.extra_phases = [("flatten", self._ft.prepare_run(st0)),
                                 ("flatten_call", zm._binding.prepare_flatten_params(
                                     self.plan, self.flatten_in, self.flatten_out, st0))]
        elif reps and not bucket:
            full = staggered_replicas(reps, P, device)
            for k, t in enumerate(full):
                synth.device_normal_bf16(t, self.seed, synth.KIND_REPLICA, 1, k, 0, phi,
                                         synth.GRAD_SIGMA)
            self.windows = [(0, P, full)]
        elif reps:
            for b0, cnt in spans:
                ws = staggered_replicas(reps, cnt, device)
                for k, t in enumerate(ws):
                    synth.device_normal_bf16(t, self.seed, synth.KIND_REPLICA, 1, k, b0, phi,
                                             synth.GRAD_SIGMA)
                self.windows.append((b0, cnt, ws))
        else:
            synth.device_normal_bf16(rs.grad, self.seed, synth.KIND_GRAD, 1, 0, lo, phi,
                                     synth.GRAD_SIGMA)
        # the other ranks' squared-norm partials, each from its own gradient as the
        # configuration produces it: the reduce of the same replicas, the reduce of
        # its bucket windows of generated replicas, or (gradients that arrive
        # averaged) the norm of its generated averaged gradient
        parts = torch.zeros(nd, dtype=torch.float64, device=device)
        tmp = torch.empty(S, dtype=torch.int16, device=device)
        bucket_reps = staggered_replicas(reps, bucket, device) if reps and bucket else None
        win_part = torch.zeros(1, dtype=torch.float64, device=device)
        for r in range(nd):
            if r == rank:
                continue
            if reps and not bucket:
                zm.zero_grad_reduce_shard(self.plan, r, self.windows[0][2], 0, P, tmp,
                                          sqnorm_out=parts[r:r + 1], workspace=rs.workspace)
            elif reps:
                total = 0.0                  # the window partials, summed in arrival order
                for b0, cnt in bucket_windows(P, bucket, r * S, (r + 1) * S):
                    a, e = max(b0, r * S), min(b0 + cnt, (r + 1) * S)
                    for k, t in enumerate(bucket_reps):
                        synth.device_normal_bf16(t, self.seed, synth.KIND_REPLICA, 1, k, a, phi,
                                                 synth.GRAD_SIGMA, n=e - a)
                    zm.zero_grad_reduce_shard(self.plan, r, [t[:e - a] for t in bucket_reps], a,
                                              e - a, tmp, sqnorm_out=win_part,
                                              workspace=rs.workspace)
                    total += float(win_part.item())
                parts[r] = total
            else:
                synth.device_normal_bf16(tmp, self.seed, synth.KIND_GRAD, 1, 0, r * S, phi,
                                         synth.GRAD_SIGMA)
                zm.zero_grad_sqnorm(tmp, parts[r:r + 1], workspace=rs.workspace)
        del tmp, bucket_reps
        rs.partials[:nd].copy_(parts)
        torch.cuda.synchronize()
        if reps:
            first = ("reduce", lambda: rs.reduce(self.windows))
        else:
            sq = zm._binding.Prepared(zm._binding._sqnorm, [
                rs.grad.data_ptr(), S, rs.partials[rank:rank + 1].data_ptr(),
                rs.workspace.data_ptr(), rs.workspace.numel(),
                torch.cuda.current_stream(device).cuda_stream], "zero_grad_sqnorm")
            first = ("sqnorm", sq)
        self.phases = [first, ("clip", rs.clip), ("adamw", rs.adamw)]
        st0 = torch.cuda.current_stream(device).cuda_stream
        extra = list(getattr(self, "extra_phases", None) or [])
        # Outside the step, the call-based gather (and flatten) beside the copy
        # tables that the step uses.
        if gather:
            self.phases.append(("gather", rs.gather))
            extra.append(("gather_call", zm._binding.prepare_gather_params(
                self.plan, rs.param_shards, rs.tensors, st0)))
        if extra:
            self.extra_phases = extra
        if reps and not bucket and not self.offload and not name.endswith("-pertensor"):
            self._setup_reduce_tensors(device)
        self.adamw_launches = 1
        self.elems_per_step = S
        if self.per_tensor:
            self._setup_per_tensor(device)
        torch.cuda.synchronize()

    def _setup_reduce_tensors(self, device):
        """Outside the step: the same reduce from replicas that are still
        per-tensor (each of the R replicas' tensors its own allocation, the
        values the flat replicas hold), through a zero_reduce_table, which needs
        no flatten of each replica first. Checked here against the step's own
        reduce over the flat replicas, bit for bit."""
        import torch

        import synth
        from zero_partitioned_mixed_partition_amd import _binding as zb
        w, rs = self.workload, self.rs
        offs = (model_offsets(w.numels) if self.layout == "shard0"
                else [self.plan.tensor_offset(t) for t in range(self.plan.num_tensors)])
        self.rt_reps = []
        for k in range(self.replicas):
            rep = []
            for n, off in zip(w.numels, offs):
                g = torch.empty(n, dtype=torch.int16, device=device)
                synth.device_normal_bf16(g, self.seed, synth.KIND_REPLICA, 1, k, off, self.phi,
                                         synth.GRAD_SIGMA)
                rep.append(g)
            self.rt_reps.append(rep)
        self.rt_grad = torch.empty(self.S, dtype=torch.int16, device=device)
        self.rt_sq = torch.zeros(1, dtype=torch.float64, device=device)
        self.rt_table = zb.ReduceTable(self.plan, self.rank, self.rt_reps, self.rt_grad)
        run = self.rt_table.prepare_run(self.rt_sq, torch.cuda.current_stream(device).cuda_stream)
        run()
        rs.reduce(self.windows)
        torch.cuda.synchronize()
        if not torch.equal(self.rt_grad, rs.grad):
            raise RuntimeError("the reduce from per-tensor replicas differs from the flat reduce")
        self.extra_phases = list(getattr(self, "extra_phases", None) or []) + [("reduce_tensors", run)]

    def _setup_per_tensor(self, device):
        """FSDP-2 as its optimizer sees it (RankStep(per_param=True)): every
        parameter's local chunk has its own fp32 master/m/v tensors, and the
        step's update is the multi-tensor AdamW through its device-resident
        table (one launch). Gradients and parameters stay views into the rank's
        coalesced buffers. The list call, which carries its descriptors in the
        kernel arguments, is timed beside it outside the step, on copies of the
        state."""
        import torch

        from zero_partitioned_mixed_partition_amd import _binding as zb
        rs = self.rs
        self.segs = rs.segments
        sl = [slice(soff, soff + ln) for (_, _, soff, ln) in self.segs]
        lm = [t.clone() for t in rs.master_tensors]
        lmm = [torch.zeros_like(t) for t in rs.master_tensors]
        lv = [torch.zeros_like(t) for t in rs.master_tensors]
        self._list_state = (lm, lmm, lv)
        st = torch.cuda.current_stream(device).cuda_stream
        call_list = zb.prepare_multi_tensor_adamw_step(
            lm, lmm, lv, [rs.grad[x] for x in sl], [rs.param_shards[self.rank][x] for x in sl],
            clip_scale=rs.scale, stream=st, **self.hyper.as_kwargs())
        self.t_list = 0

        def adamw_list():
            self.t_list += 1
            call_list(self.t_list)
        self.extra_phases = (list(getattr(self, "extra_phases", None) or [])
                             + [("adamw_list", adamw_list)])
        self.elems_per_step = sum(x.stop - x.start for x in sl)

    def state_arrays(self):
        """The rank's fp32 master, m and v over its coalesced buffer, on the host
        (per-parameter state is placed at its chunk's offset, padding zero)."""
        import numpy as np
        rs = self.rs
        if not getattr(self, "per_tensor", False):
            return [x.detach().cpu().numpy() for x in (rs.master, rs.exp_avg, rs.exp_avg_sq)]
        out = [np.zeros(self.S, np.float32) for _ in range(3)]
        for (_, _, soff, ln), *arrs in zip(self.segs, rs.master_tensors, rs.exp_avg_tensors,
                                           rs.exp_avg_sq_tensors):
            for o, a in zip(out, arrs):
                o[soff:soff + ln] = a.cpu().numpy()
        return out

    def offload_parts(self, reps: int):
        """The offload phase's two halves on their own, on copies of the state:
        the host update alone (ms) and the shard's bf16 round trip over the link
        alone (ms, pinned host memory, one copy each way)."""
        import torch

        import zero_partitioned_mixed_partition_amd as zm
        rs = self.rs
        p, m, v = rs.master.clone(), rs.exp_avg.clone(), rs.exp_avg_sq.clone()
        g = rs.grad.cpu()
        out = torch.empty(self.S, dtype=torch.int16)
        hp = self.hyper.as_kwargs()
        zm.zero_host_adamw_step(p, m, v, g, out, 1, n_threads=self.n_threads, **hp)
        t0 = time.perf_counter()
        for k in range(reps):
            zm.zero_host_adamw_step(p, m, v, g, out, 2 + k, n_threads=self.n_threads, **hp)
        host_ms = (time.perf_counter() - t0) * 1e3 / reps
        pin = torch.empty(self.S, dtype=torch.int16).pin_memory()
        pin.copy_(rs.grad, non_blocking=True)
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        c = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            pin.copy_(rs.grad, non_blocking=True)
        b.record()
        for _ in range(reps):
            rs.param_shards[self.rank].copy_(pin, non_blocking=True)
        c.record()
        torch.cuda.synchronize()
        d2h, h2d = a.elapsed_time(b) / reps, b.elapsed_time(c) / reps
        return {"host_adamw_ms": host_ms, "host_threads": self.n_threads,
                "host_adamw_gbs": 28 * self.S / (host_ms * 1e-3) / 1e9,
                "d2h_ms": d2h, "h2d_ms": h2d,
                "d2h_gbs": 2 * self.S / (d2h * 1e-3) / 1e9,
                "h2d_gbs": 2 * self.S / (h2d * 1e-3) / 1e9}

    def bytes_per_phase(self):
        S = self.S
        # the offload phase moves 2 B/elem each way over the host link; its
        # 28 B/elem of state traffic is in host DRAM. The per-parameter update
        # covers the chunks' elements only (not the coalesced buffer's padding).
        b = {"clip": 8 * (self.n_ranks + max(len(self.windows), 1)) + 4,
             "adamw": 4 * S if self.offload else 28 * self.elems_per_step}
        if self.replicas:
            b["reduce"] = (2 * self.replicas + 2) * S
        else:
            b["sqnorm"] = 2 * S
        if any(p[0] == "gather" for p in self.phases):
            b["gather"] = 4 * self.phi
        if any(p[0] == "flatten" for p in getattr(self, "extra_phases", None) or []):
            b["flatten"] = b["flatten_call"] = 4 * self.phi + 2 * (self.P - self.phi)
        if "gather" in b:
            b["gather_call"] = b["gather"]
        if getattr(self, "per_tensor", False):
            b["adamw_list"] = 28 * self.elems_per_step
        if getattr(self, "rt_table", None) is not None:
            b["reduce_tensors"] = (2 * self.replicas + 2) * S
        return b

    def describe(self):
        red = (f"reduce of {self.replicas} bf16 replicas" +
               (f" in {len(self.windows)} buckets of {self.bucket}" if self.bucket else "")
               if self.replicas else "squared norm of the averaged bf16 gradient")
        g = f" + gather of {len(self.workload.numels)} tensors" if self.rs.tensors else ""
        lay = (", FSDP-2 per-parameter Shard(0) layout (coalesced per-rank buffers)"
               if self.layout == "shard0" else "")
        upd = (f"ZeRO-Offload AdamW (fp32 state in host DRAM, {self.n_threads} host threads, "
               f"bf16 grads/params over PCIe in {OFFLOAD_CHUNK}-element chunks)"
               if self.offload else "AdamW")
        return (f"{self.workload.name} tensor list{lay}, N_d={self.n_ranks}, rank {self.rank} shard "
                f"of {self.S} elements; step = {red} + clip {self.max_norm} + {upd}{g}")


class AllRanksWorkload:
    """Every rank of one data-parallel job, in turn on one GPU: reduce, AdamW, then gather."""

    def __init__(self, name: str, device):
        import torch

        import synth
        import zero_partitioned_mixed_partition_amd as zm
        from zero_partitioned_mixed_partition_amd import _binding as zb
        from zero_partitioned_mixed_partition_amd.step import (Hyper, _staggered_arena, plan_numels,
                                                               staggered_replicas)

        # "-fused": each rank's reduce and AdamW in one pass (no clip between them)
        self.fused = name.endswith("-fused")
        w = synth.WORKLOADS[name[:-len("-fused")] if self.fused else name]
        self.name, self.workload, self.device = name, w, device
        self.n_ranks, self.rank, self.replicas = w.n_ranks, None, w.replicas
        self.seed = 1000 + w.seed
        self.plan = zm.zero_partition_plan(w.numels, w.n_ranks, w.align)
        P, S, phi = self.plan.padded_numel, self.plan.shard_numel, self.plan.numel
        self.P, self.S, self.phi = P, S, phi
        self.hyper = Hyper(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                           weight_decay=w.weight_decay)
        views, self.arena = _staggered_arena(
            [(P, torch.float32), (P, torch.float32), (P, torch.float32), (P, torch.int16),
             (P, torch.int16)], device)
        self.master, self.m, self.v, self.grad, self.param = views
        synth.device_normal_f32(self.master, self.seed, synth.KIND_MASTER, 0, 0, 0, phi,
                                synth.MASTER_SIGMA)
        self.reps = staggered_replicas(self.replicas, P, device)
        for k, t in enumerate(self.reps):
            synth.device_normal_bf16(t, self.seed, synth.KIND_REPLICA, 1, k, 0, phi, synth.GRAD_SIGMA)
        self.tensors = [torch.empty(n, dtype=torch.int16, device=device)
                        for n in plan_numels(self.plan)]
        # this job does not clip, so the reduce computes no squared norm
        if w.max_norm > 0:
            raise ValueError(f"{name}: the all-ranks workload runs without clipping")
        self.max_norm = 0.0
        st = torch.cuda.current_stream(device).cuda_stream
        sl = [slice(r * S, (r + 1) * S) for r in range(w.n_ranks)]
        self._reduce = [zb.prepare_grad_reduce_shard(self.plan, r, self.reps, 0, P,
                                                     self.grad[sl[r]], None, None, st)
                        for r in range(w.n_ranks)]
        self._adamw = [zb.prepare_shard_adamw_step(self.master[sl[r]], self.m[sl[r]],
                                                   self.v[sl[r]], self.grad[sl[r]],
                                                   self.param[sl[r]], clip_scale=None, stream=st,
                                                   **self.hyper.as_kwargs())
                       for r in range(w.n_ranks)]
        self._gt = zb.CopyTable.gather(self.plan, [self.param[s] for s in sl], self.tensors)
        self._gather = self._gt.prepare_run(st)
        # outside the step: one replica flattening its per-tensor gradients into a
        # flat buffer (the step before the reduce)
        offs = [self.plan.tensor_offset(t) for t in range(self.plan.num_tensors)]
        self.grad_tensors = []
        for n, off in zip(plan_numels(self.plan), offs):
            g = torch.empty(n, dtype=torch.int16, device=device)
            synth.device_normal_bf16(g, self.seed, synth.KIND_REPLICA, 1, 0, off, phi,
                                     synth.GRAD_SIGMA)
            self.grad_tensors.append(g)
        self.flat_out = torch.empty(P, dtype=torch.int16, device=device)
        self._ft = zb.CopyTable.flatten(self.plan, self.grad_tensors, self.flat_out)
        self.extra_phases = [("flatten", self._ft.prepare_run(st)),
                             ("flatten_call", zb.prepare_flatten_params(self.plan, self.grad_tensors,
                                                                       self.flat_out, st)),
                             ("gather_call", zb.prepare_gather_params(
                                 self.plan, [self.param[s] for s in sl], self.tensors, st))]
        self.t = 0
        torch.cuda.synchronize()

        def reduce_all():
            for f in self._reduce:
                f()

        def adamw_all():
            self.t += 1
            for f in self._adamw:
                f(self.t)

        self.phases = [("reduce", reduce_all), ("adamw", adamw_all), ("gather", self._gather)]
        # AdamW-phase bytes per element and the kernel that phase runs
        self.adamw_bpe, self.adamw_kernel = 28, "adamw_kernel"
        if self.fused:
            self._fused = [zb.prepare_reduce_adamw_step(
                self.plan, r, self.reps, 0, P, self.master[sl[r]], self.m[sl[r]], self.v[sl[r]],
                self.param[sl[r]], clip_scale=None, stream=st, **self.hyper.as_kwargs())
                for r in range(w.n_ranks)]

            def fused_all():
                self.t += 1
                for f in self._fused:
                    f(self.t)
            self.phases = [("adamw", fused_all), ("gather", self._gather)]
            # R bf16 replicas read, master/m/v read and written, bf16 parameter written
            self.adamw_bpe, self.adamw_kernel = 2 * self.replicas + 26, "reduce_adamw_kernel"
        self.adamw_launches = w.n_ranks
        self.elems_per_step = P

    def bytes_per_phase(self):
        P = self.P
        return {"reduce": (2 * self.replicas + 2) * P, "adamw": self.adamw_bpe * P,
                "gather": 4 * self.phi,
                "flatten": 4 * self.phi + 2 * (P - self.phi), "gather_call": 4 * self.phi,
                "flatten_call": 4 * self.phi + 2 * (P - self.phi)}

    def describe(self):
        update = (f"reduce of {self.replicas} bf16 replicas and AdamW in one pass per rank"
                  if self.fused else
                  f"reduce of {self.replicas} bf16 replicas per rank + AdamW per shard")
        return (f"{self.workload.name} tensor list, N_d={self.n_ranks}, all {self.n_ranks} ranks in "
                f"turn ({self.S} elements each); step = {update} (no norm or clip) + gather of "
                f"{len(self.workload.numels)} tensors")


def model_offsets(numels):
    """Each tensor's start in the model's natural (definition-order) concatenation:
    the generator keys a tensor's values by these, whatever the sharding layout."""
    offs, pos = [], 0
    for n in numels:
        offs.append(pos)
        pos += n
    return offs


def padding_mask(plan, rank: int):
    """float32 [S]: 1 where the rank's buffer holds tensor elements, 0 on padding."""
    import torch
    mask = torch.zeros(plan.shard_numel, dtype=torch.float32)
    for (_, _, soff, ln) in plan.segments(rank):
        mask[soff:soff + ln] = 1.0
    return mask


def make_workload(name: str, device, device_step: bool = False):
    if name.startswith("gpt-1.3b"):
        if device_step:
            raise SystemExit("bench.py: --device-step applies to the one-rank workloads")
        return AllRanksWorkload(name, device)
    wl = RankWorkload(name, device, device_step)
    if device_step:     # the scheduled kernels; the traffic entries are the plain kernel's
        wl.adamw_kernel = "adamw_table_sched_kernel" if wl.per_tensor else "adamw_sched_kernel"
    return wl


def run_step(wl) -> None:
    for _, fn in wl.phases:
        fn()



class AdamWEvents:
    """Timing events for the AdamW brackets, recorded on torch's current stream
    (the stream every call here launches on). They are created with HIP's
    hipEventDisableSystemFence flag: a default event's record carries a
    system-scope release, which writes back and invalidates the caches between
    the kernel and the marker, so a default bracket around one kernel times that
    flush too and slows the kernel that follows it. Measured on MI355X in the
    GPT-2 rank step: 70.8 us per AdamW launch with these events against 72.7 us
    with default ones (kernel trace: 69.9 us), and 205 us against 209 us per step.
    Events are created before the timed region, one pair per bracket."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, pairs: int):
        import ctypes
        import torch
        self._ct = ctypes
        hip = ctypes.CDLL("libamdhip64.so")
        hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                            ctypes.c_void_p]
        hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self._hip = hip
        self._stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        self._ev = []
        for _ in range(2 * pairs):
            e = ctypes.c_void_p()
            self._ok(hip.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE),
                     "hipEventCreateWithFlags")
            self._ev.append(e)
        self._next = 0

    @staticmethod
    def _ok(rc: int, what: str) -> None:
        if rc != 0:
            raise RuntimeError(f"{what} failed with HIP error {rc}")

    def record(self) -> None:
        """Record the next event of the pool on the launch stream."""
        self._ok(self._hip.hipEventRecord(self._ev[self._next], self._stream), "hipEventRecord")
        self._next += 1

    def elapsed_ms(self):
        """Durations (ms) of the recorded pairs, in recording order (after a sync)."""
        out = []
        for i in range(0, self._next - 1, 2):
            f = self._ct.c_float()
            self._ok(self._hip.hipEventElapsedTime(self._ct.byref(f), self._ev[i], self._ev[i + 1]),
                     "hipEventElapsedTime")
            out.append(f.value)
        return out

    def __del__(self):
        for e in getattr(self, "_ev", []):
            self._hip.hipEventDestroy(e)


def time_phases(wl, reps: int):
    """Mean duration (ms) of each phase on its own: the phase is issued `reps`
    times back to back between two HIP events on the launch stream, so the
    queue never drains between calls."""
    import torch
    out = {}
    for n, fn in wl.phases:
        fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        out[n] = a.elapsed_time(b) / reps
    return out


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "adamw_traffic.json")
ADAMW_SOURCES = [os.path.join(ROOT, "zero_partitioned_mixed_partition_amd", "csrc", f)
                 for f in ("adamw.hip", "device_common.hpp")]


def adamw_flushed(wl, reps: int):
    """AdamW launch time (us) with HBM-side caches cold: before each timed
    launch, 1 GiB is written (four times the 256 MB Infinity Cache), then the
    AdamW phase alone runs between two events. Returns median and min."""
    import torch
    fn = dict(wl.phases)["adamw"]
    scratch = torch.empty(1 << 28, dtype=torch.float32, device=wl.device)
    ev = AdamWEvents(reps)
    for k in range(reps):
        scratch.fill_(float(k))
        ev.record()
        fn()
        ev.record()
        torch.cuda.synchronize()
    times = [t * 1e3 / wl.adamw_launches for t in ev.elapsed_ms()]
    del scratch
    times.sort()
    return {"median_us": times[len(times) // 2], "min_us": times[0], "launches": reps}


def kernel_source_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in ADAMW_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def measured_traffic(elems_per_launch: int, kernel: str = "adamw_kernel"):
    """HBM bytes per AdamW call from the committed counter runs (FETCH_SIZE and
    WRITE_SIZE, scaled by a 1 GiB copy, summed over the call's dispatches), or
    None when the kernel sources have changed since they were taken or no run
    covers this shard size."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    d = json.load(open(TRAFFIC_FILE))
    for e in d.get("runs", []):
        if (e.get("source_sha256") == kernel_source_digest() and e.get("elems") == elems_per_launch
                and e.get("kernel", "adamw_kernel") == kernel):
            return e["bytes_per_launch"]
    return None


def _counter_means(folder: str, counter: str):
    """Per kernel name, the per-dispatch values of one rocprofv3 counter (summed
    over the rows a dispatch reports, e.g. one per L2 channel), in KiB."""
    import collections
    import csv
    import glob
    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"bench.py: no counter_collection.csv under {folder}")
    per, names = collections.defaultdict(float), {}
    for f in files:
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            key = (f, r["Dispatch_Id"])
            per[key] += float(r["Counter_Value"])
            names[key] = r["Kernel_Name"]
    out = collections.defaultdict(list)
    for k in sorted(per, key=lambda k: (k[0], int(k[1]))):
        out[names[k]].append(per[k])
    return out


def write_traffic(args) -> int:
    """profiles/adamw_traffic.json's entry for this workload, from the counter runs."""
    import synth
    import zero_partitioned_mixed_partition_amd as zm
    if args.workload == "gpt-1.3b":         # every rank's shard in turn, one launch each
        w = synth.WORKLOADS[args.workload]
        nd = w.n_ranks
        plan = zm.zero_partition_plan(w.numels, nd, w.align)
        who = f"{args.workload}, each of the {nd} ranks' shards"
    elif args.workload not in RankWorkload.SPECS or args.workload.endswith("-pertensor") \
            or args.workload.endswith("-offload"):
        raise SystemExit("bench.py: --write-traffic covers the flat-array AdamW workloads")
    else:
        lst, nd, rank, *_rest, layout = RankWorkload.SPECS[args.workload]
        w = synth.WORKLOADS[lst]
        plan = (zm.zero_partition_plan_shard0(w.numels, [x[0] for x in w.shapes], nd, w.align)
                if layout == "shard0" else zm.zero_partition_plan(w.numels, nd, w.align))
        who = f"{args.workload} rank {rank} of {nd}"
    S = plan.shard_numel
    calls = args.profile_steps
    if calls < 1:
        raise SystemExit("bench.py: give --profile-steps as in the counter runs")
    fetch = _counter_means(args.write_traffic[0], "FETCH_SIZE")
    write = _counter_means(args.write_traffic[1], "WRITE_SIZE")
    cp = [n for n in fetch if "copyBuffer" in n]
    if not cp or not [n for n in write if "copyBuffer" in n]:
        raise SystemExit("bench.py: the runs need --calibrate-copy (a 1 GiB copy to scale by)")
    gib_kib = float(1 << 20)
    f_scale = gib_kib / max(fetch[cp[0]])
    w_scale = gib_kib / max(write[[n for n in write if "copyBuffer" in n][0]])
    ad = [n for n in fetch if n.startswith("adamw_kernel")]
    if len(ad) != 1:
        raise SystemExit(f"bench.py: expected one AdamW kernel name, found {ad}")
    ad = ad[0]
    if len(fetch[ad]) % calls or len(write[ad]) != len(fetch[ad]):
        raise SystemExit(f"bench.py: {len(fetch[ad])} and {len(write[ad])} AdamW dispatches "
                         f"for {calls} steps")
    # per launch: the mean over the profiled steps' dispatches
    f_bytes = sum(fetch[ad]) * 1024 * f_scale / len(fetch[ad])
    w_bytes = sum(write[ad]) * 1024 * w_scale / len(write[ad])
    entry = {"kernel": "adamw_kernel", "workload": who,
             "elems": S, "dispatches_per_call": len(fetch[ad]) // calls,
             "fetch_bytes": f_bytes, "write_bytes": w_bytes, "bytes_per_launch": f_bytes + w_bytes,
             "algorithmic_bytes": 28 * S, "fetch_scale": f_scale, "write_scale": w_scale,
             "source_sha256": kernel_source_digest(),
             "commands": [
                 f"rocprofv3 --pmc FETCH_SIZE -T -d {args.write_traffic[0]} -o fetch -f csv -- "
                 f"python3 bench.py --workload {args.workload} --profile-steps {calls} --calibrate-copy",
                 f"rocprofv3 --pmc WRITE_SIZE -T -d {args.write_traffic[1]} -o write -f csv -- "
                 f"python3 bench.py --workload {args.workload} --profile-steps {calls} --calibrate-copy"]}
    d = json.load(open(TRAFFIC_FILE)) if os.path.exists(TRAFFIC_FILE) else {}
    runs = [e for e in d.get("runs", []) if e.get("elems") != S]
    d["runs"] = runs + [entry]
    json.dump(d, open(TRAFFIC_FILE, "w"), indent=1)
    print(json.dumps(entry, indent=1))
    print(f"AdamW traffic / algorithmic bytes: {(f_bytes + w_bytes) / (28 * S):.6f}")
    print(f"calibration: {cp[0]} fetch x{f_scale:.4f}, write x{w_scale:.4f}")
    print("| Kernel | Dispatches | Read per dispatch (KiB, scaled) | Written per dispatch (KiB, scaled) |")
    print("|---|---|---|---|")
    for n in sorted(fetch):
        if n in write:
            print(f"| {n} | {len(fetch[n])} | {sum(fetch[n]) / len(fetch[n]) * f_scale:,.1f} | "
                  f"{sum(write[n]) / len(write[n]) * w_scale:,.1f} |")
    return 0


def cpu_baseline(wl, budget_s: float):
    """The oracle on the host for the same workload, bounded in time. The default
    workload times the oracle's whole rank step; the large ones time the same
    per-element work (the reduce where the step has one, the exact norm and clip
    where it clips, AdamW) on a 2^24-element slice."""
    import numpy as np

    import oracle
    import synth
    hp = wl.hyper.as_kwargs()
    if wl.name in ("gpt2-small", "gpt2-small-offload"):
        S, phi, rank = wl.S, wl.phi, wl.rank
        ref = oracle.partition_plan(wl.workload.numels, wl.n_ranks, wl.workload.align)
        lo = rank * S
        reps = [synth.normal_bf16(S, wl.seed, synth.KIND_REPLICA, 1, k, lo, phi, synth.GRAD_SIGMA)
                for k in range(wl.replicas)]
        state = {"master": synth.normal_f32(S, wl.seed, synth.KIND_MASTER, 0, 0, lo, phi,
                                            synth.MASTER_SIGMA),
                 "exp_avg": np.zeros(S, np.float32), "exp_avg_sq": np.zeros(S, np.float32)}
        shards = [synth.normal_bf16(S, wl.seed, synth.KIND_PARAM, 0, 0, r * S, phi,
                                    synth.MASTER_SIGMA) for r in range(wl.n_ranks)]
        partials = [1.0] * wl.n_ranks

        def one(t):
            oracle.rank_step(ref, rank, reps, lo, state, shards, partials, t, hp, wl.max_norm)
        sample = (f"full rank-{rank} steps of the same workload (reduce of {wl.replicas} replica "
                  f"windows, exact norm, clip, AdamW on {S} elements, gather of {phi} parameters)")
        per_step = S
    else:
        n = min(wl.S, 1 << 24)
        clips = wl.max_norm > 0
        g0 = (wl.rank or 0) * wl.S
        R = wl.replicas
        if R:
            reps = [synth.normal_bf16(n, wl.seed, synth.KIND_REPLICA, 1, k, g0, wl.phi,
                                      synth.GRAD_SIGMA) for k in range(R)]
        else:
            reps = [synth.normal_bf16(n, wl.seed, synth.KIND_GRAD, 1, 0, g0, wl.phi,
                                      synth.GRAD_SIGMA)]
        window = oracle.partition_plan([n], 1, 1)
        st = {"p": synth.normal_f32(n, wl.seed, synth.KIND_MASTER, 0, 0, g0, wl.phi,
                                    synth.MASTER_SIGMA),
              "m": np.zeros(n, np.float32), "v": np.zeros(n, np.float32)}

        def one(t):
            if R:
                g = np.zeros(n, np.uint16)
                oracle.reduce_shard(window, 0, reps, 0, g)
            else:                   # gradients arrive averaged: no reduce in the step
                g = reps[0]
            # the all-ranks job does not clip: no norm between its reduce and AdamW
            clip = oracle.clip_scale([oracle.sqnorm(g)], wl.max_norm) if clips else 1.0
            st["p"], st["m"], st["v"], _ = oracle.adamw_step(st["p"], st["m"], st["v"], g, t,
                                                             clip=clip, **hp)
        work = f"reduce of {R} replica windows, " if R else ""
        work += "exact norm, clip, AdamW" if clips else "AdamW"
        sample = (f"passes of the per-element work of this workload ({work}) "
                  f"over a {n}-element slice of the shard")
        per_step = n
    one(1)          # untimed: the first touch of fresh host pages is not oracle work
    t0 = time.perf_counter()
    k = 0
    while True:
        k += 1
        one(1 + k)
        el = time.perf_counter() - t0
        if el >= budget_s or k >= 1000:
            break
    return {"value": per_step * k / el, "unit": "params/s", "cores": 1, "kind": "oracle",
            "sample": f"{k} {sample}, single-threaded numpy", "seconds": el,
            "host_cpus": len(os.sched_getaffinity(0))}


def measure(wl, steps: int, warmup: int) -> dict:
    """Warmup, then `steps` timed steps (the AdamW phase bracketed by events on its
    launch stream), then each phase on its own, the cold-cache AdamW launch, and
    (offload) the host update and the link on their own."""
    import torch
    # Python's cyclic garbage collector is off while steps are issued: a full
    # collection pauses the issuing thread for tens of milliseconds, which the
    # GPU would spend idle (as timeit does; the collector is run first).
    gc.collect()
    gc.disable()
    for _ in range(warmup):
        run_step(wl)
    torch.cuda.synchronize()
    # Timed region: whole steps; the AdamW phase is bracketed by events on the
    # stream it is launched on (torch's current stream, which every call here uses).
    adamw_ev = AdamWEvents(steps * sum(1 for name, _ in wl.phases if name == "adamw"))
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        for name, fn in wl.phases:
            if name == "adamw":
                adamw_ev.record()
                fn()
                adamw_ev.record()
            else:
                fn()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = start.elapsed_time(end) / steps
    adamw_each = sorted(t / wl.adamw_launches for t in adamw_ev.elapsed_ms())
    adamw_ms = sum(adamw_each) / len(adamw_each)
    print(f"[bench] {wl.name}: {steps} steps: {ms_per_step:.4f} ms/step (wall {wall:.3f} s), "
          f"adamw {adamw_ms * 1e3:.1f} us per launch", file=sys.stderr, flush=True)

    phase_ms = time_phases(wl, max(3, min(steps, 50)))
    bpp = wl.bytes_per_phase()
    offload = getattr(wl, "offload", False)

    def rates(ms):
        out = {}
        for n in ms:
            gbs = bpp[n] / (ms[n] * 1e-3) / 1e9
            if offload and n == "adamw":
                out[n] = {"ms": ms[n], "link_bytes": bpp[n], "gbs": gbs,
                          "frac_of_pcie_peak": gbs / PCIE_PEAK_GBS}
            else:
                out[n] = {"ms": ms[n], "bytes": bpp[n], "gbs": gbs,
                          "frac_of_hbm_peak": gbs / HBM_PEAK_GBS}
        return out
    kernels = rates(phase_ms)
    outside = None
    if getattr(wl, "extra_phases", None):
        class _Extra:
            phases = wl.extra_phases
        outside = rates(time_phases(_Extra, max(3, min(steps, 20))))
    parts = wl.offload_parts(max(3, min(steps, 10))) if offload else None
    flushed = None if offload else adamw_flushed(wl, 10)
    gc.enable()
    return {"ms_per_step": ms_per_step, "adamw_ms": adamw_ms, "adamw_each": adamw_each,
            "kernels": kernels, "outside": outside, "bpp": bpp, "flushed": flushed, "parts": parts,
            "elems_per_launch": wl.elems_per_step // wl.adamw_launches, "offload": offload}


def also_line(name: str, device) -> dict:
    """Another workload measured in the same run, summarised: its step and AdamW
    figures (default steps and warmup)."""
    import torch
    print(f"[bench] setting up {name} (extra keys)", file=sys.stderr, flush=True)
    wl = make_workload(name, device)
    steps, warmup = DEFAULT_STEPS[name]
    m = measure(wl, steps, warmup)
    elems = m["elems_per_launch"]
    bpe, kern = getattr(wl, "adamw_bpe", 28), getattr(wl, "adamw_kernel", "adamw_kernel")
    gbs = bpe * elems / (m["adamw_ms"] * 1e-3) / 1e9
    out = {"workload": wl.describe(), "steps": steps, "warmup": warmup,
           "ms_per_step": m["ms_per_step"], "value": wl.elems_per_step / (m["ms_per_step"] * 1e-3),
           "adamw_params_per_s": elems / (m["adamw_ms"] * 1e-3),
           "adamw_event_us": {"mean": m["adamw_ms"] * 1e3,
                              "median": m["adamw_each"][len(m["adamw_each"]) // 2] * 1e3,
                              "min": m["adamw_each"][0] * 1e3, "launches": len(m["adamw_each"])},
           "adamw_hbm_gbs": gbs, "adamw_frac_of_hbm_peak": gbs / HBM_PEAK_GBS,
           "kernels": m["kernels"], "traffic": measured_traffic(elems, kern)}
    del wl
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def _separate_arrays(specs, device):
    """The arena's arrays as separate zeroed allocations (the caching allocator
    starts each large one on its own 2 MiB-aligned segment): the layout a
    caller gets from one torch.zeros per array."""
    import torch
    views = [torch.zeros(max(numel, 1), dtype=dtype, device=device)[:numel] for numel, dtype in specs]
    return views, views


def main(argv=None):
    args = parse_args(argv)
    if args.write_traffic:
        return write_traffic(args)
    if args.gpus != 1:
        print(f"bench.py: times one rank's step on one GPU; --gpus {args.gpus} is not supported "
              "(collectives across GPUs are not implemented)", file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 2
    steps = args.steps if args.steps is not None else DEFAULT_STEPS[args.workload][0]
    warmup = args.warmup if args.warmup is not None else DEFAULT_STEPS[args.workload][1]
    device = torch.device("cuda:0")
    torch.cuda.set_device(device)
    import zero_partitioned_mixed_partition_amd.step as step_module
    if args.stagger is not None:
        if args.stagger < 0:
            print("bench.py: --stagger must be >= 0", file=sys.stderr)
            return 2
        step_module.STAGGER = args.stagger
    if args.separate_arrays:
        step_module._staggered_arena = _separate_arrays
    print(f"[bench] setting up {args.workload}", file=sys.stderr, flush=True)
    wl = make_workload(args.workload, device, args.device_step)
    if args.profile_steps:
        if args.calibrate_copy:
            src = torch.ones(1 << 28, dtype=torch.float32, device=device)
            dst = torch.empty_like(src)
            torch.cuda.synchronize()
            dst.copy_(src)                      # reads 1 GiB, writes 1 GiB
            torch.cuda.synchronize()
            del src, dst
        if args.profile_extra:
            for _, fn in getattr(wl, "extra_phases", None) or []:
                fn()
        for _ in range(args.profile_steps):
            run_step(wl)
        torch.cuda.synchronize()
        print(f"[bench] ran {args.profile_steps} steps for profiling", file=sys.stderr, flush=True)
        return 0

    m = measure(wl, steps, warmup)
    cpu = None
    if args.cpu_baseline_seconds > 0:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, args.cpu_baseline_seconds)
    ms_per_step, adamw_ms, adamw_each = m["ms_per_step"], m["adamw_ms"], m["adamw_each"]
    kernels, outside, bpp, flushed, parts = m["kernels"], m["outside"], m["bpp"], m["flushed"], m["parts"]
    elems_per_launch, offload = m["elems_per_launch"], m["offload"]
    adamw_kernel = getattr(wl, "adamw_kernel", "adamw_kernel")
    adamw_bytes = getattr(wl, "adamw_bpe", 28) * elems_per_launch
    adamw_gbs = adamw_bytes / (adamw_ms * 1e-3) / 1e9
    value = wl.elems_per_step / (ms_per_step * 1e-3)

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "params/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.describe(), "name": wl.name, "params": wl.phi,
                   "shard_elems": wl.S, "n_ranks": wl.n_ranks, "replicas": wl.replicas,
                   "parallelism": "one GPU's share of a dp job",
                   "arena_stagger_bytes": None if args.separate_arrays else step_module.STAGGER},
        "adamw_params_per_s": elems_per_launch / (adamw_ms * 1e-3),
        "adamw_event_us": {"mean": adamw_ms * 1e3, "median": adamw_each[len(adamw_each) // 2] * 1e3,
                           "min": adamw_each[0] * 1e3, "launches": len(adamw_each)},
        "adamw_flushed": flushed and dict(flushed, gbs=adamw_bytes / (flushed["median_us"] * 1e-6) / 1e9,
                                          frac_of_hbm_peak=adamw_bytes / (flushed["median_us"] * 1e-6)
                                          / 1e9 / HBM_PEAK_GBS),
        "adamw_hbm_gbs": adamw_gbs,
        "adamw_frac_of_hbm_peak": adamw_gbs / HBM_PEAK_GBS,
        "step_hbm_gbs": sum(bpp[n] for n, _ in wl.phases) / (ms_per_step * 1e-3) / 1e9,
        "kernels": kernels,
        "kernels_outside_step": outside,
        "roofline": {"bound": "hbm", "kernel": adamw_kernel, "achieved": adamw_gbs,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": adamw_gbs / HBM_PEAK_GBS,
                     "traffic": measured_traffic(elems_per_launch, adamw_kernel)},
        "cpu_baseline": cpu,
    }
    also = args.also or []
    if also:
        del wl, m
        gc.collect()
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        line["also"] = {name: also_line(name, device) for name in also}
    if offload:
        # The update runs on the host: the GPU-side figures above do not apply.
        link_gbs = 4 * elems_per_launch / (adamw_ms * 1e-3) / 1e9
        for k in ("adamw_hbm_gbs", "adamw_frac_of_hbm_peak"):
            del line[k]
        line["dtype"] = "f32"
        line["offload"] = dict(parts, step_adamw_ms=adamw_ms,
                               overlap=(parts["host_adamw_ms"] + parts["d2h_ms"] + parts["h2d_ms"])
                               / adamw_ms)
        line["roofline"] = {"bound": "pcie", "kernel": "zero_offload_adamw_step",
                            "achieved": link_gbs, "peak": PCIE_PEAK_GBS, "unit": "GB/s",
                            "frac": link_gbs / PCIE_PEAK_GBS, "traffic": None}
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
