"""One data-parallel rank's optimizer step as a sequence of C-ABI calls.

"Zero Redundancy Optimizer (ZeRO) and Fully Sharded Data Parallelism (FSDP):
Mathematical Foundations ...", section "Execution Flow for ZeRO-1", steps 2-4,
with section "ZeRO-Stage 2"'s bucketed reduction:

  1. zero_grad_reduce_shard  per gradient window (whole flat buffer or bucket):
                             the rank's averaged slice, plus its squared norm
  2. zero_clip_scale         global-norm clip coefficient from every partial
  3. zero_shard_adamw_step   fp32 master/m/v update, bf16 shard emitted into
                             the rank's slot of the parameter shards
  4. zero_gather_params      all shards -> per-tensor bf16 parameters (through a
                             copy table: zero_gather_table_create, zero_copy_table_run)

Without clipping, nothing waits on the global norm, and steps 1 and 3 run as
one pass per window (zero_reduce_adamw_step): the averaged gradient is used
where it is formed instead of going through HBM.

Everything stays on the device and on one stream; nothing synchronises with
the host inside a step. The other ranks' norm partials and parameter shards
are inputs: on a cluster they arrive through a scalar all-reduce and the
parameter all-gather.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple

import torch

from . import _binding as zb


@dataclass
class Hyper:
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01

    def as_kwargs(self) -> dict:
        return dict(lr=self.lr, beta1=self.beta1, beta2=self.beta2, eps=self.eps,
                    weight_decay=self.weight_decay)


class RankStep:
    """Device state of one rank and the call sequence of its step.

    plan         zero_partition_plan of the model's tensor list.
    rank         this rank.
    n_windows    gradient windows reduced per step (1 for a whole flat buffer,
                 the number of buckets that meet the shard otherwise).
    max_norm     clip threshold (<= 0: no clipping).
    offload      ZeRO-Offload ("ZeRO-Offload Mechanics"): the fp32 master, m and
                 v live in host memory (CPU tensors) and the update runs on the
                 host through zero_offload_adamw_step, with `offload_chunk`
                 elements per pinned staging slot and `host_threads` workers
                 (0: one per CPU this process may use). Reduce, clip and gather
                 stay on the device.
    fuse         with max_norm <= 0 (and no offload), step() reduces and
                 updates each window in one pass (reduce_update) when every
                 window has at most FUSE_MAX_REPLICAS replicas. Such a step
                 leaves self.grad and the own norm partials as they were.
    per_param    FSDP-2's optimizer-state layout ("FSDP-2: Per-Parameter
                 Sharding via DTensor (fully_shard)"): every segment of the
                 rank's shard (a parameter's local chunk) has fp32 master, m
                 and v tensors of its own (self.master_tensors,
                 self.exp_avg_tensors, self.exp_avg_sq_tensors, in segment
                 order), updated by the multi-tensor AdamW through a
                 device-resident table; self.master, self.exp_avg and
                 self.exp_avg_sq are then None. The gradient and the
                 parameter shard stay coalesced buffers (the reduce's output
                 and the gather's input), and the shard's padding is never
                 updated.
    device_step  AdamW's step counted on the device (a zero_adamw_schedule,
                 self.schedule): the update reads the step's scalars from device
                 memory and an advance call after it counts the step, only when
                 the clip coefficient is finite. A skipped step is then not
                 counted, and the whole step can be captured in a HIP graph and
                 replayed for successive steps. Flat or per-parameter device
                 state, and the one-pass update; not with offload (the host
                 update computes its own scalars).
    """

    # Measured on MI355X, no clip: with 8 replicas per window the one pass takes
    # 1,060.7 us per 164 M-element shard against 1,162.1 us for reduce then
    # AdamW; with 64 replicas over Llama-3-8B's six bucket windows it takes
    # 3.32 ms per step against 3.10-3.19 ms, so wider windows keep the two calls.
    FUSE_MAX_REPLICAS = 8

    def __init__(self, plan: zb.Plan, rank: int, n_windows: int, hyper: Hyper, max_norm: float,
                 device: torch.device, gather: bool = True, offload: bool = False,
                 offload_chunk: int = 1 << 21, host_threads: int = 0, fuse: bool = True,
                 per_param: bool = False, device_step: bool = False):
        if per_param and offload:
            raise ValueError("per-parameter state and ZeRO-Offload are separate layouts")
        if device_step and offload:
            raise ValueError("the device-counted step takes device state, not ZeRO-Offload's")
        self.plan, self.rank, self.hyper, self.max_norm = plan, rank, hyper, max_norm
        self.device = device
        self.offload, self.host_threads = offload, host_threads
        self.fuse, self.per_param = fuse, per_param
        s, nd = plan.shard_numel, plan.num_ranks
        # The arrays the AdamW kernel streams live in one arena, each start
        # moved STAGGER bytes past the previous end (the value measured best
        # on MI355X; see STAGGER).
        self.segments = plan.segments(rank) if per_param else []
        if per_param:
            views, self.arena = _staggered_arena([(s, torch.int16), (s, torch.int16)], device)
            self.grad, own_param = views
            self.master = self.exp_avg = self.exp_avg_sq = None
            lens = [ln for (_, _, _, ln) in self.segments]
            self.master_tensors = [torch.zeros(n, dtype=torch.float32, device=device) for n in lens]
            self.exp_avg_tensors = [torch.zeros(n, dtype=torch.float32, device=device) for n in lens]
            self.exp_avg_sq_tensors = [torch.zeros(n, dtype=torch.float32, device=device) for n in lens]
        elif offload:
            views, self.arena = _staggered_arena([(s, torch.int16), (s, torch.int16)], device)
            self.grad, own_param = views
            self.master = torch.zeros(s, dtype=torch.float32)
            self.exp_avg = torch.zeros(s, dtype=torch.float32)
            self.exp_avg_sq = torch.zeros(s, dtype=torch.float32)
            self.staging = torch.empty(4 * max(int(offload_chunk), 1), dtype=torch.int16).pin_memory()
        else:
            views, self.arena = _staggered_arena(
                [(s, torch.float32), (s, torch.float32), (s, torch.float32), (s, torch.int16),
                 (s, torch.int16)], device)
            self.master, self.exp_avg, self.exp_avg_sq, self.grad, own_param = views
        # per-rank partials [0, N_d) (own slot left 0), then one per own window
        self.partials = torch.zeros(nd + n_windows, dtype=torch.float64, device=device)
        self.scale = torch.ones(1, dtype=torch.float32, device=device)
        # other ranks' shards (gather inputs) exist only when this step gathers
        self.param_shards = [own_param if r == rank else
                             (torch.zeros(s, dtype=torch.int16, device=device) if gather else None)
                             for r in range(nd)]
        self.tensors: List[torch.Tensor] = []
        if gather:
            self.tensors = [torch.empty(max(n, 0), dtype=torch.int16, device=device)
                            for n in plan_numels(plan)]
        # sized for the one-pass reduce (or squared norm) of as much as the whole shard
        self.workspace = zb.reduce_workspace(s, device)
        self.n_windows = n_windows
        self.t = 0
        self.device_step = device_step
        self.schedule = None
        if device_step:
            with torch.cuda.device(device):
                self.schedule = zb.AdamWSchedule(hyper.lr, hyper.beta1, hyper.beta2, hyper.eps,
                                                 hyper.weight_decay)
        self._calls = {}

    def set_remote_partials(self, partials: Sequence[float]) -> None:
        p = torch.tensor(list(partials), dtype=torch.float64)
        p[self.rank] = 0.0
        self.partials[:self.plan.num_ranks].copy_(p.to(self.device))

    def _prepared(self, key, stream, build, sig=None):
        """Marshal a call's arguments once and reuse them while the stream and
        `sig` (the caller's buffers) stay the same. One entry per key: a new
        signature replaces the old entry and releases the buffers it held."""
        if stream is None:
            stream = torch.cuda.current_stream(self.device).cuda_stream
        cached = self._calls.get(key)
        if cached is None or cached[0] != stream or cached[1] != sig:
            cached = (stream, sig, build(stream))
            self._calls[key] = cached
        return cached[2]

    def reduce(self, windows: Sequence[Tuple[int, int, Sequence[torch.Tensor]]], stream=None):
        """windows: (begin, count, replica tensors) per window, in arrival order."""
        if len(windows) != self.n_windows:
            raise ValueError("window count differs from the one the step was built for")
        nd = self.plan.num_ranks
        for w, (begin, count, reps) in enumerate(windows):
            sig = (begin, count, tuple(r.data_ptr() for r in reps))
            self._prepared(("reduce", w), stream, lambda st: zb.prepare_grad_reduce_shard(
                self.plan, self.rank, reps, begin, count, self.grad,
                self.partials[nd + w:nd + w + 1], self.workspace, st), sig)()

    def reduce_tensors(self, replicas: Sequence[Sequence[torch.Tensor]], stream=None):
        """The reduce from replicas that are still per-tensor (replicas[k][t]
        = replica k's tensor t), through a zero_reduce_table built on first use
        for these buffers: the same gradient as flattening every replica and
        calling reduce() over the whole flat buffer, with the rank's norm
        partial in the one window slot (the step must be built with
        n_windows=1)."""
        if self.n_windows != 1:
            raise ValueError("the per-tensor reduce fills one window slot: build the step with n_windows=1")
        nd = self.plan.num_ranks
        sig = tuple(t.data_ptr() for rep in replicas for t in rep)
        self._prepared("reduce_tensors", stream, lambda st: zb.ReduceTable(
            self.plan, self.rank, replicas, self.grad).prepare_run(
                self.partials[nd:nd + 1], st), sig)()

    def clip(self, stream=None):
        if self.max_norm > 0:
            self._prepared("clip", stream, lambda st: zb.prepare_clip_scale(
                self.partials, self.max_norm, self.scale, st))()

    def adamw(self, stream=None):
        """The AdamW update with bias-correction step t = self.t + 1. self.t
        counts the iterations issued, skipped ones included: a non-finite global
        norm makes the kernel skip the update on the device, and nothing reports
        that back to the host inside a step, so after a skipped iteration the
        state holds one update fewer than t. (A caller that wants skipped
        iterations left uncounted reads the coefficient back, self.scale, and
        lowers self.t.)"""
        self.t += 1
        clip = self.scale if self.max_norm > 0 else None
        if self.device_step:    # the step's scalars on the device, then the count moves on
            if self.per_param:
                self._prepared("adamw", stream, lambda st: self._mt_table().prepare_step_scheduled(
                    self.schedule, clip_scale=clip, stream=st))()
            else:
                self._prepared("adamw", stream, lambda st: zb.prepare_shard_adamw_step_scheduled(
                    self.master, self.exp_avg, self.exp_avg_sq, self.grad, self.param_shards[self.rank],
                    self.schedule, clip_scale=clip, stream=st))()
            self._prepared("advance", stream, lambda st: self.schedule.prepare_advance(clip, st))()
            return
        if self.per_param:
            self._prepared("adamw", stream, lambda st: self._mt_table().prepare_step(
                clip_scale=clip, stream=st, **self.hyper.as_kwargs()))(self.t)
            return
        if self.offload:        # returns once the host update is done; `stream` orders the copies
            self._prepared("adamw", stream, lambda st: zb.prepare_offload_adamw_step(
                self.master, self.exp_avg, self.exp_avg_sq, self.grad, self.param_shards[self.rank],
                self.staging, clip_scale=clip, stream=st, n_threads=self.host_threads,
                **self.hyper.as_kwargs()))(self.t)
            return
        self._prepared("adamw", stream, lambda st: zb.prepare_shard_adamw_step(
            self.master, self.exp_avg, self.exp_avg_sq, self.grad, self.param_shards[self.rank],
            clip_scale=clip, stream=st, **self.hyper.as_kwargs()))(self.t)

    def _mt_table(self) -> zb.MultiTensorTable:
        """The per-parameter state's device table (the gradient and the parameter
        shard cut at the segments)."""
        own = self.param_shards[self.rank]
        sl = [slice(soff, soff + ln) for (_, _, soff, ln) in self.segments]
        return zb.MultiTensorTable(self.master_tensors, self.exp_avg_tensors, self.exp_avg_sq_tensors,
                                   [self.grad[x] for x in sl], [own[x] for x in sl])

    def steps_applied(self) -> int:
        """Updates applied: the device count with device_step (a synchronous read),
        else self.t (iterations issued, skipped ones included)."""
        return self.schedule.applied() if self.device_step else self.t

    def reduce_update(self, windows: Sequence[Tuple[int, int, Sequence[torch.Tensor]]],
                      stream=None):
        """reduce() then adamw() with no clip, as one pass per window
        (zero_reduce_adamw_step), every window with the bias-correction step
        t = self.t + 1. The update is elementwise, so over disjoint windows this
        is the same as the two calls; overlapping windows raise ValueError. The
        averaged gradient is not stored and no norm partial is taken."""
        if len(windows) != self.n_windows:
            raise ValueError("window count differs from the one the step was built for")
        if self.offload or self.per_param or self.max_norm > 0:
            raise ValueError("the one-pass update runs on the device, over flat state, without "
                             "clipping")
        spans = sorted((b, b + c) for b, c, _ in windows if c > 0)
        if any(a[1] > b[0] for a, b in zip(spans, spans[1:])):
            raise ValueError("windows overlap: the one-pass update needs disjoint windows")
        self.t += 1
        for w, (begin, count, reps) in enumerate(windows):
            sig = (begin, count, tuple(r.data_ptr() for r in reps))
            if self.device_step:
                self._prepared(("reduce_update", w), stream, lambda st: zb.prepare_reduce_adamw_step_scheduled(
                    self.plan, self.rank, reps, begin, count, self.master, self.exp_avg,
                    self.exp_avg_sq, self.param_shards[self.rank], self.schedule, stream=st), sig)()
            else:
                self._prepared(("reduce_update", w), stream, lambda st: zb.prepare_reduce_adamw_step(
                    self.plan, self.rank, reps, begin, count, self.master, self.exp_avg,
                    self.exp_avg_sq, self.param_shards[self.rank], clip_scale=None, stream=st,
                    **self.hyper.as_kwargs()), sig)(self.t)
        if self.device_step:    # every window updated: the step counts once
            self._prepared("advance", stream, lambda st: self.schedule.prepare_advance(None, st))()

    def gather(self, stream=None):
        # The shards and tensors are this object's fixed buffers, so the gather
        # goes through a device-resident copy table, built on first use.
        if self.tensors:
            self._prepared("gather", stream, lambda st: zb.CopyTable.gather(
                self.plan, self.param_shards, self.tensors).prepare_run(st))()

    def step(self, windows, stream=None) -> None:
        spans = sorted((b, b + c) for b, c, _ in windows if c > 0)
        disjoint = all(a[1] <= b[0] for a, b in zip(spans, spans[1:]))
        narrow = all(len(reps) <= self.FUSE_MAX_REPLICAS for _, _, reps in windows)
        if (self.fuse and self.max_norm <= 0 and not self.offload and not self.per_param
                and disjoint and narrow):
            self.reduce_update(windows, stream)
        else:
            self.reduce(windows, stream)
            self.clip(stream)
            self.adamw(stream)
        self.gather(stream)


# Gap between consecutive arrays of an arena (and between replica buffers).
# Measured on MI355X over the benchmark's steps, two runs each: 2048 bytes was
# the fastest or level on every workload; against 4352 bytes it took the 1.3B
# GPT step from 10.04 to 9.83-9.88 ms, Llama-3-8B's from 3.12 to 3.06 ms and
# Llama-3-70B's from 40.51-40.55 to 40.10-40.11 ms (AdamW 81.5% -> 82.2% of
# HBM peak); 0 (packed) was level with 2048 except on the 1.3B GPT (10.02 ms).
STAGGER = 2048


def _staggered_arena(specs, device):
    """One zeroed allocation holding arrays of (numel, dtype), 256-byte aligned
    starts, STAGGER bytes between the end of one array and the next start."""
    offsets, off = [], 0
    for numel, dtype in specs:
        nbytes = numel * torch.empty(0, dtype=dtype).element_size()
        offsets.append((off, nbytes, dtype))
        off += (nbytes + 255) // 256 * 256 + STAGGER
    arena = torch.zeros(max(off, 1), dtype=torch.uint8, device=device)
    views = [arena[o:o + nb].view(dt) for o, nb, dt in offsets]
    return views, arena


def staggered_replicas(n_replicas: int, numel: int, device) -> List[torch.Tensor]:
    """R bf16 buffers of numel elements in one allocation, STAGGER bytes apart
    (the reduce reads the replica streams in lockstep)."""
    views, _ = _staggered_arena([(numel, torch.int16)] * n_replicas, device)
    return views      # each view keeps the shared allocation alive


def plan_numels(plan: zb.Plan) -> List[int]:
    return [plan.tensor_numel(i) for i in range(plan.num_tensors)]


def bucket_windows(padded_numel: int, bucket: int, lo: int, hi: int) -> List[Tuple[int, int]]:
    """Fixed-size flat-index buckets [b*bucket, (b+1)*bucket) meeting [lo, hi), in
    backward (descending) order, each clipped to the padded buffer."""
    out = []
    if bucket <= 0:
        return [(0, padded_numel)]
    first, last = lo // bucket, (hi - 1) // bucket
    for b in range(last, first - 1, -1):
        begin = b * bucket
        out.append((begin, min(bucket, padded_numel - begin)))
    return out


def rank_step_plan_windows(plan: zb.Plan, rank: int, bucket: int) -> List[Tuple[int, int]]:
    s = plan.shard_numel
    return bucket_windows(plan.padded_numel, bucket, rank * s, (rank + 1) * s)


def optional_stream(stream: Optional[torch.cuda.Stream]):
    return None if stream is None else stream.cuda_stream
