"""ctypes binding of libzero_mi355x.so: the same entry points, argument marshalling only.

Device buffers are torch tensors on a ROCm device (torch supplies memory and
streams, nothing else); every computation runs in the library's HIP kernels.
If the library is not built, importing this module raises: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence, Tuple

# ZERO_MI355X_LIB may name another build of the same sources (one built with
# other compile-time switches by _build.py, for a measured comparison).
LIB_PATH = os.environ.get("ZERO_MI355X_LIB") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libzero_mi355x.so")

ZERO_OK, ZERO_EINVAL, ZERO_ERANGE, ZERO_ENOMEM, ZERO_EHIP, ZERO_ENOSPACE = range(6)
ZERO_MAX_REPLICAS = 64

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                      "(hipcc, gfx950); there is no CPU fallback")

_lib = ctypes.CDLL(LIB_PATH)

c_i32, c_i64, c_dbl, c_sz, c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_double, ctypes.c_size_t, \
    ctypes.c_void_p


class zero_segment(ctypes.Structure):
    _fields_ = [("tensor", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("tensor_offset", ctypes.c_int64), ("shard_offset", ctypes.c_int64),
                ("length", ctypes.c_int64)]


def _fn(name, restype, argtypes):
    f = getattr(_lib, name)
    f.restype = restype
    f.argtypes = argtypes
    return f


_partition_plan = _fn("zero_partition_plan", c_i32,
                      [ctypes.POINTER(c_i64), c_i32, c_i32, c_i32, ctypes.POINTER(c_vp)])
_plan_shard0 = _fn("zero_partition_plan_shard0", c_i32,
                   [ctypes.POINTER(c_i64), ctypes.POINTER(c_i64), c_i32, c_i32, c_i32,
                    ctypes.POINTER(c_vp)])
_plan_kind = _fn("zero_plan_kind", c_i32, [c_vp])
_plan_tnumel = _fn("zero_plan_tensor_numel", c_i64, [c_vp, c_i32])
_plan_free = _fn("zero_plan_free", None, [c_vp])
_plan_numel = _fn("zero_plan_numel", c_i64, [c_vp])
_plan_padded = _fn("zero_plan_padded_numel", c_i64, [c_vp])
_plan_shard = _fn("zero_plan_shard_numel", c_i64, [c_vp])
_plan_ntensors = _fn("zero_plan_num_tensors", c_i32, [c_vp])
_plan_nranks = _fn("zero_plan_num_ranks", c_i32, [c_vp])
_plan_offset = _fn("zero_plan_tensor_offset", c_i64, [c_vp, c_i32])
_plan_nsegs = _fn("zero_plan_num_segments", c_i32, [c_vp, c_i32])
_plan_segments = _fn("zero_plan_segments", c_i32,
                     [c_vp, c_i32, ctypes.POINTER(zero_segment), c_i32, ctypes.POINTER(c_i32)])
_plan_memory = _fn("zero_plan_memory_bytes", c_i32, [c_vp, c_i32, c_i32, ctypes.POINTER(c_dbl)])
_reduce = _fn("zero_grad_reduce_shard", c_i32,
              [c_vp, c_i32, ctypes.POINTER(c_vp), c_i32, c_i64, c_i64, c_vp, c_vp, c_vp, c_sz, c_vp])
_reduce_noalloc = _fn("zero_grad_reduce_shard_noalloc", c_i32,
                      [c_vp, c_i32, ctypes.POINTER(c_vp), c_i32, c_i64, c_i64, c_vp, c_vp, c_vp])
_sqnorm = _fn("zero_grad_sqnorm", c_i32, [c_vp, c_i64, c_vp, c_vp, c_sz, c_vp])
_ws_bytes = _fn("zero_sqnorm_workspace_bytes", c_sz, [])
_rws_bytes = _fn("zero_reduce_workspace_bytes", c_sz, [c_i64])
_clip = _fn("zero_clip_scale", c_i32, [c_vp, c_i32, c_dbl, c_vp, c_vp])
_adamw = _fn("zero_shard_adamw_step", c_i32,
             [c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_dbl, c_dbl, c_dbl, c_dbl, c_dbl, c_vp,
              c_vp])
_reduce_adamw = _fn("zero_reduce_adamw_step", c_i32,
                    [c_vp, c_i32, ctypes.POINTER(c_vp), c_i32, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp,
                     c_vp, c_i64, c_dbl, c_dbl, c_dbl, c_dbl, c_dbl, c_vp, c_vp])
_gather = _fn("zero_gather_params", c_i32, [c_vp, ctypes.POINTER(c_vp), ctypes.POINTER(c_vp), c_vp])
_flatten = _fn("zero_flatten_params", c_i32, [c_vp, ctypes.POINTER(c_vp), c_vp, c_vp])
_host_adamw = _fn("zero_host_adamw_step", c_i32,
                  [c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_dbl, c_dbl, c_dbl, c_dbl, c_dbl,
                   ctypes.c_float, c_i32])
_offload = _fn("zero_offload_adamw_step", c_i32,
               [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_dbl, c_dbl, c_dbl, c_dbl,
                c_dbl, c_vp, c_i32, c_vp])
_mt_adamw = _fn("zero_multi_tensor_adamw_step", c_i32,
                [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i64, c_dbl, c_dbl, c_dbl, c_dbl, c_dbl,
                 c_vp, c_vp])
_mt_create = _fn("zero_mt_table_create", c_i32,
                 [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, ctypes.POINTER(c_vp)])
_mt_free = _fn("zero_mt_table_free", None, [c_vp])
_mt_blocks = _fn("zero_mt_table_blocks", c_i64, [c_vp])
_mt_step = _fn("zero_mt_table_adamw_step", c_i32,
               [c_vp, c_i64, c_dbl, c_dbl, c_dbl, c_dbl, c_dbl, c_vp, c_vp])
_gt_create = _fn("zero_gather_table_create", c_i32,
                 [c_vp, ctypes.POINTER(c_vp), ctypes.POINTER(c_vp), ctypes.POINTER(c_vp)])
_ft_create = _fn("zero_flatten_table_create", c_i32,
                 [c_vp, ctypes.POINTER(c_vp), c_vp, ctypes.POINTER(c_vp)])
_ct_run = _fn("zero_copy_table_run", c_i32, [c_vp, c_vp])
_ct_blocks = _fn("zero_copy_table_blocks", c_i64, [c_vp])
_ct_free = _fn("zero_copy_table_free", None, [c_vp])
_rt_create = _fn("zero_reduce_table_create", c_i32,
                 [c_vp, c_i32, ctypes.POINTER(c_vp), c_i32, c_vp, ctypes.POINTER(c_vp)])
_rt_run = _fn("zero_reduce_table_run", c_i32, [c_vp, c_vp, c_vp])
_sched_create = _fn("zero_adamw_schedule_create", c_i32,
                    [ctypes.POINTER(c_dbl), c_i64, c_dbl, c_dbl, c_dbl, c_dbl, c_i64, ctypes.POINTER(c_vp)])
_sched_free = _fn("zero_adamw_schedule_free", None, [c_vp])
_sched_length = _fn("zero_adamw_schedule_length", c_i64, [c_vp])
_sched_applied = _fn("zero_adamw_schedule_applied", c_i32, [c_vp, ctypes.POINTER(c_i64)])
_sched_advance = _fn("zero_adamw_schedule_advance", c_i32, [c_vp, c_vp, c_vp])
_adamw_sched = _fn("zero_shard_adamw_step_scheduled", c_i32,
                   [c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_vp, c_vp, c_vp])
_mt_step_sched = _fn("zero_mt_table_adamw_step_scheduled", c_i32, [c_vp, c_vp, c_vp, c_vp])
_reduce_adamw_sched = _fn("zero_reduce_adamw_step_scheduled", c_i32,
                          [c_vp, c_i32, ctypes.POINTER(c_vp), c_i32, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp,
                           c_vp, c_vp, c_vp, c_vp])
_step_scalars = _fn("zero_adamw_step_scalars", c_i32,
                    [c_i64, c_dbl, c_dbl, c_dbl, c_dbl, c_dbl, ctypes.POINTER(ctypes.c_float)])
_rt_blocks = _fn("zero_reduce_table_blocks", c_i64, [c_vp])
_rt_free = _fn("zero_reduce_table_free", None, [c_vp])
_status_string = _fn("zero_status_string", ctypes.c_char_p, [c_i32])
_last_error = _fn("zero_last_error", ctypes.c_char_p, [])


class ZeroError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        detail = _last_error().decode()
        super().__init__(f"{where}: {_status_string(status).decode()} ({detail})")


def _check(status: int, where: str) -> None:
    if status != ZERO_OK:
        raise ZeroError(status, where)


# --------------------------------------------------------------------------- plan

class Plan:
    """Owner of a zero_plan handle."""

    def __init__(self, handle: int):
        self._h = c_vp(handle)
        # held by the instance: at interpreter exit the module's globals may be
        # cleared before the last plan is collected
        self._free = _plan_free

    def __del__(self):
        h = getattr(self, "_h", None)
        free = getattr(self, "_free", None)
        if h is not None and h.value and free is not None:
            free(h)
            h.value = None      # no module globals here: they may be gone at exit

    @property
    def handle(self) -> c_vp:
        return self._h

    @property
    def numel(self) -> int:
        return _plan_numel(self._h)

    @property
    def padded_numel(self) -> int:
        return _plan_padded(self._h)

    @property
    def shard_numel(self) -> int:
        return _plan_shard(self._h)

    @property
    def num_tensors(self) -> int:
        return _plan_ntensors(self._h)

    @property
    def num_ranks(self) -> int:
        return _plan_nranks(self._h)

    @property
    def kind(self) -> int:
        """0: flat (FSDP-1 / ZeRO) layout; 1: FSDP-2 per-parameter Shard(0) layout."""
        return _plan_kind(self._h)

    def tensor_offset(self, t: int) -> int:
        return _plan_offset(self._h, t)

    def tensor_numel(self, t: int) -> int:
        return _plan_tnumel(self._h, t)

    def num_segments(self, rank: int) -> int:
        return _plan_nsegs(self._h, rank)

    def segments(self, rank: int) -> List[Tuple[int, int, int, int]]:
        """(tensor, offset in tensor, offset in shard, length) in flat order."""
        n = _plan_nsegs(self._h, rank)
        if n < 0:
            raise ValueError("rank out of range")
        arr = (zero_segment * max(n, 1))()
        count = c_i32(0)
        _check(_plan_segments(self._h, rank, arr, n, ctypes.byref(count)), "zero_plan_segments")
        return [(s.tensor, s.tensor_offset, s.shard_offset, s.length) for s in arr[:count.value]]

    def memory_bytes(self, stage: int, padded: bool = False) -> float:
        out = c_dbl(0.0)
        _check(_plan_memory(self._h, stage, int(padded), ctypes.byref(out)),
               "zero_plan_memory_bytes")
        return out.value


def zero_partition_plan_shard0(numels: Sequence[int], dim0: Sequence[int], n_ranks: int,
                               align_elems: int = 128) -> Plan:
    n = len(numels)
    if len(dim0) != n:
        raise ValueError("one dim0 per tensor")
    arr = (c_i64 * max(n, 1))(*[int(x) for x in numels])
    d0 = (c_i64 * max(n, 1))(*[int(x) for x in dim0])
    h = c_vp(None)
    _check(_plan_shard0(arr, d0, n, n_ranks, align_elems, ctypes.byref(h)),
           "zero_partition_plan_shard0")
    return Plan(h.value)


def zero_partition_plan(numels: Sequence[int], n_ranks: int, align_elems: int = 128) -> Plan:
    arr = (c_i64 * max(len(numels), 1))(*[int(n) for n in numels])
    h = c_vp(None)
    _check(_partition_plan(arr, len(numels), n_ranks, align_elems, ctypes.byref(h)),
           "zero_partition_plan")
    return Plan(h.value)


# --------------------------------------------------------------------------- device calls

def _stream(stream, tensor) -> int:
    if stream is not None:
        return int(stream)
    import torch
    return torch.cuda.current_stream(tensor.device).cuda_stream


def _ptr(t, elem_size: int, what: str) -> int:
    if t is None:
        return 0
    if not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor")
    if t.element_size() != elem_size:
        raise ValueError(f"{what} must have {elem_size}-byte elements")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return t.data_ptr()


def _need(t, n: int, what: str) -> None:
    """The C ABI receives bare device pointers and cannot see buffer sizes:
    refuse here a tensor shorter than what the call will read or write."""
    if t is not None and t.numel() < n:
        raise ValueError(f"{what} holds {t.numel()} elements; the call touches {n}")


def _check_reduce_args(plan: "Plan", replicas, count: int, shard_grad, sqnorm_out) -> None:
    for r in replicas:
        _need(r, count, "a replica")
    _need(shard_grad, plan.shard_numel, "shard_grad")
    _need(sqnorm_out, 1, "sqnorm_out")


def _check_gather_args(plan: "Plan", shards, tensors) -> None:
    if len(shards) != plan.num_ranks or len(tensors) != plan.num_tensors:
        raise ValueError("need N_d shards and T tensors")
    for sh in shards:
        _need(sh, plan.shard_numel, "a shard")
    for i, t in enumerate(tensors):
        _need(t, plan.tensor_numel(i), f"tensor {i}")


def _check_flatten_args(plan: "Plan", tensors, flat) -> None:
    if len(tensors) != plan.num_tensors:
        raise ValueError("need T tensors")
    _need(flat, plan.padded_numel, "flat")
    for i, t in enumerate(tensors):
        _need(t, plan.tensor_numel(i), f"tensor {i}")


def _check_adamw_args(n: int, arrays, clip_scale) -> None:
    for t, what in zip(arrays, ("master", "exp_avg", "exp_avg_sq", "grad", "param_out")):
        _need(t, n, what)
    _need(clip_scale, 1, "clip_scale")


_ws_cache = {}


def sqnorm_workspace(device) -> "object":
    """A cached device workspace of zero_sqnorm_workspace_bytes() bytes (torch-allocated),
    one per device, used by every call that passes no workspace of its own. Calls
    issued on different streams that may overlap must pass their own workspaces."""
    import torch
    dev = torch.device(device)
    key = (dev.type, dev.index if dev.index is not None else torch.cuda.current_device())
    ws = _ws_cache.get(key)
    if ws is None:
        ws = torch.empty(_ws_bytes(), dtype=torch.uint8, device=dev)
        _ws_cache[key] = ws
    return ws


def zero_sqnorm_workspace_bytes() -> int:
    return _ws_bytes()


def zero_reduce_workspace_bytes(count: int) -> int:
    return int(_rws_bytes(int(count)))


def reduce_workspace(count: int, device) -> "object":
    """A new device workspace of zero_reduce_workspace_bytes(count) bytes: with it,
    zero_grad_reduce_shard takes its one-pass kernel, with the norm, on windows
    of up to count elements."""
    import torch
    return torch.empty(zero_reduce_workspace_bytes(count), dtype=torch.uint8, device=torch.device(device))


def zero_grad_reduce_shard(plan: Plan, rank: int, replicas: Sequence, begin: int, count: int,
                           shard_grad, sqnorm_out=None, workspace=None, stream=None) -> None:
    """replicas: R device tensors (2-byte elements) covering flat window [begin, begin+count)."""
    _check_reduce_args(plan, replicas, count, shard_grad, sqnorm_out)
    ptrs = (c_vp * max(len(replicas), 1))(*[_ptr(r, 2, "replica") for r in replicas])
    out = _ptr(shard_grad, 2, "shard_grad")
    sq = _ptr(sqnorm_out, 8, "sqnorm_out")
    if sqnorm_out is not None and workspace is None:
        workspace = sqnorm_workspace(shard_grad.device)
    ws = workspace.data_ptr() if workspace is not None else 0
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_reduce(plan.handle, rank, ptrs, len(replicas), begin, count, out, sq, ws, wsb,
                   _stream(stream, shard_grad)), "zero_grad_reduce_shard")


ZERO_NOALLOC_SCRATCH_BYTES = 4 << 20


def zero_grad_reduce_shard_noalloc(plan: Plan, rank: int, replicas: Sequence, begin: int, count: int,
                                   shard_grad, sqnorm_out=None, stream=None) -> None:
    """zero_grad_reduce_shard with the norm partials in the library's own device
    array: no workspace, no allocation. Calls that may overlap on one device race."""
    _check_reduce_args(plan, replicas, count, shard_grad, sqnorm_out)
    ptrs = (c_vp * max(len(replicas), 1))(*[_ptr(r, 2, "replica") for r in replicas])
    _check(_reduce_noalloc(plan.handle, rank, ptrs, len(replicas), begin, count,
                           _ptr(shard_grad, 2, "shard_grad"), _ptr(sqnorm_out, 8, "sqnorm_out"),
                           _stream(stream, shard_grad)), "zero_grad_reduce_shard_noalloc")


def zero_grad_sqnorm(grad, sqnorm_out, n: Optional[int] = None, workspace=None, stream=None) -> None:
    n = grad.numel() if n is None else n
    _need(grad, n, "grad")
    _need(sqnorm_out, 1, "sqnorm_out")
    if workspace is None:
        workspace = sqnorm_workspace(grad.device)
    _check(_sqnorm(_ptr(grad, 2, "grad"), n, _ptr(sqnorm_out, 8, "sqnorm_out"), workspace.data_ptr(),
                   workspace.numel() * workspace.element_size(), _stream(stream, grad)),
           "zero_grad_sqnorm")


def zero_clip_scale(partials, max_norm: float, scale_out, n_partials: Optional[int] = None,
                    stream=None) -> None:
    n = partials.numel() if n_partials is None else n_partials
    _need(partials, n, "partials")
    _need(scale_out, 1, "scale_out")
    _check(_clip(_ptr(partials, 8, "partials"), n, float(max_norm), _ptr(scale_out, 4, "scale_out"),
                 _stream(stream, partials)), "zero_clip_scale")


def zero_shard_adamw_step(master, exp_avg, exp_avg_sq, grad, param_out, step: int, lr: float,
                          beta1: float, beta2: float, eps: float, weight_decay: float,
                          clip_scale=None, n: Optional[int] = None, stream=None) -> None:
    n = master.numel() if n is None else n
    _check_adamw_args(n, (master, exp_avg, exp_avg_sq, grad, param_out), clip_scale)
    _check(_adamw(_ptr(master, 4, "master"), _ptr(exp_avg, 4, "exp_avg"),
                  _ptr(exp_avg_sq, 4, "exp_avg_sq"), _ptr(grad, 2, "grad"),
                  _ptr(param_out, 2, "param_out"), n, step, lr, beta1, beta2, eps, weight_decay,
                  _ptr(clip_scale, 4, "clip_scale"), _stream(stream, master)),
           "zero_shard_adamw_step")


def prepare_reduce_adamw_step(plan: Plan, rank: int, replicas: Sequence, begin: int, count: int,
                              master, exp_avg, exp_avg_sq, param_out, lr: float, beta1: float,
                              beta2: float, eps: float, weight_decay: float, clip_scale=None,
                              shard_grad=None, stream=None) -> "Prepared":
    """zero_reduce_adamw_step with its arguments marshalled once; call the result
    with the 1-based step number. The state arrays are the rank's shard ([S])."""
    S = plan.shard_numel
    for r in replicas:
        _need(r, count, "a replica")
    for t, what in ((master, "master"), (exp_avg, "exp_avg"), (exp_avg_sq, "exp_avg_sq"),
                    (param_out, "param_out")):
        _need(t, S, what)
    _need(shard_grad, S, "shard_grad")
    _need(clip_scale, 1, "clip_scale")
    ptrs = (c_vp * max(len(replicas), 1))(*[_ptr(r, 2, "replica") for r in replicas])
    p = Prepared(_reduce_adamw, [plan.handle, rank, ptrs, len(replicas), begin, count,
                                 _ptr(master, 4, "master"), _ptr(exp_avg, 4, "exp_avg"),
                                 _ptr(exp_avg_sq, 4, "exp_avg_sq"), _ptr(param_out, 2, "param_out"),
                                 _ptr(shard_grad, 2, "shard_grad"), 1, lr, beta1, beta2, eps,
                                 weight_decay, _ptr(clip_scale, 4, "clip_scale"),
                                 _stream(stream, master)], "zero_reduce_adamw_step", step_index=11)
    p._keep = (ptrs, replicas, master, exp_avg, exp_avg_sq, param_out, shard_grad, clip_scale)
    return p


def zero_reduce_adamw_step(plan: Plan, rank: int, replicas: Sequence, begin: int, count: int,
                           master, exp_avg, exp_avg_sq, param_out, step: int, lr: float,
                           beta1: float, beta2: float, eps: float, weight_decay: float,
                           clip_scale=None, shard_grad=None, stream=None) -> None:
    """The rank's averaged gradient and its AdamW update in one pass (no global
    norm between them): the bits of zero_grad_reduce_shard then zero_shard_adamw_step."""
    prepare_reduce_adamw_step(plan, rank, replicas, begin, count, master, exp_avg, exp_avg_sq,
                              param_out, lr, beta1, beta2, eps, weight_decay, clip_scale, shard_grad,
                              stream)(step)


def prepare_reduce_adamw_step_scheduled(plan: Plan, rank: int, replicas: Sequence, begin: int,
                                        count: int, master, exp_avg, exp_avg_sq, param_out,
                                        schedule: "AdamWSchedule", clip_scale=None, shard_grad=None,
                                        stream=None) -> "Prepared":
    """zero_reduce_adamw_step_scheduled with its arguments marshalled once."""
    S = plan.shard_numel
    for r in replicas:
        _need(r, count, "a replica")
    for t, what in ((master, "master"), (exp_avg, "exp_avg"), (exp_avg_sq, "exp_avg_sq"),
                    (param_out, "param_out")):
        _need(t, S, what)
    _need(shard_grad, S, "shard_grad")
    _need(clip_scale, 1, "clip_scale")
    ptrs = (c_vp * max(len(replicas), 1))(*[_ptr(r, 2, "replica") for r in replicas])
    p = Prepared(_reduce_adamw_sched, [plan.handle, rank, ptrs, len(replicas), begin, count,
                                       _ptr(master, 4, "master"), _ptr(exp_avg, 4, "exp_avg"),
                                       _ptr(exp_avg_sq, 4, "exp_avg_sq"), _ptr(param_out, 2, "param_out"),
                                       _ptr(shard_grad, 2, "shard_grad"), schedule.handle,
                                       _ptr(clip_scale, 4, "clip_scale"), _stream(stream, master)],
                 "zero_reduce_adamw_step_scheduled")
    p._keep = (ptrs, replicas, master, exp_avg, exp_avg_sq, param_out, shard_grad, schedule, clip_scale)
    return p


def zero_reduce_adamw_step_scheduled(plan: Plan, rank: int, replicas: Sequence, begin: int, count: int,
                                     master, exp_avg, exp_avg_sq, param_out, schedule: "AdamWSchedule",
                                     clip_scale=None, shard_grad=None, stream=None) -> None:
    """zero_reduce_adamw_step with the step's scalars read on the device from `schedule`."""
    prepare_reduce_adamw_step_scheduled(plan, rank, replicas, begin, count, master, exp_avg, exp_avg_sq,
                                        param_out, schedule, clip_scale, shard_grad, stream)()


def zero_gather_params(plan: Plan, shards: Sequence, tensors: Sequence, stream=None) -> None:
    _check_gather_args(plan, shards, tensors)
    sp = (c_vp * max(len(shards), 1))(*[_ptr(s, 2, "shard") for s in shards])   # None skips a rank
    tp = (c_vp * max(len(tensors), 1))(*[_ptr(t, 2, "tensor") for t in tensors])
    ref = next((x for x in list(shards) + list(tensors) if x is not None), None)
    _check(_gather(plan.handle, sp, tp, _stream(stream, ref) if ref is not None else 0),
           "zero_gather_params")


def zero_flatten_params(plan: Plan, tensors: Sequence, flat, stream=None) -> None:
    """tensors: T device buffers (2-byte elements, numel_t each); flat: device [P]."""
    _check_flatten_args(plan, tensors, flat)
    tp = (c_vp * max(len(tensors), 1))(*[_ptr(t, 2, "tensor") for t in tensors])
    _check(_flatten(plan.handle, tp, _ptr(flat, 2, "flat"), _stream(stream, flat)),
           "zero_flatten_params")


def prepare_multi_tensor_adamw_step(masters, exp_avgs, exp_avg_sqs, grads, params_out, lr: float,
                                    beta1: float, beta2: float, eps: float, weight_decay: float,
                                    clip_scale, stream) -> Prepared:
    """Lists of T device tensors (fp32 state; 2-byte grads and params), tensor t
    updated over masters[t].numel() elements. Call the result with the step."""
    lists = (masters, exp_avgs, exp_avg_sqs, grads, params_out)
    T = len(masters)
    if any(len(x) != T for x in lists):
        raise ValueError("the five lists must have the same length")
    numels = [t.numel() for t in masters]
    for lst in lists[1:]:
        if any(x.numel() < n for x, n in zip(lst, numels)):
            raise ValueError("a tensor holds fewer elements than its master")
    _need(clip_scale, 1, "clip_scale")
    tabs = []
    for lst, size, what in zip(lists, (4, 4, 4, 2, 2), ("master", "exp_avg", "exp_avg_sq", "grad", "param")):
        tabs.append((c_vp * max(T, 1))(*[_ptr(x, size, what) for x in lst]))
    ns = (c_i64 * max(T, 1))(*numels)
    st = _stream(stream, masters[0]) if T else (stream or 0)
    p = Prepared(_mt_adamw, tabs + [ns, T, 1, lr, beta1, beta2, eps, weight_decay,
                                    _ptr(clip_scale, 4, "clip_scale"), st],
                 "zero_multi_tensor_adamw_step", step_index=7)
    p._keep = (lists, tabs, ns, clip_scale)
    return p


def zero_multi_tensor_adamw_step(masters, exp_avgs, exp_avg_sqs, grads, params_out, step: int,
                                 lr: float, beta1: float, beta2: float, eps: float,
                                 weight_decay: float, clip_scale=None, stream=None) -> None:
    prepare_multi_tensor_adamw_step(masters, exp_avgs, exp_avg_sqs, grads, params_out, lr, beta1,
                                    beta2, eps, weight_decay, clip_scale, stream)(step)


class MultiTensorTable:
    """Owner of a zero_mt_table: a fixed list of per-parameter tensors described
    once in device memory (on the current device), stepped in one launch. The
    tensors are held here, so their buffers outlive the table."""

    def __init__(self, masters, exp_avgs, exp_avg_sqs, grads, params_out):
        lists = (masters, exp_avgs, exp_avg_sqs, grads, params_out)
        T = len(masters)
        if any(len(x) != T for x in lists):
            raise ValueError("the five lists must have the same length")
        numels = [t.numel() for t in masters]
        for lst in lists[1:]:
            if any(x.numel() < n for x, n in zip(lst, numels)):
                raise ValueError("a tensor holds fewer elements than its master")
        tabs = []
        for lst, size, what in zip(lists, (4, 4, 4, 2, 2),
                                   ("master", "exp_avg", "exp_avg_sq", "grad", "param")):
            tabs.append((c_vp * max(T, 1))(*[_ptr(x, size, what) for x in lst]))
        ns = (c_i64 * max(T, 1))(*numels)
        h = c_vp()
        _check(_mt_create(*tabs, ns, T, ctypes.byref(h)), "zero_mt_table_create")
        self._h = h
        self._free = _mt_free          # held by the instance for interpreter exit
        self._keep = lists
        self.device = masters[0].device if T else None

    def __del__(self):
        h = getattr(self, "_h", None)
        free = getattr(self, "_free", None)
        if h is not None and h.value and free is not None:
            free(h)
            h.value = None

    @property
    def handle(self) -> c_vp:
        return self._h

    @property
    def blocks(self) -> int:
        return int(_mt_blocks(self._h))

    def prepare_step(self, lr: float, beta1: float, beta2: float, eps: float,
                     weight_decay: float, clip_scale, stream) -> "Prepared":
        """zero_mt_table_adamw_step with its arguments marshalled once; call the
        result with the step."""
        _need(clip_scale, 1, "clip_scale")
        st = stream if stream is not None else (
            _stream(None, self._keep[0][0]) if self._keep[0] else 0)
        p = Prepared(_mt_step, [self._h, 1, lr, beta1, beta2, eps, weight_decay,
                                _ptr(clip_scale, 4, "clip_scale"), st],
                     "zero_mt_table_adamw_step", step_index=1)
        p._keep = (self, clip_scale)
        return p

    def step(self, step: int, lr: float, beta1: float, beta2: float, eps: float,
             weight_decay: float, clip_scale=None, stream=None) -> None:
        if clip_scale is not None:
            _need(clip_scale, 1, "clip_scale")
        st = stream if stream is not None else (
            _stream(None, self._keep[0][0]) if self._keep[0] else 0)
        _check(_mt_step(self._h, step, lr, beta1, beta2, eps, weight_decay,
                        _ptr(clip_scale, 4, "clip_scale"), st), "zero_mt_table_adamw_step")

    def prepare_step_scheduled(self, schedule: "AdamWSchedule", clip_scale=None, stream=None) -> "Prepared":
        """zero_mt_table_adamw_step_scheduled with its arguments marshalled once."""
        _need(clip_scale, 1, "clip_scale")
        st = stream if stream is not None else (
            _stream(None, self._keep[0][0]) if self._keep[0] else 0)
        p = Prepared(_mt_step_sched, [self._h, schedule.handle, _ptr(clip_scale, 4, "clip_scale"), st],
                     "zero_mt_table_adamw_step_scheduled")
        p._keep = (self, schedule, clip_scale)
        return p

    def step_scheduled(self, schedule: "AdamWSchedule", clip_scale=None, stream=None) -> None:
        self.prepare_step_scheduled(schedule, clip_scale, stream)()


class CopyTable:
    """Owner of a zero_copy_table: the gather (CopyTable.gather) or flatten
    (CopyTable.flatten) of fixed buffers, described once in device memory (on
    the current device) and run in one launch. The plan and the buffers are
    held here, so they outlive the table."""

    def __init__(self, handle: c_vp, keep):
        self._h = handle
        self._free = _ct_free          # held by the instance for interpreter exit
        self._keep = keep

    @classmethod
    def gather(cls, plan: Plan, shards: Sequence, tensors: Sequence) -> "CopyTable":
        _check_gather_args(plan, shards, tensors)
        sp = (c_vp * max(len(shards), 1))(*[_ptr(x, 2, "shard") for x in shards])
        tp = (c_vp * max(len(tensors), 1))(*[_ptr(t, 2, "tensor") for t in tensors])
        h = c_vp()
        _check(_gt_create(plan.handle, sp, tp, ctypes.byref(h)), "zero_gather_table_create")
        return cls(h, (plan, list(shards), list(tensors)))

    @classmethod
    def flatten(cls, plan: Plan, tensors: Sequence, flat) -> "CopyTable":
        _check_flatten_args(plan, tensors, flat)
        tp = (c_vp * max(len(tensors), 1))(*[_ptr(t, 2, "tensor") for t in tensors])
        h = c_vp()
        _check(_ft_create(plan.handle, tp, _ptr(flat, 2, "flat"), ctypes.byref(h)),
               "zero_flatten_table_create")
        return cls(h, (plan, list(tensors), flat))

    def __del__(self):
        h = getattr(self, "_h", None)
        free = getattr(self, "_free", None)
        if h is not None and h.value and free is not None:
            free(h)
            h.value = None

    @property
    def blocks(self) -> int:
        return int(_ct_blocks(self._h))

    def run(self, stream=None) -> None:
        _check(_ct_run(self._h, int(stream) if stream is not None else self._default_stream()),
               "zero_copy_table_run")

    def prepare_run(self, stream) -> "Prepared":
        p = Prepared(_ct_run, [self._h, int(stream) if stream is not None else
                               self._default_stream()], "zero_copy_table_run")
        p._keep = self
        return p

    def _default_stream(self) -> int:
        import torch
        return torch.cuda.current_stream().cuda_stream


class ReduceTable:
    """Owner of a zero_reduce_table: the rank's averaged gradient reduced
    straight from R per-tensor replicas (replicas[k][t] = replica k's tensor t)
    into shard_grad, described once in device memory (on the current device).
    The plan and the buffers are held here, so they outlive the table."""

    def __init__(self, plan: Plan, rank: int, replicas: Sequence[Sequence], shard_grad):
        T = plan.num_tensors
        for k, rep in enumerate(replicas):
            if len(rep) != T:
                raise ValueError(f"replica {k} lists {len(rep)} tensors; the plan has {T}")
            for t, x in enumerate(rep):
                _need(x, plan.tensor_numel(t), f"tensor {t} of replica {k}")
        _need(shard_grad, plan.shard_numel, "shard_grad")
        ptrs = (c_vp * max(len(replicas) * T, 1))(
            *[_ptr(x, 2, "replica tensor") for rep in replicas for x in rep])
        h = c_vp()
        _check(_rt_create(plan.handle, rank, ptrs, len(replicas), _ptr(shard_grad, 2, "shard_grad"),
                          ctypes.byref(h)), "zero_reduce_table_create")
        self._h = h
        self._free = _rt_free          # held by the instance for interpreter exit
        self._keep = (plan, [list(r) for r in replicas], shard_grad)
        self._device_ref = shard_grad

    def __del__(self):
        h = getattr(self, "_h", None)
        free = getattr(self, "_free", None)
        if h is not None and h.value and free is not None:
            free(h)
            h.value = None

    @property
    def blocks(self) -> int:
        return int(_rt_blocks(self._h))

    def run(self, sqnorm_out=None, stream=None) -> None:
        self.prepare_run(sqnorm_out, stream)()

    def prepare_run(self, sqnorm_out=None, stream=None) -> "Prepared":
        _need(sqnorm_out, 1, "sqnorm_out")
        p = Prepared(_rt_run, [self._h, _ptr(sqnorm_out, 8, "sqnorm_out"),
                               _stream(stream, self._device_ref)], "zero_reduce_table_run")
        p._keep = (self, sqnorm_out)
        return p


def _host_ptr(a, itemsize: int, what: str) -> int:
    """Host buffer: a C-contiguous numpy array or a CPU torch tensor."""
    if hasattr(a, "ctypes"):
        if not a.flags.c_contiguous or a.itemsize != itemsize or not a.flags.writeable and what != "grad":
            raise ValueError(f"{what} must be a contiguous, writable host array of {itemsize}-byte items")
        return a.ctypes.data
    if a.is_cuda or not a.is_contiguous() or a.element_size() != itemsize:
        raise ValueError(f"{what} must be a contiguous host tensor of {itemsize}-byte items")
    return a.data_ptr()


def zero_host_adamw_step(master, exp_avg, exp_avg_sq, grad, param_out, step: int, lr: float,
                         beta1: float, beta2: float, eps: float, weight_decay: float,
                         clip_scale: float = 1.0, n_threads: int = 0) -> None:
    """Host arrays (numpy or CPU tensors): fp32 master/m/v, bf16 bits grad/param_out."""
    n = len(master)
    for a in (exp_avg, exp_avg_sq, grad, param_out):
        if len(a) < n:
            raise ValueError("an array holds fewer elements than master")
    _check(_host_adamw(_host_ptr(master, 4, "master"), _host_ptr(exp_avg, 4, "exp_avg"),
                       _host_ptr(exp_avg_sq, 4, "exp_avg_sq"), _host_ptr(grad, 2, "grad"),
                       _host_ptr(param_out, 2, "param_out"), n, step, lr, beta1, beta2, eps,
                       weight_decay, float(clip_scale), n_threads), "zero_host_adamw_step")


def zero_offload_adamw_step(h_master, h_exp_avg, h_exp_avg_sq, d_grad, d_param_out, h_staging,
                            step: int, lr: float, beta1: float, beta2: float, eps: float,
                            weight_decay: float, clip_scale=None, n_threads: int = 0,
                            stream=None) -> None:
    """Host fp32 state (CPU tensors), device bf16 grad/params, pinned host staging."""
    n = h_master.numel()
    for t, what in ((h_exp_avg, "exp_avg"), (h_exp_avg_sq, "exp_avg_sq"), (d_grad, "d_grad"),
                    (d_param_out, "d_param_out")):
        _need(t, n, what)
    _need(clip_scale, 1, "clip_scale")
    if not h_staging.is_pinned():
        raise ValueError("h_staging must be pinned host memory")
    _check(_offload(_host_ptr(h_master, 4, "master"), _host_ptr(h_exp_avg, 4, "exp_avg"),
                    _host_ptr(h_exp_avg_sq, 4, "exp_avg_sq"), _ptr(d_grad, 2, "d_grad"),
                    _ptr(d_param_out, 2, "d_param_out"), _host_ptr(h_staging, 2, "h_staging"),
                    h_staging.numel(), n, step, lr, beta1, beta2, eps, weight_decay,
                    _ptr(clip_scale, 4, "clip_scale"), n_threads, _stream(stream, d_grad)),
           "zero_offload_adamw_step")


def zero_status_string(status: int) -> str:
    return _status_string(status).decode()


def zero_last_error() -> str:
    return _last_error().decode()


# --------------------------------------------------------------------------- prepared calls
#
# The same entry points with their arguments marshalled once, for loops that
# call them with unchanged buffers every step: each call then costs one ctypes
# dispatch instead of rebuilding pointer tables.

def zero_adamw_step_scalars(step: int, lr: float, beta1: float, beta2: float, eps: float,
                            weight_decay: float):
    """The eight fp32 scalars every AdamW call computes for `step` (host only): beta1,
    1-beta1, beta2, 1-beta2, eps, lr/(1-beta1^t), sqrt(1-beta2^t), 1-lr*weight_decay."""
    import numpy as np
    out = (ctypes.c_float * 8)()
    _check(_step_scalars(step, lr, beta1, beta2, eps, weight_decay, out), "zero_adamw_step_scalars")
    return np.frombuffer(bytes(out), dtype=np.float32).copy()


class AdamWSchedule:
    """Owner of a zero_adamw_schedule: AdamW's step counted on the device (on the
    current device), so that a step captured in a HIP graph replays successive
    steps. lr: one learning rate, or a sequence (step t uses lr[min(t, len) - 1])."""

    def __init__(self, lr, beta1: float, beta2: float, eps: float, weight_decay: float,
                 first_step: int = 1):
        rates = [float(x) for x in (lr if hasattr(lr, "__len__") else [lr])]
        arr = (c_dbl * max(len(rates), 1))(*rates)
        self._h = c_vp()
        _check(_sched_create(arr, len(rates), beta1, beta2, eps, weight_decay, first_step,
                             ctypes.byref(self._h)), "zero_adamw_schedule_create")
        self._free = _sched_free
        import torch
        self._device = torch.cuda.current_device()

    def __del__(self):
        h = getattr(self, "_h", None)
        free = getattr(self, "_free", None)
        if h is not None and h.value and free is not None:
            free(h)
            h.value = None

    @property
    def handle(self) -> c_vp:
        return self._h

    @property
    def length(self) -> int:
        return int(_sched_length(self._h))

    def applied(self) -> int:
        """Updates applied so far (a synchronous read; wait for the streams first)."""
        out = c_i64()
        _check(_sched_applied(self._h, ctypes.byref(out)), "zero_adamw_schedule_applied")
        return int(out.value)

    def _stream_of(self, stream) -> int:
        if stream is not None:
            return int(stream)
        import torch
        return torch.cuda.current_stream(self._device).cuda_stream

    def advance(self, clip_scale=None, stream=None) -> None:
        self.prepare_advance(clip_scale, stream)()

    def prepare_advance(self, clip_scale=None, stream=None) -> "Prepared":
        _need(clip_scale, 1, "clip_scale")
        p = Prepared(_sched_advance, [self._h, _ptr(clip_scale, 4, "clip_scale"), self._stream_of(stream)],
                     "zero_adamw_schedule_advance")
        p._keep = (self, clip_scale)
        return p


def prepare_shard_adamw_step_scheduled(master, exp_avg, exp_avg_sq, grad, param_out,
                                       schedule: AdamWSchedule, clip_scale=None, stream=None) -> "Prepared":
    """zero_shard_adamw_step_scheduled with its arguments marshalled once."""
    n = master.numel()
    _check_adamw_args(n, (master, exp_avg, exp_avg_sq, grad, param_out), clip_scale)
    p = Prepared(_adamw_sched, [_ptr(master, 4, "master"), _ptr(exp_avg, 4, "exp_avg"),
                                _ptr(exp_avg_sq, 4, "exp_avg_sq"), _ptr(grad, 2, "grad"),
                                _ptr(param_out, 2, "param_out"), n, schedule.handle,
                                _ptr(clip_scale, 4, "clip_scale"), _stream(stream, master)],
                 "zero_shard_adamw_step_scheduled")
    p._keep = (master, exp_avg, exp_avg_sq, grad, param_out, schedule, clip_scale)
    return p


def zero_shard_adamw_step_scheduled(master, exp_avg, exp_avg_sq, grad, param_out,
                                    schedule: AdamWSchedule, clip_scale=None, stream=None) -> None:
    """The flat AdamW update with the step's scalars read on the device from `schedule`
    (which this call does not move on: call schedule.advance once per step)."""
    prepare_shard_adamw_step_scheduled(master, exp_avg, exp_avg_sq, grad, param_out, schedule,
                                       clip_scale, stream)()


class Prepared:
    def __init__(self, fn, args, where: str, step_index: Optional[int] = None):
        self._fn, self._args, self._where, self._step_index = fn, list(args), where, step_index

    def __call__(self, step: Optional[int] = None) -> None:
        args = self._args
        if self._step_index is not None:
            args = list(args)
            args[self._step_index] = step
        _check(self._fn(*args), self._where)


def prepare_grad_reduce_shard(plan: Plan, rank: int, replicas: Sequence, begin: int, count: int,
                              shard_grad, sqnorm_out, workspace, stream) -> Prepared:
    _check_reduce_args(plan, replicas, count, shard_grad, sqnorm_out)
    ptrs = (c_vp * max(len(replicas), 1))(*[_ptr(r, 2, "replica") for r in replicas])
    ws = workspace.data_ptr() if workspace is not None else 0
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    p = Prepared(_reduce, [plan.handle, rank, ptrs, len(replicas), begin, count,
                           _ptr(shard_grad, 2, "shard_grad"), _ptr(sqnorm_out, 8, "sqnorm_out"), ws,
                           wsb, _stream(stream, shard_grad)], "zero_grad_reduce_shard")
    p._keep = (ptrs, replicas, shard_grad, sqnorm_out, workspace)
    return p


def prepare_clip_scale(partials, max_norm: float, scale_out, stream) -> Prepared:
    _need(scale_out, 1, "scale_out")
    p = Prepared(_clip, [_ptr(partials, 8, "partials"), partials.numel(), float(max_norm),
                         _ptr(scale_out, 4, "scale_out"), _stream(stream, partials)],
                 "zero_clip_scale")
    p._keep = (partials, scale_out)
    return p


def prepare_shard_adamw_step(master, exp_avg, exp_avg_sq, grad, param_out, lr: float, beta1: float,
                             beta2: float, eps: float, weight_decay: float, clip_scale, stream
                             ) -> Prepared:
    """Call the result with the 1-based step number."""
    n = master.numel()
    _check_adamw_args(n, (master, exp_avg, exp_avg_sq, grad, param_out), clip_scale)
    p = Prepared(_adamw, [_ptr(master, 4, "master"), _ptr(exp_avg, 4, "exp_avg"),
                          _ptr(exp_avg_sq, 4, "exp_avg_sq"), _ptr(grad, 2, "grad"),
                          _ptr(param_out, 2, "param_out"), n, 1, lr, beta1, beta2, eps,
                          weight_decay, _ptr(clip_scale, 4, "clip_scale"),
                          _stream(stream, master)], "zero_shard_adamw_step", step_index=6)
    p._keep = (master, exp_avg, exp_avg_sq, grad, param_out, clip_scale)
    return p


def prepare_offload_adamw_step(h_master, h_exp_avg, h_exp_avg_sq, d_grad, d_param_out, h_staging,
                               lr: float, beta1: float, beta2: float, eps: float,
                               weight_decay: float, clip_scale, stream, n_threads: int = 0
                               ) -> Prepared:
    """Call the result with the 1-based step number."""
    n = h_master.numel()
    for t in (h_exp_avg, h_exp_avg_sq, d_grad, d_param_out):
        if t.numel() < n:
            raise ValueError("an array holds fewer elements than master")
    _need(clip_scale, 1, "clip_scale")
    if not h_staging.is_pinned():
        raise ValueError("h_staging must be pinned host memory")
    p = Prepared(_offload, [_host_ptr(h_master, 4, "master"), _host_ptr(h_exp_avg, 4, "exp_avg"),
                            _host_ptr(h_exp_avg_sq, 4, "exp_avg_sq"), _ptr(d_grad, 2, "d_grad"),
                            _ptr(d_param_out, 2, "d_param_out"),
                            _host_ptr(h_staging, 2, "h_staging"), h_staging.numel(), n, 1, lr,
                            beta1, beta2, eps, weight_decay, _ptr(clip_scale, 4, "clip_scale"),
                            n_threads, _stream(stream, d_grad)],
                 "zero_offload_adamw_step", step_index=8)
    p._keep = (h_master, h_exp_avg, h_exp_avg_sq, d_grad, d_param_out, h_staging, clip_scale)
    return p


def prepare_gather_params(plan: Plan, shards: Sequence, tensors: Sequence, stream) -> Prepared:
    _check_gather_args(plan, shards, tensors)
    sp = (c_vp * max(len(shards), 1))(*[_ptr(s, 2, "shard") for s in shards])
    tp = (c_vp * max(len(tensors), 1))(*[_ptr(t, 2, "tensor") for t in tensors])
    ref = next((x for x in list(shards) + list(tensors) if x is not None), None)
    p = Prepared(_gather, [plan.handle, sp, tp, _stream(stream, ref) if ref is not None else 0],
                 "zero_gather_params")
    p._keep = (sp, tp, shards, tensors)
    return p


def prepare_flatten_params(plan: Plan, tensors: Sequence, flat, stream) -> Prepared:
    _check_flatten_args(plan, tensors, flat)
    tp = (c_vp * max(len(tensors), 1))(*[_ptr(t, 2, "tensor") for t in tensors])
    p = Prepared(_flatten, [plan.handle, tp, _ptr(flat, 2, "flat"), _stream(stream, flat)],
                 "zero_flatten_params")
    p._keep = (tp, tensors, flat)
    return p
