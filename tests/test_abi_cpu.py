"""The C-ABI library on the host (no GPU calls): symbols, plan logic, argument checks."""
import ctypes
import os
import re
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.fixture(scope="module")
def zm():
    import zero_partitioned_mixed_partition_amd as m
    return m


def _declared_functions():
    names = set()
    inc = os.path.join(ROOT, "include")
    for fn in os.listdir(inc):
        if fn.endswith(".h"):
            text = open(os.path.join(inc, fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(zero_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_function(zm):
    names = _declared_functions()
    assert len(names) >= 18, names
    lib = ctypes.CDLL(zm.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


@pytest.mark.parametrize("name", sorted(synth.WORKLOADS))
def test_plan_matches_oracle_on_workloads(zm, name):
    w = synth.WORKLOADS[name]
    for n_ranks in sorted({w.n_ranks, 1, 3}):
        ref = oracle.partition_plan(w.numels, n_ranks, w.align)
        plan = zm.zero_partition_plan(w.numels, n_ranks, w.align)
        assert (plan.numel, plan.padded_numel, plan.shard_numel, plan.num_tensors,
                plan.num_ranks) == (ref.numel, ref.padded_numel, ref.shard_numel,
                                    len(w.numels), n_ranks)
        assert [plan.tensor_offset(t) for t in range(len(w.numels))] == ref.offsets
        for r in range(n_ranks):
            assert plan.segments(r) == ref.segments(r), (name, n_ranks, r)
        for stage in range(4):
            for padded in (False, True):
                assert plan.memory_bytes(stage, padded) == oracle.memory_bytes(ref, stage, padded)


@pytest.mark.parametrize("seed", range(30))
def test_plan_matches_oracle_random(zm, seed):
    rng = np.random.default_rng(1000 + seed)
    t = int(rng.integers(0, 12))
    numels = [int(x) for x in rng.integers(0, 5000, t)]
    if seed % 5 == 0 and t:
        numels[int(rng.integers(0, t))] = 0
    n_ranks = int(rng.choice([1, 2, 3, 5, 8, 64]))
    align = int(rng.choice([1, 2, 8, 128, 1000]))
    ref = oracle.partition_plan(numels, n_ranks, align)
    plan = zm.zero_partition_plan(numels, n_ranks, align)
    assert (plan.numel, plan.padded_numel, plan.shard_numel) == (
        ref.numel, ref.padded_numel, ref.shard_numel)
    for r in range(n_ranks):
        assert plan.segments(r) == ref.segments(r)


def test_plan_page_figures_through_the_abi(zm):
    plan = zm.zero_partition_plan([70_000_000_000], 64, 1)
    gb = [plan.memory_bytes(s) / 1e9 for s in range(4)]
    assert gb == [1120.0, 280 + 840 / 64, 140 + 980 / 64, 1120 / 64]


def test_plan_errors(zm):
    with pytest.raises(zm.ZeroError):
        zm.zero_partition_plan([5, -1], 2, 1)
    with pytest.raises(zm.ZeroError):
        zm.zero_partition_plan([5], 0, 1)
    with pytest.raises(zm.ZeroError):
        zm.zero_partition_plan([5], 1, 0)
    with pytest.raises(zm.ZeroError):   # total overflows int64
        zm.zero_partition_plan([2 ** 62, 2 ** 62], 1, 1)
    with pytest.raises(zm.ZeroError):   # padding overflows int64
        zm.zero_partition_plan([2 ** 63 - 2], 1, 1 << 20)
    plan = zm.zero_partition_plan([], 4, 128)
    assert (plan.numel, plan.padded_numel, plan.shard_numel, plan.num_segments(0)) == (0, 0, 0, 0)
    plan = zm.zero_partition_plan([10], 2, 1)
    with pytest.raises(ValueError):
        plan.segments(2)
    with pytest.raises(zm.ZeroError):
        plan.memory_bytes(4)
    assert plan.tensor_offset(1) == -1


def test_device_calls_reject_bad_arguments_before_touching_the_gpu(zm):
    lib = zm._binding
    st = lib._adamw(None, None, None, None, None, 16, 0, 1e-3, 0.9, 0.999, 1e-8, 0.0, None, None)
    assert st == zm._binding.ZERO_EINVAL            # step < 1
    st = lib._adamw(None, None, None, None, None, -1, 1, 1e-3, 0.9, 0.999, 1e-8, 0.0, None, None)
    assert st == zm._binding.ZERO_EINVAL            # n < 0
    st = lib._adamw(None, None, None, None, None, 0, 1, 1e-3, 0.9, 0.999, 1e-8, 0.0, None, None)
    assert st == zm._binding.ZERO_OK                # empty: nothing to do
    st = lib._adamw(None, None, None, None, None, 4, 1, 1e-3, 0.9, 0.999, 1e-8, 0.0, None, None)
    assert st == zm._binding.ZERO_EINVAL            # NULL arrays
    assert "NULL" in zm.zero_last_error()
    st = lib._sqnorm(None, -1, None, None, 0, None)
    assert st == zm._binding.ZERO_EINVAL
    st = lib._clip(None, 1, 1.0, None, None)
    assert st == zm._binding.ZERO_EINVAL
    st = lib._gather(None, None, None, None)
    assert st == zm._binding.ZERO_EINVAL
    plan = zm.zero_partition_plan([100], 2, 1)
    st = lib._reduce(plan.handle, 5, None, 1, 0, 100, None, None, None, 0, None)
    assert st == zm._binding.ZERO_EINVAL
    assert zm.zero_status_string(zm._binding.ZERO_ENOSPACE).startswith("workspace")
    assert zm.zero_sqnorm_workspace_bytes() >= 8


def test_reduce_adamw_rejects_bad_arguments_before_touching_the_gpu(zm):
    """zero_reduce_adamw_step's argument checks, which all run before any HIP
    call (the addresses below are never dereferenced)."""
    import ctypes
    lib = zm._binding
    plan = zm.zero_partition_plan([1000], 2, 1)          # S = 500
    reps = (ctypes.c_void_p * 2)(0x10000, 0x20000)
    hp = (1e-3, 0.9, 0.999, 1e-8, 0.01)
    f32 = [ctypes.c_void_p(0x100000 * (k + 1)) for k in range(3)]   # disjoint 500-float arrays
    par, grd = ctypes.c_void_p(0x900000), ctypes.c_void_p(0xA00000)

    def call(plan_h=plan.handle, rank=1, n_rep=2, begin=0, count=1000, state=f32, param=par,
             grad=grd, step=1, h=hp, replicas=reps):
        return lib._reduce_adamw(plan_h, rank, replicas, n_rep, begin, count, *state, param, grad,
                                 step, *h, None, None)
    E = lib.ZERO_EINVAL
    assert call(plan_h=None) == E
    assert call(replicas=None) == E
    assert call(rank=2) == E and call(rank=-1) == E
    assert call(n_rep=0) == E and call(n_rep=65) == E
    assert call(begin=-1) == E and call(count=1001) == E and call(begin=600, count=401) == E
    assert call(step=0) == E
    assert call(h=(1e-3, 1.0, 0.999, 1e-8, 0.01)) == E          # beta1 outside [0, 1)
    assert call(h=(1e-3, 0.9, 0.999, 0.0, 0.01)) == E           # eps <= 0
    assert call(begin=0, count=500) == lib.ZERO_OK              # window misses rank 1's shard
    assert call(state=[f32[0], None, f32[2]]) == E              # NULL state array
    assert "NULL" in zm.zero_last_error()
    assert call(replicas=(ctypes.c_void_p * 2)(0x10000, None)) == E   # NULL replica
    assert call(param=ctypes.c_void_p(0x100000 + 1000)) == E    # param_out inside master
    assert "overlaps" in zm.zero_last_error()
    assert call(grad=ctypes.c_void_p(0x300000 + 200)) == E      # shard_grad inside exp_avg_sq
    assert call(grad=ctypes.c_void_p(0x900000 + 100)) == E      # shard_grad over param_out
    assert "shard_grad" in zm.zero_last_error()


def test_overlapping_arrays_are_refused_before_touching_the_gpu(zm):
    """Each kernel reads and writes element i of its arrays from one lane, so a
    written array shifted against another array it touches would race: the
    entry points refuse such arguments and name the pair (checked before any
    HIP call; the addresses are never dereferenced). Arrays that are only read
    may overlap one another."""
    lib = zm._binding
    E = lib.ZERO_EINVAL
    hp = (1e-3, 0.9, 0.999, 1e-8, 0.01)
    master, m, v = 0x100000, 0x200000, 0x300000                # 500 floats each
    param, grad = 0x900000, 0xA00000                           # 500 bf16 each

    def adamw(mst=master, ea=m, eas=v, g=grad, p=param, n=500):
        return lib._adamw(mst, ea, eas, g, p, n, 1, *hp, None, None)
    assert adamw(ea=master + 4) == E
    assert zm.zero_last_error().endswith("master overlaps exp_avg")
    assert adamw(g=param + 2) == E
    assert zm.zero_last_error().endswith("param_out overlaps grad")
    assert adamw(g=v + 1996) == E                                  # the last 4 bytes of v
    assert zm.zero_last_error().endswith("exp_avg_sq overlaps grad")

    # rank 1 of a [1000] list over 2 ranks reads elements [500, 1000) of each replica
    plan = zm.zero_partition_plan([1000], 2, 1)
    reps = (ctypes.c_void_p * 2)(0x10000, 0x20000)

    def fused(state=(master, m, v), p=param, g=None, replicas=reps):
        return lib._reduce_adamw(plan.handle, 1, replicas, 2, 0, 1000, *state, p, g, 1, *hp, None, None)
    assert fused(p=0x20000 + 1000) == E
    assert zm.zero_last_error().endswith("param_out overlaps replica 1")
    assert fused(state=(0x10000 + 1998, m, v)) == E                # master's first 2 bytes
    assert zm.zero_last_error().endswith("master overlaps replica 0")
    assert fused(g=m + 100) == E
    assert zm.zero_last_error().endswith("exp_avg overlaps shard_grad")

    def reduce(g=0x900000, sq=None, ws=None, ws_bytes=0):
        return lib._reduce(plan.handle, 1, reps, 2, 0, 1000, g, sq, ws, ws_bytes, None)
    assert reduce(g=0x10000 + 2) == E                              # 2 bytes into replica 0's slice
    assert zm.zero_last_error().endswith("shard_grad overlaps replica 0")
    wsb = zm.zero_sqnorm_workspace_bytes()
    assert reduce(sq=0xB00000, ws=0x900000 - wsb + 8, ws_bytes=wsb) == E
    assert zm.zero_last_error().endswith("shard_grad overlaps workspace")
    assert reduce(sq=0xB00000, ws=0x20000 + 1024, ws_bytes=wsb) == E
    assert zm.zero_last_error().endswith("workspace overlaps replica 1")
    assert lib._reduce_noalloc(plan.handle, 1, reps, 2, 0, 1000, 0x20000 + 1500, None, None) == E
    assert zm.zero_last_error().endswith("shard_grad overlaps replica 1")

    # the multi-tensor list and table, per tensor
    def ptrs(*a):
        return (ctypes.c_void_p * len(a))(*a)
    n = (ctypes.c_int64 * 2)(500, 300)
    ok = dict(ms=ptrs(master, 0x400000), ea=ptrs(m, 0x500000), eas=ptrs(v, 0x600000),
              g=ptrs(grad, 0x700000), p=ptrs(param, 0x800000))
    bad = dict(ok, g=ptrs(grad, 0x800000 + 598))                    # tensor 1's grad over its param
    assert lib._mt_adamw(bad["ms"], bad["ea"], bad["eas"], bad["g"], bad["p"], n, 2, 1, *hp,
                         None, None) == E
    assert zm.zero_last_error().endswith("param overlaps grad of tensor 1")
    out = ctypes.c_void_p()
    assert lib._mt_create(bad["ms"], bad["ea"], bad["eas"], bad["g"], bad["p"], n, 2,
                          ctypes.byref(out)) == E
    assert "of tensor 1" in zm.zero_last_error() and not out.value


def test_gather_and_flatten_refuse_overlapping_ranges_before_touching_the_gpu(zm):
    """The gather writes the tensors and reads the shards; the flatten writes
    the flat buffer and reads the tensors. A written range that meets another
    range of the call is refused, naming the pair, in the per-call and in the
    table forms (fake addresses, never dereferenced)."""
    lib = zm._binding
    E = lib.ZERO_EINVAL
    plan = zm.zero_partition_plan([100, 28], 2, 1)            # P = 128, S = 64

    def arr(*a):
        return (ctypes.c_void_p * len(a))(*a)
    shards = arr(0x30000, 0x30080)                              # 128 bytes each, back to back
    out = ctypes.c_void_p()
    # tensor 0 (200 bytes) runs into tensor 1
    for f in (lambda s, t: lib._gather(plan.handle, s, t, None),
              lambda s, t: lib._gt_create(plan.handle, s, t, ctypes.byref(out))):
        assert f(shards, arr(0x10000, 0x10000 + 198)) == E
        assert zm.zero_last_error().endswith("tensor 0 overlaps tensor 1")
        assert f(arr(0x20000 + 20, 0x30080), arr(0x10000, 0x20000)) == E
        assert zm.zero_last_error().endswith("tensor 1 overlaps shard 0")
        assert f(arr(None, 0x10000 + 100), arr(0x10000, 0x20000)) == E   # a NULL shard is skipped
        assert zm.zero_last_error().endswith("tensor 0 overlaps shard 1")
    assert not out.value
    # the flat buffer (256 bytes) meets tensor 1's last element
    for f in (lambda t, fl: lib._flatten(plan.handle, t, fl, None),
              lambda t, fl: lib._ft_create(plan.handle, t, fl, ctypes.byref(out))):
        assert f(arr(0x10000, 0x40000 - 54), 0x40000) == E
        assert zm.zero_last_error().endswith("flat overlaps tensor 1")
    assert not out.value


def test_reduce_table_rejects_bad_arguments_before_touching_the_gpu(zm):
    """zero_reduce_table_create's argument checks, all before any HIP call (the
    addresses are never dereferenced)."""
    import ctypes
    lib = zm._binding
    plan = zm.zero_partition_plan([1000, 24, 3000], 2, 8)      # S = 2016
    T, R = 3, 2
    good = [ctypes.c_void_p(0x100000 * (i + 1)) for i in range(T * R)]
    grad = ctypes.c_void_p(0x900000)
    out = ctypes.c_void_p()
    E = lib.ZERO_EINVAL

    def create(plan_h=plan.handle, rank=0, reps=good, n_rep=R, g=grad, o=ctypes.byref(out)):
        arr = None if reps is None else (ctypes.c_void_p * len(reps))(*reps)
        return lib._rt_create(plan_h, rank, arr, n_rep, g, o)
    assert create(o=None) == E
    assert create(plan_h=None) == E
    assert create(reps=None) == E
    assert create(rank=2) == E and create(rank=-1) == E
    assert create(n_rep=0) == E and create(n_rep=65) == E
    assert create(g=None) == E
    missing = list(good)
    missing[1 * T + 2] = None               # replica 1's tensor 2, which rank 1's shard needs
    assert create(rank=1, reps=missing) == E
    assert "replica 1" in zm.zero_last_error()
    # shard_grad (2016 elements) inside replica 0's tensor 2 (3000 elements at 0x300000)
    assert create(rank=1, g=ctypes.c_void_p(0x300000 + 1000)) == E
    assert "overlaps" in zm.zero_last_error()
    assert lib._rt_run(None, None, None) == E
    assert lib._rt_blocks(None) == -1
    lib._rt_free(None)


@pytest.mark.parametrize("name,n_ranks", [("gpt2-small", 8), ("llama3-8b", 64), ("tiny-a", 4),
                                          ("gpt-1.3b", 3)])
def test_shard0_plan_matches_oracle_on_workloads(zm, name, n_ranks):
    shapes = synth.WORKLOADS[name].shapes
    numels = [int(np.prod(s)) for s in shapes]
    dim0 = [s[0] for s in shapes]
    ref = oracle.partition_plan_shard0(numels, dim0, n_ranks, 128)
    plan = zm.zero_partition_plan_shard0(numels, dim0, n_ranks, 128)
    assert plan.kind == 1
    assert (plan.numel, plan.padded_numel, plan.shard_numel) == (
        ref.numel, ref.padded_numel, ref.shard_numel)
    assert [plan.tensor_offset(t) for t in range(len(numels))] == ref.offsets
    assert [plan.tensor_numel(t) for t in range(len(numels))] == numels
    for r in range(n_ranks):
        assert plan.segments(r) == ref.segments(r), (name, r)


@pytest.mark.parametrize("seed", range(20))
def test_shard0_plan_matches_oracle_random(zm, seed):
    rng = np.random.default_rng(700 + seed)
    t = int(rng.integers(0, 8))
    dim0 = [int(x) for x in rng.integers(1, 50, t)]
    numels = [d * int(k) for d, k in zip(dim0, rng.integers(1, 20, t))]
    if t and seed % 4 == 0:
        numels[0], dim0[0] = 0, 0
    n_ranks = int(rng.choice([1, 2, 3, 8, 64]))
    align = int(rng.choice([1, 8, 128]))
    ref = oracle.partition_plan_shard0(numels, dim0, n_ranks, align)
    plan = zm.zero_partition_plan_shard0(numels, dim0, n_ranks, align)
    assert (plan.numel, plan.padded_numel, plan.shard_numel) == (
        ref.numel, ref.padded_numel, ref.shard_numel)
    for r in range(n_ranks):
        assert plan.segments(r) == ref.segments(r)


def test_shard0_plan_errors(zm):
    with pytest.raises(zm.ZeroError):
        zm.zero_partition_plan_shard0([10], [3], 2, 1)      # dim0 does not divide numel
    with pytest.raises(zm.ZeroError):
        zm.zero_partition_plan_shard0([10], [0], 2, 1)
    assert zm.zero_partition_plan([4], 2, 1).kind == 0


def test_multi_tensor_adamw_rejects_bad_arguments_before_touching_the_gpu(zm):
    lib = zm._binding
    f = lib._mt_adamw
    args = (1e-3, 0.9, 0.999, 1e-8, 0.0, None, None)
    assert f(None, None, None, None, None, None, 0, 1, *args) == lib.ZERO_OK          # empty list
    assert f(None, None, None, None, None, None, -1, 1, *args) == lib.ZERO_EINVAL     # n_tensors < 0
    assert f(None, None, None, None, None, None, 2, 1, *args) == lib.ZERO_EINVAL      # NULL tables
    assert f(None, None, None, None, None, None, 0, 0, *args) == lib.ZERO_EINVAL      # step < 1
    one = (ctypes.c_void_p * 1)(None)
    n = (ctypes.c_int64 * 1)(5)
    assert f(one, one, one, one, one, n, 1, 1, *args) == lib.ZERO_EINVAL              # NULL arrays
    assert "tensor 0" in zm.zero_last_error()
    n[0] = -3
    assert f(one, one, one, one, one, n, 1, 1, *args) == lib.ZERO_EINVAL              # numel < 0
    n[0] = 0
    assert f(one, one, one, one, one, n, 1, 1, *args) == lib.ZERO_OK                  # empty tensor


def test_multi_tensor_table_rejects_bad_arguments_before_touching_the_gpu(zm):
    """Table creation checks the list as the list call does; an empty list needs
    no device, and its step enqueues nothing."""
    lib = zm._binding
    out = ctypes.c_void_p()
    assert lib._mt_create(None, None, None, None, None, None, 1, None) == lib.ZERO_EINVAL  # NULL out
    assert lib._mt_create(None, None, None, None, None, None, -1, ctypes.byref(out)) == lib.ZERO_EINVAL
    assert lib._mt_create(None, None, None, None, None, None, 2, ctypes.byref(out)) == lib.ZERO_EINVAL
    one = (ctypes.c_void_p * 1)(None)
    n = (ctypes.c_int64 * 1)(5)
    assert lib._mt_create(one, one, one, one, one, n, 1, ctypes.byref(out)) == lib.ZERO_EINVAL
    assert "tensor 0" in zm.zero_last_error()
    assert not out.value
    n[0] = 0
    assert lib._mt_create(one, one, one, one, one, n, 1, ctypes.byref(out)) == lib.ZERO_OK
    assert out.value and lib._mt_blocks(out) == 0
    hp = (1e-3, 0.9, 0.999, 1e-8, 0.0, None, None)
    assert lib._mt_step(out, 1, *hp) == lib.ZERO_OK
    assert lib._mt_step(out, 0, *hp) == lib.ZERO_EINVAL                               # step < 1
    assert lib._mt_step(None, 1, *hp) == lib.ZERO_EINVAL                              # NULL table
    lib._mt_free(out)
    lib._mt_free(None)
    assert lib._mt_blocks(None) == -1


def test_reduce_workspace_bytes(zm):
    """The one-pass reduce's workspace: the fixed size below 2^24 elements, then
    a partial per 512 elements plus the first-level sums (8 bytes each)."""
    fixed = zm.zero_sqnorm_workspace_bytes()
    assert zm.zero_reduce_workspace_bytes(0) == fixed
    assert zm.zero_reduce_workspace_bytes((1 << 24) - 1) == fixed
    for n in ((1 << 24), (1 << 24) + 4097, 164_465_408, 8_819_213_312):
        blocks = ((n + 1) // 2 + 255) // 256
        want = 8 * (blocks + (blocks + 2047) // 2048)
        assert zm.zero_reduce_workspace_bytes(n) == max(want, fixed), n


def test_copy_tables_reject_bad_arguments_before_touching_the_gpu(zm):
    """Gather and flatten tables check their arguments as the calls do; a plan
    with nothing to copy makes an empty table, which needs no device."""
    lib = zm._binding
    out = ctypes.c_void_p()
    plan = zm.zero_partition_plan([5, 3], 2, 8)
    two = (ctypes.c_void_p * 2)(None, None)
    assert lib._gt_create(plan.handle, two, two, None) == lib.ZERO_EINVAL             # NULL out
    assert lib._gt_create(None, two, two, ctypes.byref(out)) == lib.ZERO_EINVAL       # NULL plan
    assert lib._gt_create(plan.handle, None, two, ctypes.byref(out)) == lib.ZERO_EINVAL
    assert lib._gt_create(plan.handle, two, two, ctypes.byref(out)) == lib.ZERO_EINVAL  # NULL tensor
    assert "tensor 0" in zm.zero_last_error()
    assert lib._ft_create(plan.handle, two, None, ctypes.byref(out)) == lib.ZERO_EINVAL  # NULL flat
    assert lib._ft_create(None, two, None, ctypes.byref(out)) == lib.ZERO_EINVAL
    assert not out.value
    # NULL shards skip every rank: an empty gather table
    empty = zm.zero_partition_plan([0, 0], 2, 8)
    assert lib._gt_create(empty.handle, two, two, ctypes.byref(out)) == lib.ZERO_OK
    assert out.value and lib._ct_blocks(out) == 0
    assert lib._ct_run(out, None) == lib.ZERO_OK
    lib._ct_free(out)
    assert lib._ct_run(None, None) == lib.ZERO_EINVAL
    assert lib._ct_blocks(None) == -1
    lib._ct_free(None)


def test_builder_loads_without_importing_the_package():
    """build() must work when the in-tree library is stale or missing, so its
    build script is loaded without importing the package (which loads the
    library)."""
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r); import __graft_entry__ as g; m = g._load_builder(); "
            "assert callable(m.build); "
            "assert 'zero_partitioned_mixed_partition_amd' not in sys.modules; print('ok')" % ROOT)
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0 and out.stdout.strip() == "ok", out.stderr


def test_binding_refuses_buffers_shorter_than_the_call_touches(zm):
    """The C ABI sees bare device pointers; the binding checks every buffer's
    length first, so a short tensor raises ValueError naming it (here with CPU
    tensors: the check comes before any pointer is taken)."""
    import torch
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0)
    f = lambda n: torch.zeros(n, dtype=torch.float32)      # noqa: E731
    h = lambda n: torch.zeros(n, dtype=torch.int16)        # noqa: E731
    d = lambda n: torch.zeros(n, dtype=torch.float64)      # noqa: E731
    with pytest.raises(ValueError, match="master"):
        zm.zero_shard_adamw_step(f(8), f(16), f(16), h(16), h(16), 1, n=16, **hp)
    with pytest.raises(ValueError, match="param_out"):
        zm.zero_shard_adamw_step(f(16), f(16), f(16), h(16), h(8), 1, **hp)
    with pytest.raises(ValueError, match="grad"):
        zm.zero_grad_sqnorm(h(10), d(1), n=11)
    with pytest.raises(ValueError, match="sqnorm_out"):
        zm.zero_grad_sqnorm(h(10), d(0))
    with pytest.raises(ValueError, match="partials"):
        zm.zero_clip_scale(d(3), 1.0, f(1), n_partials=4)
    plan = zm.zero_partition_plan([100, 28], 2, 8)       # P = 128, S = 64
    with pytest.raises(ValueError, match="replica"):
        zm.zero_grad_reduce_shard(plan, 0, [h(128), h(127)], 0, 128, h(64))
    with pytest.raises(ValueError, match="shard_grad"):
        zm.zero_grad_reduce_shard(plan, 0, [h(128)], 0, 128, h(63))
    with pytest.raises(ValueError, match="tensor 1"):
        zm.zero_gather_params(plan, [h(64), h(64)], [h(100), h(27)])
    with pytest.raises(ValueError, match="shard"):
        zm.zero_gather_params(plan, [h(64), h(60)], [h(100), h(28)])
    with pytest.raises(ValueError, match="flat"):
        zm.zero_flatten_params(plan, [h(100), h(28)], h(127))
    with pytest.raises(ValueError, match="tensor 0"):
        zm.zero_flatten_params(plan, [h(99), h(28)], h(128))
    # the device tables check the same way before anything is created
    with pytest.raises(ValueError, match="tensor 1"):
        zm.CopyTable.gather(plan, [h(64), h(64)], [h(100), h(27)])
    with pytest.raises(ValueError, match="need N_d shards"):
        zm.CopyTable.gather(plan, [h(64)], [h(100), h(28)])
    with pytest.raises(ValueError, match="flat"):
        zm.CopyTable.flatten(plan, [h(100), h(28)], h(127))
    with pytest.raises(ValueError, match="device tensor"):  # host tensors are refused
        zm.CopyTable.gather(plan, [h(64), h(64)], [h(100), h(28)])
    with pytest.raises(ValueError, match="same length"):
        zm.MultiTensorTable([f(4)], [f(4)], [f(4)], [h(4)], [])
    with pytest.raises(ValueError, match="fewer elements"):
        zm.MultiTensorTable([f(4)], [f(4)], [f(3)], [h(4)], [h(4)])
    with pytest.raises(ValueError, match="device tensor"):
        zm.MultiTensorTable([f(4)], [f(4)], [f(4)], [h(4)], [h(4)])
    # the one-pass reduce and update, and the reduce table
    with pytest.raises(ValueError, match="replica"):
        zm.zero_reduce_adamw_step(plan, 0, [h(128), h(120)], 0, 128, f(64), f(64), f(64), h(64), 1, **hp)
    with pytest.raises(ValueError, match="exp_avg_sq"):
        zm.zero_reduce_adamw_step(plan, 0, [h(128)], 0, 128, f(64), f(64), f(63), h(64), 1, **hp)
    with pytest.raises(ValueError, match="shard_grad"):
        zm.zero_reduce_adamw_step(plan, 0, [h(128)], 0, 128, f(64), f(64), f(64), h(64), 1,
                                  shard_grad=h(32), **hp)
    with pytest.raises(ValueError, match="lists 1 tensors"):
        zm.ReduceTable(plan, 0, [[h(100)]], h(64))
    with pytest.raises(ValueError, match="tensor 1 of replica 1"):
        zm.ReduceTable(plan, 0, [[h(100), h(28)], [h(100), h(27)]], h(64))
    with pytest.raises(ValueError, match="shard_grad"):
        zm.ReduceTable(plan, 0, [[h(100), h(28)]], h(63))
    with pytest.raises(ValueError, match="device tensor"):
        zm.ReduceTable(plan, 0, [[h(100), h(28)]], h(64))


@pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None
                    or not os.path.exists(os.path.join(ROCM, "include", "hip")),
                    reason="needs gcc, g++ and the HIP headers")
@pytest.mark.parametrize("lang", ["c", "c++"])
def test_header_compiles_as_c_and_cpp(tmp_path, lang):
    """include/zero_mi355x.h is a C interface: it compiles as C99 (gcc) and as
    C++17 (g++), and a translation unit can name every declared type."""
    src = tmp_path / ("use.c" if lang == "c" else "use.cpp")
    src.write_text('#include "zero_mi355x.h"\n'
                   "int main(void) {\n"
                   "    zero_plan* p = 0; zero_mt_table* t = 0; zero_copy_table* c = 0;\n"
                   "    zero_segment s; zero_status st = ZERO_OK;\n"
                   "    (void)p; (void)t; (void)c; (void)s; (void)st;\n"
                   "    return (int)(zero_sqnorm_workspace_bytes() * 0);\n"
                   "}\n")
    cc, std = ("gcc", "-std=c99") if lang == "c" else ("g++", "-std=c++17")
    r = subprocess.run([cc, std, "-Wall", "-Wextra", "-Werror", "-fsyntax-only",
                        f"-I{os.path.join(ROOT, 'include')}", f"-isystem{os.path.join(ROCM, 'include')}",
                        "-D__HIP_PLATFORM_AMD__", str(src)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]
