"""Seeded synthetic inputs shared by the oracle-side tests and the GPU path.

This package holds input generation and workload shapes only, none of the
optimizer step's arithmetic. Three implementations of one counter-based
definition (documented in ``synth_host.c``) exist:

* ``reference_normal``: a pure-Python transcription, used on tiny windows to
  pin the two compiled ones;
* ``normal_f32`` / ``normal_bf16``: plain C with OpenMP on the host
  (``libsynth_host.so``);
* ``device_normal_f32`` / ``device_normal_bf16``: the HIP twin
  (``libsynth_device.so``), which writes straight into device memory.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

from .models import (GRAD_SIGMA, KIND_GRAD, KIND_MASTER, KIND_PARAM, KIND_REPLICA,  # noqa: F401
                     MASTER_SIGMA, WORKLOADS, Workload, numels)

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(_HERE, "libsynth_host.so")
DEVICE_LIB = os.path.join(_HERE, "libsynth_device.so")

_MASK = (1 << 64) - 1
_GAMMA = 0x9E3779B97F4A7C15


def build(verbose: bool = False) -> None:
    """Compile the host generator (gcc) and its device twin (hipcc, gfx950)."""
    cmds = [
        ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
         os.path.join(_HERE, "synth_host.c"), "-o", HOST_LIB + ".tmp"],
        ["hipcc", "--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-std=c++17",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         os.path.join(_HERE, "synth_device.hip"), "-o", DEVICE_LIB + ".tmp"],
    ]
    for cmd in cmds:
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
    os.replace(HOST_LIB + ".tmp", HOST_LIB)
    os.replace(DEVICE_LIB + ".tmp", DEVICE_LIB)


# --------------------------------------------------------------------------- pure Python

def _mix(z: int) -> int:
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK
    return z ^ (z >> 31)


def _h(x: int) -> int:
    return _mix((x + _GAMMA) & _MASK)


def reference_key(seed: int, kind: int, step: int, replica: int) -> int:
    k = _h(seed & _MASK)
    for field in (kind, step, replica):
        k = _h(k ^ (field & _MASK))
    return k


def reference_normal(n: int, seed: int, kind: int, step: int = 0, replica: int = 0,
                     g0: int = 0, phi: Optional[int] = None, sigma: float = 1.0) -> np.ndarray:
    """Slow transcription of the definition; float32 values for g0 .. g0+n-1."""
    if phi is None:
        phi = g0 + n
    key = reference_key(seed, kind, step, replica)
    out = np.zeros(n, dtype=np.float32)
    for i in range(n):
        g = g0 + i
        if g >= phi:
            continue
        s = 0
        for j in range(3):
            w = _mix((key + (3 * g + j + 1) * _GAMMA) & _MASK)
            s += (w & 0xFFFF) + ((w >> 16) & 0xFFFF) + ((w >> 32) & 0xFFFF) + ((w >> 48) & 0xFFFF)
        z = (s - 393210) / 65536.0
        out[i] = np.float32(z * sigma)
    return out


# --------------------------------------------------------------------------- host C

_host = None


def _host_lib():
    global _host
    if _host is None:
        if not os.path.exists(HOST_LIB):
            raise RuntimeError(f"{HOST_LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(HOST_LIB)
        args = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64, ctypes.c_double]
        for name in ("synth_normal_f32", "synth_normal_bf16"):
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = None
        lib.synth_key.argtypes = [ctypes.c_uint64] * 4
        lib.synth_key.restype = ctypes.c_uint64
        _host = lib
    return _host


def normal_f32(n: int, seed: int, kind: int, step: int = 0, replica: int = 0, g0: int = 0,
               phi: Optional[int] = None, sigma: float = 1.0, out: Optional[np.ndarray] = None
               ) -> np.ndarray:
    if phi is None:
        phi = g0 + n
    if out is None:
        out = np.empty(n, dtype=np.float32)
    assert out.dtype == np.float32 and out.size == n and out.flags.c_contiguous
    _host_lib().synth_normal_f32(out.ctypes.data, n, seed, kind, step, replica, g0, phi, sigma)
    return out


def normal_bf16(n: int, seed: int, kind: int, step: int = 0, replica: int = 0, g0: int = 0,
                phi: Optional[int] = None, sigma: float = 1.0, out: Optional[np.ndarray] = None
                ) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of the generated values."""
    if phi is None:
        phi = g0 + n
    if out is None:
        out = np.empty(n, dtype=np.uint16)
    assert out.dtype == np.uint16 and out.size == n and out.flags.c_contiguous
    _host_lib().synth_normal_bf16(out.ctypes.data, n, seed, kind, step, replica, g0, phi, sigma)
    return out


# --------------------------------------------------------------------------- device HIP

_dev = None


def _device_lib():
    global _dev
    if _dev is None:
        if not os.path.exists(DEVICE_LIB):
            raise RuntimeError(f"{DEVICE_LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(DEVICE_LIB)
        args = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p]
        for name in ("synth_device_normal_f32", "synth_device_normal_bf16"):
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        _dev = lib
    return _dev


def _device_fill(name: str, t, elem: int, n: Optional[int], seed: int, kind: int, step: int,
                 replica: int, g0: int, phi: Optional[int], sigma: float, stream) -> None:
    import torch
    assert t.is_cuda and t.is_contiguous() and t.element_size() == elem
    if n is None:
        n = t.numel()
    assert 0 <= n <= t.numel()
    if phi is None:
        phi = g0 + n
    if stream is None:
        stream = torch.cuda.current_stream(t.device).cuda_stream
    rc = getattr(_device_lib(), name)(t.data_ptr(), n, seed, kind, step, replica, g0, phi, sigma,
                                      stream)
    if rc != 0:
        raise RuntimeError(f"{name} failed with hipError {rc}")


def device_normal_f32(t, seed: int, kind: int, step: int = 0, replica: int = 0, g0: int = 0,
                      phi: Optional[int] = None, sigma: float = 1.0, n: Optional[int] = None,
                      stream=None) -> None:
    _device_fill("synth_device_normal_f32", t, 4, n, seed, kind, step, replica, g0, phi, sigma,
                 stream)


def device_normal_bf16(t, seed: int, kind: int, step: int = 0, replica: int = 0, g0: int = 0,
                       phi: Optional[int] = None, sigma: float = 1.0, n: Optional[int] = None,
                       stream=None) -> None:
    _device_fill("synth_device_normal_bf16", t, 2, n, seed, kind, step, replica, g0, phi, sigma,
                 stream)
