"""Helpers for the GPU parity tests: device transfer and the comparison bars.

Bars: integer, byte and index results bit for bit; fp32 master/m/v within
max(1e-6 * |ref|, 4 fp32 ulp of ref); bf16 values within 1 bf16 ulp
(distance of ordered integer encodings); NaN must meet NaN.
"""
import numpy as np
import pytest
import torch

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a ROCm GPU")


def dev():
    return torch.device("cuda:0")


def note(msg: str) -> None:
    print(msg, flush=True)


def to_dev_u16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).to(dev())


def to_dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev())


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().view(np.uint16)


def host_f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.float32, copy=False)


def assert_bits_equal(got: np.ndarray, want: np.ndarray, what: str) -> None:
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{what}: {bad.size} mismatches, first at {bad[:5]}: " \
                          f"{got[bad[:5]]} vs {want[bad[:5]]}"


def f32_close_mask(got: np.ndarray, want: np.ndarray) -> np.ndarray:
    g = np.asarray(got, np.float32)
    w = np.asarray(want, np.float32)
    both_nan = np.isnan(g) & np.isnan(w)
    same = g.view(np.uint32) == w.view(np.uint32)
    wd = w.astype(np.float64)
    tol = np.maximum(1e-6 * np.abs(wd), 4.0 * np.spacing(np.abs(w)).astype(np.float64))
    with np.errstate(invalid="ignore"):
        close = np.abs(g.astype(np.float64) - wd) <= tol
    return both_nan | same | close


def assert_f32_close(got, want, what: str) -> float:
    """Returns the fraction of elements that are bit-identical."""
    ok = f32_close_mask(got, want)
    bad = np.flatnonzero(~ok)
    assert bad.size == 0, f"{what}: {bad.size} outside tolerance, first at {bad[:5]}: " \
                          f"{np.asarray(got)[bad[:5]]} vs {np.asarray(want)[bad[:5]]}"
    g = np.asarray(got, np.float32).view(np.uint32)
    w = np.asarray(want, np.float32).view(np.uint32)
    return float(np.mean(g == w)) if g.size else 1.0


def _ordered(bits: np.ndarray) -> np.ndarray:
    b = bits.astype(np.int32)
    return np.where(b & 0x8000, 0x8000 - b, b)    # monotone in the represented value


def assert_bf16_close(got: np.ndarray, want: np.ndarray, what: str) -> float:
    got = np.asarray(got, np.uint16)
    want = np.asarray(want, np.uint16)
    gnan = (got & 0x7FFF) > 0x7F80
    wnan = (want & 0x7FFF) > 0x7F80
    assert (gnan == wnan).all(), f"{what}: NaN positions differ"
    d = np.abs(_ordered(got) - _ordered(want))
    d[gnan] = 0
    bad = np.flatnonzero(d > 1)
    assert bad.size == 0, f"{what}: {bad.size} beyond 1 bf16 ulp, first at {bad[:5]}"
    return float(np.mean(got == want)) if got.size else 1.0
