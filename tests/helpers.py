"""Shared helpers of the GPU tests: seeded inputs on the device and oracle comparisons."""
from __future__ import annotations

import os
import sys

import numpy as np

import msel_inputs


def log(msg: str) -> None:
    """Name the case before each GPU step (flushed), so a failing run says what it was doing."""
    sys.stdout.write(f"[case] {msg}\n")
    sys.stdout.flush()


def to_device(t: msel_inputs.Tensors, device="cuda"):
    import torch
    act = torch.bfloat16 if t.dtype == "bf16" else torch.float32
    out = {}
    for k, v in t.items():
        if v is None:
            out[k] = None
        else:
            v = np.ascontiguousarray(v)
            if not v.flags.writeable:  # torch.from_numpy wants a writable array
                v = v.copy()
            if v.dtype == np.uint16:
                out[k] = torch.from_numpy(v.view(np.int16)).to(device).view(torch.bfloat16)
            else:
                dt = act if k in ("u", "delta", "z", "B", "C", "dout") else torch.float32
                out[k] = torch.from_numpy(v).to(device=device, dtype=dt)
    return out


def host(x) -> np.ndarray:
    """Device tensor -> float64 numpy."""
    import torch
    return x.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def tol(dtype: str) -> float:
    """Parity bound: max|gpu - oracle| <= tol * max|oracle| (1e-4 fp32, 1e-2 bf16 inputs)."""
    return 1e-4 if dtype == "f32" else 1e-2


def rel_err(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite values in GPU output"
    scale = np.max(np.abs(ref))
    if scale == 0.0:
        return float(np.max(np.abs(got)))
    return float(np.max(np.abs(got - ref)) / scale)


def _record_margin(name, e, dtype):
    """With MSEL_MARGINS_LOG set to a file, append 'test | tensor | err/tol' to it: the
    parity margins of a whole run, for the design notes."""
    path = os.environ.get("MSEL_MARGINS_LOG")
    if path:
        test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
        with open(path, "a") as fh:
            fh.write(f"{test} | {name} | {dtype} | {e:.4e} | {e / tol(dtype):.4f}\n")


def assert_close(name, got, ref, dtype):
    e = rel_err(got, ref)
    _record_margin(name, e, dtype)
    assert e <= tol(dtype), f"{name}: max|err|/max|ref| = {e:.3e} > {tol(dtype):.0e}"
    return e


def oracle_vals(t: msel_inputs.Tensors) -> dict:
    return {k: t.values(k) for k in ("u", "delta", "z", "B", "C", "A", "D", "bias", "h0", "dout")}


class MaxErr:
    """max|got - ref| and max|ref| of one tensor accumulated over slices, so that a tensor too
    large for one oracle call is still held to the per-tensor bar as a whole."""

    def __init__(self, name: str, dtype: str):
        self.name, self.dtype = name, dtype
        self.err = 0.0
        self.scale = 0.0
        self.count = 0

    def add(self, got, ref) -> None:
        got = np.asarray(got, np.float64)
        ref = np.asarray(ref, np.float64)
        assert got.shape == ref.shape, (self.name, got.shape, ref.shape)
        assert np.all(np.isfinite(got)), f"{self.name}: non-finite values in GPU output"
        if got.size:
            self.err = max(self.err, float(np.max(np.abs(got - ref))))
            self.scale = max(self.scale, float(np.max(np.abs(ref))))
        self.count += got.size

    def check(self, expect_count=None) -> float:
        if expect_count is not None:
            assert self.count == expect_count, (self.name, self.count, expect_count)
        e = self.err / self.scale if self.scale > 0 else self.err
        log(f"{self.name}: {self.count} elements, max|err|/max|ref| = {e:.3e}")
        _record_margin(self.name, e, self.dtype)
        assert e <= tol(self.dtype), \
            f"{self.name}: max|err|/max|ref| = {e:.3e} > {tol(self.dtype):.0e}"
        return e
