"""Shared helpers of the GPU tests: seeded inputs on the device and oracle comparisons."""
from __future__ import annotations

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
        elif v.dtype == np.uint16:
            out[k] = torch.from_numpy(v.view(np.int16)).to(device).view(torch.bfloat16)
        else:
            dt = act if k in ("u", "delta", "z", "B", "C", "dout") else torch.float32
            out[k] = torch.from_numpy(np.ascontiguousarray(v)).to(device=device, dtype=dt)
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


def assert_close(name, got, ref, dtype):
    e = rel_err(got, ref)
    assert e <= tol(dtype), f"{name}: max|err|/max|ref| = {e:.3e} > {tol(dtype):.0e}"
    return e


def oracle_vals(t: msel_inputs.Tensors) -> dict:
    return {k: t.values(k) for k in ("u", "delta", "z", "B", "C", "A", "D", "bias", "h0", "dout")}
