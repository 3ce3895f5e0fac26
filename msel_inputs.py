"""Seeded synthetic inputs for the selective scan -- shared by the tests, the oracle and bench.

This module holds no arithmetic of the method itself: it only draws random numbers, rounds
them to bfloat16 when a workload asks for it and shapes them.  Both the CPU oracle and the GPU
path consume exactly the bytes made here.

Distributions (the workloads' recipe): u, z ~ N(0,1) and delta = 0.5*N(0,1) of shape
[batch, dim, seqlen]; bias[d] = log(expm1(U[1e-3, 1e-1])) (so that softplus(bias) is uniform in
[1e-3, 1e-1]); A[d, n] = -(n+1) (S4D-real); B, C ~ N(0,1) of shape [batch, dstate, seqlen],
shared by all channels; D ~ N(0,1) of shape [dim]; dout ~ N(0,1) for the backward.

The trapezoidal variant adds (``make(..., with_lam=True)``) the mixing weight lam ~ U[0, 1]
of shape [batch, dim, seqlen], and for continued sequences (``with_prev=True``) the inputs of
the step before the first, u_prev ~ N(0,1) [batch, dim] and B_prev ~ N(0,1) [batch, dstate].

The complex variant (``complex_A=True``, even dstate) takes A[d, 2j] + i A[d, 2j+1] =
-1/2 + i pi j (S4D-Lin) for state pair j.

The short convolution before the scan (``make_conv``): x ~ N(0,1) of shape [batch, dim,
seqlen]; taps w[d, k] and bias b[d] ~ U(-1/sqrt(W), 1/sqrt(W)) (the default initialisation of a
depthwise 1-d convolution, whose fan-in is the width W); the incoming state (the W-1 inputs
before the first step) ~ N(0,1) of shape [batch, dim, W-1]; dout ~ N(0,1).

Every tensor has its own PCG64 stream, ``default_rng([seed, tensor_id])``, drawn in float32 and,
for bf16 workloads, rounded to nearest-even bfloat16 on u, delta, z, B, C and dout.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

TENSOR_IDS = {"u": 0, "delta": 1, "z": 2, "B": 3, "C": 4, "D": 5, "bias": 6, "dout": 7,
              "h0": 8, "conv_x": 9, "conv_w": 10, "conv_b": 11, "conv_state": 12,
              "conv_dout": 13, "lam": 14, "u_prev": 15, "B_prev": 16}


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    dim: int
    dstate: int
    seqlen: int
    dtype: str          # "f32" or "bf16": the type of u, delta, z, B, C, out, dout, du, ...
    seed: int
    passes: tuple = field(default=("fwd",))

    @property
    def tc(self) -> int:
        return self.batch * self.dim * self.seqlen


# The five workloads.  Shapes: B=1 D=4 N=4 L=64 (tiny, fp32); the selective-copying shape
# (batch 64, model dim 64 x expand 2, L=4096, fp32); d_model 768 x 2 at L=2048 (bf16, fwd+bwd);
# d_model 2560 x 2 at L=65536 (bf16, chunked long sequence); B=4 D=2048 L=8192 (fp32 bwd).
WORKLOADS = {
    0: Workload("tiny_f32_fwd", 1, 4, 4, 64, "f32", 0, ("fwd",)),
    1: Workload("selcopy_f32_fwd", 64, 128, 16, 4096, "f32", 1, ("fwd",)),
    2: Workload("d768x2_bf16_fwdbwd", 8, 1536, 16, 2048, "bf16", 2, ("fwd", "bwd")),
    3: Workload("d2560x2_L64k_bf16_fwd", 1, 5120, 16, 65536, "bf16", 3, ("fwd",)),
    4: Workload("b4_d2048_L8k_f32_bwd", 4, 2048, 16, 8192, "f32", 4, ("bwd",)),
}


def rng(seed: int, name: str) -> np.random.Generator:
    return np.random.default_rng([int(seed), TENSOR_IDS[name]])


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to nearest-even bfloat16; returns the 16-bit patterns as uint16."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    out = np.empty(bits.shape, dtype=np.uint16)
    # chunked to bound temporary memory on the long-sequence workload
    flat_in, flat_out = bits.reshape(-1), out.reshape(-1)
    step = 1 << 24
    for s in range(0, flat_in.size, step):
        b = flat_in[s:s + step]
        nan = (b & 0x7F800000) == 0x7F800000
        nan &= (b & 0x007FFFFF) != 0
        r = ((b + np.uint32(0x7FFF) + ((b >> 16) & np.uint32(1))) >> 16).astype(np.uint16)
        r[nan] = ((b[nan] >> 16) | np.uint32(0x40)).astype(np.uint16)
        flat_out[s:s + step] = r
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


class Tensors(dict):
    """name -> numpy array.  bf16 tensors are uint16 bit patterns; ``values(name)`` gives the
    exact float32 values either way."""

    def __init__(self, dtype: str):
        super().__init__()
        self.dtype = dtype

    def values(self, name: str) -> np.ndarray | None:
        a = self.get(name)
        if a is None:
            return None
        if a.dtype == np.uint16:
            return bf16_bits_to_f32(a)
        return a


def _normal(seed, name, shape, scale=1.0):
    x = rng(seed, name).standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


def make(batch: int, dim: int, dstate: int, seqlen: int, dtype: str = "f32", seed: int = 0,
         with_z: bool = True, with_D: bool = True, with_bias: bool = True,
         with_dout: bool = False, with_h0: bool = False, with_lam: bool = False,
         with_prev: bool = False, complex_A: bool = False) -> Tensors:
    """Draw one problem.  Activation-shaped tensors follow ``dtype``; A, D, bias, h0 are fp32."""
    if dtype not in ("f32", "bf16"):
        raise ValueError(dtype)
    t = Tensors(dtype)

    def act(name, shape, scale=1.0):
        x = _normal(seed, name, shape, scale)
        return f32_to_bf16_bits(x) if dtype == "bf16" else x

    t["u"] = act("u", (batch, dim, seqlen))
    t["delta"] = act("delta", (batch, dim, seqlen), 0.5)
    t["z"] = act("z", (batch, dim, seqlen)) if with_z else None
    t["B"] = act("B", (batch, dstate, seqlen))
    t["C"] = act("C", (batch, dstate, seqlen))
    if complex_A:
        # the complex variant: rates -1/2 + i pi j of state pair j (S4D-Lin), interleaved
        # (real, imaginary) along dstate
        row = np.zeros(dstate, dtype=np.float32)
        row[0::2] = -0.5
        row[1::2] = np.pi * np.arange(dstate // 2, dtype=np.float32)
        t["A"] = np.ascontiguousarray(np.broadcast_to(row, (dim, dstate)))
    else:
        t["A"] = np.ascontiguousarray(
            np.broadcast_to(-(np.arange(dstate, dtype=np.float32) + 1.0), (dim, dstate)))
    t["D"] = _normal(seed, "D", (dim,)) if with_D else None
    if with_bias:
        dt0 = rng(seed, "bias").uniform(1e-3, 1e-1, size=dim)
        t["bias"] = np.log(np.expm1(dt0)).astype(np.float32)
    else:
        t["bias"] = None
    t["h0"] = _normal(seed, "h0", (batch, dim, dstate)) if with_h0 else None
    t["dout"] = act("dout", (batch, dim, seqlen)) if with_dout else None
    if with_lam:
        lam = rng(seed, "lam").uniform(0.0, 1.0, size=(batch, dim, seqlen)).astype(np.float32)
        t["lam"] = f32_to_bf16_bits(lam) if dtype == "bf16" else lam
    if with_prev:
        t["u_prev"] = act("u_prev", (batch, dim))
        t["B_prev"] = act("B_prev", (batch, dstate))
    return t


def make_workload(w: Workload, **kw) -> Tensors:
    kw.setdefault("with_dout", "bwd" in w.passes)
    return make(w.batch, w.dim, w.dstate, w.seqlen, w.dtype, w.seed, **kw)


def channel_slice(t: Tensors, b: int, ds) -> dict:
    """float32 values of one batch row restricted to channels ``ds`` -- an independent
    sub-problem (channels never interact in the forward), for oracle checks of samples."""
    ds = np.asarray(ds)
    sub = {}
    for name in ("u", "delta", "z", "dout"):
        v = t.get(name)
        sub[name] = None if v is None else t.values(name)[b:b + 1, ds, :]
    for name in ("B", "C"):
        sub[name] = t.values(name)[b:b + 1]
    sub["A"] = t["A"][ds]
    for name in ("D", "bias"):
        v = t.get(name)
        sub[name] = None if v is None else v[ds]
    h0 = t.get("h0")
    sub["h0"] = None if h0 is None else h0[b:b + 1, ds, :]
    return sub


def make_conv(batch: int, dim: int, seqlen: int, width: int, dtype: str = "f32", seed: int = 0,
              with_bias: bool = True, with_state: bool = False,
              with_dout: bool = False) -> Tensors:
    """Draw one problem of the short causal convolution.  x, state and dout follow ``dtype``
    (state is a copy of earlier inputs); the taps and the bias are fp32."""
    if dtype not in ("f32", "bf16"):
        raise ValueError(dtype)
    t = Tensors(dtype)

    def act(name, shape):
        x = _normal(seed, name, shape)
        return f32_to_bf16_bits(x) if dtype == "bf16" else x

    bound = 1.0 / np.sqrt(width)
    t["x"] = act("conv_x", (batch, dim, seqlen))
    t["weight"] = rng(seed, "conv_w").uniform(-bound, bound, size=(dim, width)).astype(np.float32)
    t["bias"] = (rng(seed, "conv_b").uniform(-bound, bound, size=dim).astype(np.float32)
                 if with_bias else None)
    t["state"] = act("conv_state", (batch, dim, width - 1)) if with_state else None
    t["dout"] = act("conv_dout", (batch, dim, seqlen)) if with_dout else None
    return t
