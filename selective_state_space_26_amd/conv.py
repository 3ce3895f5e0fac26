"""Python binding of the short causal convolution entry points of libmsel.so (argument
marshalling only: the convolution, its activation and its backward run in the HIP kernels).

Layouts, as in include/msel.h:

    x, out, dout, dx       : [batch, dim, seqlen]   float32 or bfloat16, contiguous
    weight, dweight        : [dim, width]           float32
    bias, dbias            : [dim]                  float32
    state, state_out       : [batch, dim, width-1]  same dtype as x (earlier inputs, oldest first)
    dstate                 : [batch, dim, width-1]  float32
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from .scan import _dtype_code, _need, _ptr, _stream


def _conv_args(x, weight, bias, state, activation):
    if not isinstance(x, torch.Tensor) or x.dim() != 3:
        raise ValueError("x must be a [batch, dim, seqlen] tensor")
    if not isinstance(weight, torch.Tensor) or weight.dim() != 2:
        raise ValueError("weight must be a [dim, width] tensor")
    bsz, dim, L = x.shape
    W = weight.shape[1]
    dev, dt = x.device, x.dtype
    if dev.type != "cuda":
        raise ValueError("tensors must be on the GPU")
    _need(x, "x", (bsz, dim, L), dt, dev)
    _need(weight, "weight", (dim, W), torch.float32, dev)
    _need(bias, "bias", (dim,), torch.float32, dev)
    _need(state, "state", (bsz, dim, W - 1), dt, dev)
    a = _lib.ConvArgs()
    a.abi_version = _lib.ABI_VERSION
    a.batch, a.dim, a.seqlen, a.width = int(bsz), int(dim), int(L), int(W)
    a.dtype = _dtype_code(dt)
    a.activation = 1 if activation else 0
    a.reserved = 0
    a.x, a.weight, a.bias, a.state_in = _ptr(x), _ptr(weight), _ptr(bias), _ptr(state)
    return a, (bsz, dim, L, W)


def msel_conv1d_fwd(x, weight, bias=None, state=None, activation=True, out=None,
                    return_state=False, state_out=None):
    """out = silu(causal depthwise conv(x) + bias) (no SiLU when activation is False).

    state: the width-1 inputs before x[..., 0] (None: zeros).  With return_state (or a given
    state_out, which may be `state` itself to update a cache in place) the last width-1 inputs
    are written too.  Returns (out, state_out or None)."""
    a, (bsz, dim, L, W) = _conv_args(x, weight, bias, state, activation)
    dev = x.device
    out = torch.empty_like(x) if out is None else _need(out, "out", (bsz, dim, L), x.dtype, dev)
    if return_state and state_out is None:
        state_out = torch.empty((bsz, dim, W - 1), device=dev, dtype=x.dtype)
    _need(state_out, "state_out", (bsz, dim, W - 1), x.dtype, dev)
    a.out, a.state_out = _ptr(out), _ptr(state_out)
    _lib.check("msel_conv1d_fwd", _lib.load().msel_conv1d_fwd(ctypes.byref(a), _stream(dev)))
    return out, state_out


def msel_conv1d_bwd(x, weight, dout, bias=None, state=None, activation=True, want_dweight=True,
                    want_dbias=True, want_dstate=False):
    """Gradients of sum(dout * out) for msel_conv1d_fwd's out, recomputing the activation.
    Returns {"dx", "dweight", "dbias", "dstate"} (absent ones are None)."""
    a, (bsz, dim, L, W) = _conv_args(x, weight, bias, state, activation)
    dev = x.device
    _need(dout, "dout", (bsz, dim, L), x.dtype, dev)
    f32 = dict(device=dev, dtype=torch.float32)
    r = {"dx": torch.empty_like(x),
         "dweight": torch.empty((dim, W), **f32) if want_dweight else None,
         "dbias": torch.empty((dim,), **f32) if want_dbias else None,
         "dstate": torch.empty((bsz, dim, W - 1), **f32) if want_dstate else None}
    g = _lib.ConvGrads()
    g.dout, g.dx, g.dweight, g.dbias, g.dstate_in = (_ptr(dout), _ptr(r["dx"]),
                                                     _ptr(r["dweight"]), _ptr(r["dbias"]),
                                                     _ptr(r["dstate"]))
    _lib.check("msel_conv1d_bwd", _lib.load().msel_conv1d_bwd(ctypes.byref(a), ctypes.byref(g),
                                                              _stream(dev)))
    return r
