"""fp64 CPU oracle of the short causal convolution and activation that feed the selective scan.

TEST INFRASTRUCTURE ONLY: only the test suite, the smoke check and the benchmark's CPU-baseline
leg may import this module.  It shares no code with the HIP library and imports nothing from
the product package.

What it computes (the web pages collected on "mamba paper"):

* The selective SSM block applies an input projection, a short convolution, an activation, the
  scan and an output projection, and its backward recomputes the convolution and activation
  outputs instead of storing them (page 4, Gu & Dao "Mamba", Appendix D "Hardware-aware
  Algorithm For Selective SSMs", Memory paragraph).
* The layer's cache keeps convolutional states beside the SSM state, and the fast path calls a
  dedicated causal-convolution kernel next to the scan kernels (page 1, "A Secret Weapon For
  mamba paper", the paragraphs on the cache and on the CUDA kernels).

Readings where the pages are silent (each is listed in the design notes):

* Depthwise and causal.  Channel d has its own W taps w[d, 0..W-1] and a bias b[d]:
  pre[t] = b[d] + sum_k w[d, k] * xe[t + k], where xe is the extended sequence [s, x] of
  length W-1+L, so tap W-1 multiplies the current input x[t] and tap 0 the input W-1 steps
  back.
* The convolutional state s[b, d, 0..W-2] holds the W-1 inputs before the first step (s[j] is
  the input at time j-(W-1)); with no state they are 0.  The state after the call is the last
  W-1 entries of xe.
* The activation is SiLU, a(p) = p * sigmoid(p), or the identity.
* "Short" means W in 1..4.

Everything is float64.  The forward is the definition above written out tap by tap; the
backward is the chain rule of it, derived by hand: dpre = dout * a'(pre) with
a'(p) = sigmoid(p) * (1 + p * (1 - sigmoid(p))), then every tap scatters w[d, k] * dpre[t]
back to xe[t + k] and gathers dpre[t] * xe[t + k] into dw[d, k].
"""
from __future__ import annotations

import numpy as np


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def _extended(x, state, W):
    """[s, x] along time: shape [batch, dim, W-1+L]."""
    bsz, dim, _ = x.shape
    s = np.zeros((bsz, dim, W - 1)) if state is None else _f64(state).reshape(bsz, dim, W - 1)
    return np.concatenate([s, x], axis=2)


def _sigmoid(p):
    return 1.0 / (1.0 + np.exp(-p))


def preactivation(x, w, bias=None, state=None):
    """pre[b, d, t] = bias[d] + sum_k w[d, k] * xe[b, d, t + k] (see the module docstring)."""
    x, w = _f64(x), _f64(w)
    W = w.shape[1]
    L = x.shape[2]
    xe = _extended(x, state, W)
    pre = np.zeros_like(x)
    if bias is not None:
        pre += _f64(bias)[None, :, None]
    for k in range(W):
        pre += w[None, :, k, None] * xe[:, :, k:k + L]
    return pre


def fwd(x, w, bias=None, state=None, silu=True):
    """Returns (out, final_state): out = a(pre), final_state = the last W-1 entries of [s, x]."""
    x, w = _f64(x), _f64(w)
    W = w.shape[1]
    pre = preactivation(x, w, bias, state)
    out = pre * _sigmoid(pre) if silu else pre
    xe = _extended(x, state, W)
    final_state = xe[:, :, xe.shape[2] - (W - 1):]
    return out, final_state


def bwd(x, w, dout, bias=None, state=None, silu=True):
    """Gradients of sum(dout * out) with respect to x, w, bias and the incoming state."""
    x, w, dout = _f64(x), _f64(w), _f64(dout)
    W = w.shape[1]
    L = x.shape[2]
    pre = preactivation(x, w, bias, state)
    if silu:
        sg = _sigmoid(pre)
        dpre = dout * sg * (1.0 + pre * (1.0 - sg))
    else:
        dpre = dout
    xe = _extended(x, state, W)
    dxe = np.zeros_like(xe)
    dw = np.zeros_like(w)
    for k in range(W):
        dxe[:, :, k:k + L] += w[None, :, k, None] * dpre
        dw[:, k] = np.sum(dpre * xe[:, :, k:k + L], axis=(0, 2))
    return dict(dx=dxe[:, :, W - 1:], dweight=dw, dbias=dpre.sum(axis=(0, 2)),
                dstate=dxe[:, :, :W - 1])
