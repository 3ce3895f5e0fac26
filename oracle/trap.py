"""fp64 CPU oracle of the exponential-trapezoidal variant of the selective scan.

TEST INFRASTRUCTURE ONLY: only the test suite, the smoke check and the benchmark's CPU-baseline
leg may import this module.  It shares no code with the HIP library, and none with the C
oracle either (its agreement with the C loop at lambda = 1 is one of its pins).

What it computes (page 5, the Mamba-3 post, first bullet on the new discretization): the
integral of the input over a step is approximated from both ends of the interval instead of
one, mixed by a data-dependent weight lambda, which makes the recurrence apply a two-tap
convolution to the state's input.  Written out, for batch row b, channel d, state n and step t:

    Delta_t = softplus(delta_t + bias[d])        (or delta_t + bias[d] without the softplus)
    a_t     = exp(Delta_t * A[d, n])             the transition over the step (exact)
    h_t     = a_t h_{t-1} + Delta_t * ( lambda_t B_t u_t + (1 - lambda_t) a_t B_{t-1} u_{t-1} )
    y_t     = sum_n C_t h_t + D[d] u_t,          out_t = y_t * silu(z_t)

Readings where the page is silent (each is listed in the design notes):

* The right end of the interval is the current step (weight lambda_t), the left end the
  previous step's input carried over the step by the exact transition a_t -- the
  "exponential" part; lambda_t = 1 gives back the zero-order-hold/Euler scan of the other
  entry points exactly, and lambda_t = 1/2 the trapezoidal rule.
* lambda has the shape of delta, one value per (b, d, t), already in [0, 1].
* The input before step 0, B_{-1} u_{-1}, comes from u_prev[b, d] and B_prev[b, n] (the last
  step of a sequence being continued); without them it is 0.
* h0, the gate, D, the bias and the chunk states are as in the other entry points.

Everything is float64; the loop runs over time, vectorized over (b, d, n).  ``bwd`` is reverse
mode of that loop written by hand, one operation of a step at a time, run backwards in time.
"""
from __future__ import annotations

import numpy as np


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def _softplus(x):
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def fwd(u, delta, lam, A, B, C, D=None, z=None, bias=None, h0=None, u_prev=None, B_prev=None,
        softplus=True, chunk_len=None):
    """Returns (out [b,d,L], final_state [b,d,n], chunk_states [b,d,nc,n] or None).

    chunk_states[..., c, :] is the state before step c * chunk_len (h0 for c = 0)."""
    u, delta, lam, A, B, C = map(_f64, (u, delta, lam, A, B, C))
    bsz, dim, L = u.shape
    N = A.shape[1]
    x = delta + (0.0 if bias is None else _f64(bias)[None, :, None])
    dt = _softplus(x) if softplus else x                              # [b, d, L]
    h = np.zeros((bsz, dim, N)) if h0 is None else _f64(h0).copy()
    up = np.zeros((bsz, dim)) if u_prev is None else _f64(u_prev)      # u_{t-1}
    Bp = np.zeros((bsz, N)) if B_prev is None else _f64(B_prev)        # B_{t-1}
    y = np.zeros((bsz, dim, L))
    nc = None if chunk_len is None else -(-L // chunk_len)
    cs = None if chunk_len is None else np.zeros((bsz, dim, nc, N))
    for t in range(L):
        if chunk_len is not None and t % chunk_len == 0:
            cs[:, :, t // chunk_len, :] = h
        a = np.exp(dt[:, :, t, None] * A[None, :, :])                   # [b, d, n]
        right = lam[:, :, t, None] * B[:, None, :, t] * u[:, :, t, None]
        left = (1.0 - lam[:, :, t, None]) * a * Bp[:, None, :] * up[:, :, None]
        h = a * h + dt[:, :, t, None] * (right + left)
        y[:, :, t] = np.sum(C[:, None, :, t] * h, axis=2)
        up = u[:, :, t]
        Bp = B[:, :, t]
    if D is not None:
        y += _f64(D)[None, :, None] * u
    if z is not None:
        zz = _f64(z)
        y *= zz / (1.0 + np.exp(-zz))
    return y, h, cs


def bwd(u, delta, lam, A, B, C, dout, D=None, z=None, bias=None, h0=None, u_prev=None,
        B_prev=None, softplus=True):
    """Gradients of sum(dout * out) for fwd(...): reverse mode of the forward loop, one step at
    a time in reverse, each operation of the step differentiated by hand.  Returns a dict with
    du, ddelta (w.r.t. the raw delta), dlam, dz, dA, dB, dC, dD, ddelta_bias, dh0, du_prev and
    dB_prev (the inputs of the step before the first)."""
    u, delta, lam, A, B, C, dout = map(_f64, (u, delta, lam, A, B, C, dout))
    bsz, dim, L = u.shape
    N = A.shape[1]
    x = delta + (0.0 if bias is None else _f64(bias)[None, :, None])
    dt = _softplus(x) if softplus else x
    up0 = np.zeros((bsz, dim)) if u_prev is None else _f64(u_prev)
    Bp0 = np.zeros((bsz, N)) if B_prev is None else _f64(B_prev)
    # forward again, keeping every state
    hs = np.zeros((L + 1, bsz, dim, N))
    hs[0] = 0.0 if h0 is None else _f64(h0)
    ys = np.zeros((bsz, dim, L))
    for t in range(L):
        up = up0 if t == 0 else u[:, :, t - 1]
        Bp = Bp0 if t == 0 else B[:, :, t - 1]
        a = np.exp(dt[:, :, t, None] * A[None])
        right = lam[:, :, t, None] * B[:, None, :, t] * u[:, :, t, None]
        left = (1.0 - lam[:, :, t, None]) * a * Bp[:, None, :] * up[:, :, None]
        hs[t + 1] = a * hs[t] + dt[:, :, t, None] * (right + left)
        ys[:, :, t] = np.sum(C[:, None, :, t] * hs[t + 1], axis=2)
    if D is not None:
        ys += _f64(D)[None, :, None] * u
    g = {k: np.zeros_like(v) for k, v in (("du", u), ("dlam", lam), ("dB", B), ("dC", C))}
    ddt = np.zeros_like(dt)
    dA = np.zeros_like(A)
    dup0 = np.zeros_like(up0)
    dBp0 = np.zeros_like(Bp0)
    # the gate
    if z is not None:
        zz = _f64(z)
        sg = 1.0 / (1.0 + np.exp(-zz))
        dy = dout * zz * sg
        dz = dout * ys * sg * (1.0 + zz * (1.0 - sg))
    else:
        dy, dz = dout, None
    dD = np.sum(dy * u, axis=(0, 2))
    if D is not None:
        g["du"] += _f64(D)[None, :, None] * dy
    gh = np.zeros((bsz, dim, N))  # dL/dh_t, accumulated from the future
    for t in range(L - 1, -1, -1):
        up = up0 if t == 0 else u[:, :, t - 1]
        Bp = Bp0 if t == 0 else B[:, :, t - 1]
        h_old, h_new = hs[t], hs[t + 1]
        a = np.exp(dt[:, :, t, None] * A[None])
        # y_t = C_t . h_new
        gh = gh + C[:, None, :, t] * dy[:, :, t, None]
        g["dC"][:, :, t] += np.sum(dy[:, :, t, None] * h_new, axis=1)
        # h_new = a h_old + dt (right + left)
        lt = lam[:, :, t, None]
        dtt = dt[:, :, t, None]
        right = lt * B[:, None, :, t] * u[:, :, t, None]
        left = (1.0 - lt) * a * Bp[:, None, :] * up[:, :, None]
        d_a = gh * h_old + gh * dtt * (1.0 - lt) * Bp[:, None, :] * up[:, :, None]
        ddt[:, :, t] += np.sum(gh * (right + left), axis=2)
        # right = lam B_t u_t ; left = (1 - lam) a B_{t-1} u_{t-1}
        g["dlam"][:, :, t] += np.sum(gh * dtt * (B[:, None, :, t] * u[:, :, t, None]
                                                 - a * Bp[:, None, :] * up[:, :, None]), axis=2)
        g["dB"][:, :, t] += np.sum(gh * dtt * lt * u[:, :, t, None], axis=1)
        g["du"][:, :, t] += np.sum(gh * dtt * lt * B[:, None, :, t], axis=2)
        dBp = np.sum(gh * dtt * (1.0 - lt) * a * up[:, :, None], axis=1)
        dup = np.sum(gh * dtt * (1.0 - lt) * a * Bp[:, None, :], axis=2)
        if t == 0:
            dBp0 += dBp
            dup0 += dup
        else:
            g["dB"][:, :, t - 1] += dBp
            g["du"][:, :, t - 1] += dup
        # a = exp(dt A)
        ddt[:, :, t] += np.sum(d_a * A[None] * a, axis=2)
        dA += np.sum(d_a * dtt * a, axis=0)
        gh = gh * a
    sig = 1.0 / (1.0 + np.exp(-x)) if softplus else np.ones_like(x)
    ddelta = ddt * sig
    return dict(du=g["du"], ddelta=ddelta, dlam=g["dlam"], dz=dz, dA=dA, dB=g["dB"],
                dC=g["dC"], dD=dD, ddelta_bias=ddelta.sum(axis=(0, 2)), dh0=gh, du_prev=dup0,
                dB_prev=dBp0)
