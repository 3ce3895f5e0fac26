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

Everything is float64; the loop runs over time, vectorized over (b, d, n).
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
