"""numpy restatement of the forward recurrence -- TEST INFRASTRUCTURE ONLY.

A second, independently written oracle of the recurrent-mode forward (page 3, recurrent-mode
sentence; page 5 Mamba-3 post, ZOH + Euler discretization bullet): vectorized over
(batch, channel, state) with a Python loop over time, softplus through ``numpy.logaddexp`` and
the sigmoid through ``scipy.special.expit`` instead of the C loop's log1p/exp formulas.  It is
only meant for small shapes (a few hundred time steps).
"""
from __future__ import annotations

import numpy as np
from scipy.special import expit


def twin_fwd(u, delta, A, B, C, D=None, z=None, bias=None, h0=None, softplus=True):
    u = np.asarray(u, dtype=np.float64)
    delta = np.asarray(delta, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    bsz, dim, L = u.shape
    N = A.shape[1]
    x = delta + (0.0 if bias is None else np.asarray(bias, np.float64)[None, :, None])
    dt = np.logaddexp(0.0, x) if softplus else x                  # [b, d, L]
    h = np.zeros((bsz, dim, N)) if h0 is None else np.array(h0, dtype=np.float64)
    ys = np.empty((bsz, dim, L))
    for t in range(L):
        decay = np.exp(dt[:, :, t, None] * A[None, :, :])         # [b, d, n]
        drive = (dt[:, :, t] * u[:, :, t])[:, :, None] * B[:, None, :, t]
        h = decay * h + drive
        ys[:, :, t] = np.einsum("bdn,bn->bd", h, C[:, :, t])
    if D is not None:
        ys = ys + np.asarray(D, np.float64)[None, :, None] * u
    if z is not None:
        zz = np.asarray(z, dtype=np.float64)
        ys = ys * zz * expit(zz)
    return ys, h
