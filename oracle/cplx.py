"""fp64 CPU oracle of the complex-valued (rotational) variant of the selective scan.

TEST INFRASTRUCTURE ONLY: only the test suite, the smoke check and the benchmark's CPU-baseline
leg may import this module.  It shares no code with the HIP library or with the C oracle.

What it computes (page 5, the Mamba-3 post, second bullet: a complex-valued state recovers
state tracking such as parity; the transition is split into a scaling and a rotation in a
two-dimensional plane, so no complex arithmetic is needed in the kernels).  The states are
taken in pairs (2j, 2j+1) as one complex state h_j = h_{2j} + i h_{2j+1}:

    Delta_t = softplus(delta_t + bias[d])     (or delta_t + bias[d] without the softplus)
    a_t     = exp(Delta_t * (A[d, 2j] + i A[d, 2j+1]))     scaling exp(Delta A_re), rotation
                                                           by the angle Delta A_im
    h_t     = a_t h_{t-1} + Delta_t u_t (B[b, 2j, t] + i B[b, 2j+1, t])
    y_t     = sum_j ( C[b, 2j, t] Re h_t + C[b, 2j+1, t] Im h_t ) + D[d] u_t
    out_t   = y_t * silu(z_t)

Readings (each is listed in the design notes): A stores the complex rates interleaved
(real, imaginary) in its [dim, dstate] layout, dstate even; B, C and the states keep their
layouts, rows 2j and 2j+1 being a pair's two components; the readout is the real inner product
of C and h, so with every A[d, 2j+1] = 0 the variant is the real scan with A[d, 2j+1] replaced
by A[d, 2j].  h0, final states and chunk states hold (Re, Im) interleaved the same way.

This is written with numpy complex128, a loop over time vectorized over (b, d, j); ``bwd`` is
reverse mode of that loop by hand, run backwards in time.
"""
from __future__ import annotations

import numpy as np


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def _softplus(x):
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def fwd(u, delta, A, B, C, D=None, z=None, bias=None, h0=None, softplus=True, chunk_len=None):
    """Returns (out [b,d,L], final_state [b,d,N], chunk_states [b,d,nc,N] or None), the states
    as (Re, Im) pairs; chunk_states[..., c, :] is the state before step c * chunk_len."""
    u, delta, A, B, C = map(_f64, (u, delta, A, B, C))
    bsz, dim, L = u.shape
    N = A.shape[1]
    if N % 2:
        raise ValueError("the complex variant needs an even dstate")
    J = N // 2
    Ac = A[:, 0::2] + 1j * A[:, 1::2]                                   # [d, j]
    Bc = B[:, 0::2, :] + 1j * B[:, 1::2, :]                             # [b, j, L]
    x = delta + (0.0 if bias is None else _f64(bias)[None, :, None])
    dt = _softplus(x) if softplus else x
    if h0 is None:
        h = np.zeros((bsz, dim, J), dtype=np.complex128)
    else:
        hh = _f64(h0)
        h = hh[:, :, 0::2] + 1j * hh[:, :, 1::2]

    def interleave(hc):
        out = np.empty(hc.shape[:-1] + (N,))
        out[..., 0::2] = hc.real
        out[..., 1::2] = hc.imag
        return out

    y = np.zeros((bsz, dim, L))
    nc = None if chunk_len is None else -(-L // chunk_len)
    cs = None if chunk_len is None else np.zeros((bsz, dim, nc, N))
    for t in range(L):
        if chunk_len is not None and t % chunk_len == 0:
            cs[:, :, t // chunk_len, :] = interleave(h)
        a = np.exp(dt[:, :, t, None] * Ac[None, :, :])
        h = a * h + (dt[:, :, t] * u[:, :, t])[:, :, None] * Bc[:, None, :, t]
        y[:, :, t] = np.sum(C[:, None, 0::2, t] * h.real + C[:, None, 1::2, t] * h.imag, axis=2)
    if D is not None:
        y += _f64(D)[None, :, None] * u
    if z is not None:
        zz = _f64(z)
        y *= zz / (1.0 + np.exp(-zz))
    return y, interleave(h), cs


def bwd(u, delta, A, B, C, dout, D=None, z=None, bias=None, h0=None, softplus=True):
    """Gradients of sum(dout * out) for fwd(...): reverse mode of the forward loop by hand, in
    complex arithmetic.  With G = dL/dRe h + i dL/dIm h, a step h = a h' + p sends
    G' = conj(a) G back to h', Re(conj(G) dp) to p's inputs and Re(conj(G) da) to a's.
    Returns du, ddelta (w.r.t. the raw delta), dz, dA, dB, dC, dD, ddelta_bias, dh0; dA, dh0
    interleaved (Re, Im) like A and h0."""
    u, delta, A, B, C, dout = map(_f64, (u, delta, A, B, C, dout))
    bsz, dim, L = u.shape
    N = A.shape[1]
    J = N // 2
    Ac = A[:, 0::2] + 1j * A[:, 1::2]
    Bc = B[:, 0::2, :] + 1j * B[:, 1::2, :]
    x = delta + (0.0 if bias is None else _f64(bias)[None, :, None])
    dt = _softplus(x) if softplus else x
    hs = np.zeros((L + 1, bsz, dim, J), dtype=np.complex128)
    if h0 is not None:
        hh = _f64(h0)
        hs[0] = hh[:, :, 0::2] + 1j * hh[:, :, 1::2]
    ys = np.zeros((bsz, dim, L))
    for t in range(L):
        a = np.exp(dt[:, :, t, None] * Ac[None])
        hs[t + 1] = a * hs[t] + (dt[:, :, t] * u[:, :, t])[:, :, None] * Bc[:, None, :, t]
        ys[:, :, t] = np.sum(C[:, None, 0::2, t] * hs[t + 1].real
                             + C[:, None, 1::2, t] * hs[t + 1].imag, axis=2)
    if D is not None:
        ys += _f64(D)[None, :, None] * u
    if z is not None:
        zz = _f64(z)
        sg = 1.0 / (1.0 + np.exp(-zz))
        dy = dout * zz * sg
        dz = dout * ys * sg * (1.0 + zz * (1.0 - sg))
    else:
        dy, dz = dout, None
    du = np.zeros_like(u) if D is None else _f64(D)[None, :, None] * dy
    ddt = np.zeros_like(dt)
    dAc = np.zeros((dim, J), dtype=np.complex128)
    dB = np.zeros_like(B)
    dC = np.zeros_like(C)
    G = np.zeros((bsz, dim, J), dtype=np.complex128)
    for t in range(L - 1, -1, -1):
        h_new, h_old = hs[t + 1], hs[t]
        # y_t = sum_j C_r Re h + C_i Im h
        G = G + dy[:, :, t, None] * (C[:, None, 0::2, t] + 1j * C[:, None, 1::2, t])
        dC[:, 0::2, t] += np.sum(dy[:, :, t, None] * h_new.real, axis=1)
        dC[:, 1::2, t] += np.sum(dy[:, :, t, None] * h_new.imag, axis=1)
        # h_new = a h_old + dt u Bc
        a = np.exp(dt[:, :, t, None] * Ac[None])
        gp = np.conj(G)                                     # Re(gp * d(.)) is the pullback
        pin = dt[:, :, t, None] * u[:, :, t, None]
        dB[:, 0::2, t] += np.sum((gp * pin).real, axis=1)   # d/dB_r: Re(conj(G) pin)
        dB[:, 1::2, t] += np.sum((gp * 1j * pin).real, axis=1)
        du[:, :, t] += np.sum((gp * dt[:, :, t, None] * Bc[:, None, :, t]).real, axis=2)
        ddt[:, :, t] += np.sum((gp * u[:, :, t, None] * Bc[:, None, :, t]).real, axis=2)
        X = gp * a * h_old                                   # conj(G) a h_old
        ddt[:, :, t] += np.sum((X * Ac[None]).real, axis=2)
        dAc += np.sum(X * dt[:, :, t, None], axis=0)        # Re part -> dA_r, Re(i X dt) -> dA_i
        G = np.conj(a) * G
    dD = np.sum(dy * u, axis=(0, 2))
    sig = 1.0 / (1.0 + np.exp(-x)) if softplus else np.ones_like(x)
    ddelta = ddt * sig
    dA = np.empty((dim, N))
    dA[:, 0::2] = dAc.real
    dA[:, 1::2] = (1j * dAc).real                            # d/dA_i = Re(i conj(G) dt a h)
    dh0 = np.empty((bsz, dim, N))
    dh0[:, :, 0::2] = G.real
    dh0[:, :, 1::2] = G.imag
    return dict(du=du, ddelta=ddelta, dz=dz, dA=dA, dB=dB, dC=dC, dD=dD,
                ddelta_bias=ddelta.sum(axis=(0, 2)), dh0=dh0)
