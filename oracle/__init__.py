"""fp64 CPU oracle of the selective SSM scan -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this package.  The product path (the HIP library and its Python binding) never does, and
this package never imports the product package.  The two share nothing but the seeded input
generator ``msel_inputs``.

The implementations here:

* ``fwd`` / ``chunk_states_formula`` / ``bwd`` call the plain C loop in ``msel_oracle.c``
  (sequential over time, one (batch, channel) recurrence per work unit, double precision).
* ``trap.py`` is the exponential-trapezoidal variant of the scan (Mamba-3), a numpy loop over
  time in float64 that shares nothing with the C loop.
* ``cplx.py`` is the complex-valued (rotational) variant: state pairs as complex numbers,
  numpy complex128.
* ``conv.py`` is the short causal convolution and activation that feed the scan (forward,
  hand-derived backward, convolutional state), written out tap by tap in float64.
* ``twin_fwd`` in ``twin.py`` is a numpy restatement, vectorized over (batch, channel, state)
  with a Python loop over time, used to cross-check the C loop on small shapes.

Every function states the passage of the pages it follows in the C source header.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "msel_oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (no fast-math, no fused multiply-add)."""
    if force or not os.path.exists(_SO):
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
               "-fno-fast-math", "-Wall", "-Wextra", "-o", _SO + ".tmp", _SRC, "-lm"]
        subprocess.run(cmd, check=True, cwd=_HERE)
        os.replace(_SO + ".tmp", _SO)
    return _SO


class _In(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_long), ("dim", ctypes.c_long), ("dstate", ctypes.c_long),
                ("seqlen", ctypes.c_long), ("softplus", ctypes.c_int)] + [
        (name, ctypes.c_void_p) for name in ("u", "delta", "A", "B", "C", "D", "z", "bias", "h0")]


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build(force=True)
        lib = ctypes.CDLL(_SO)
        P = ctypes.c_void_p
        lib.oracle_fwd.argtypes = [ctypes.POINTER(_In), P, P, ctypes.c_long, P, ctypes.c_int]
        lib.oracle_chunk_states_formula.argtypes = [ctypes.POINTER(_In), ctypes.c_long, P, P,
                                                    ctypes.c_int]
        lib.oracle_bwd.argtypes = [ctypes.POINTER(_In), P, P, P, P, P, P, P, P, P, P,
                                   ctypes.c_int]
        for f in (lib.oracle_fwd, lib.oracle_chunk_states_formula, lib.oracle_bwd):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _f64(x):
    if x is None:
        return None
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data


class _Problem:
    """Holds float64 copies of the inputs and the ctypes struct that points at them."""

    def __init__(self, u, delta, A, B, C, D=None, z=None, bias=None, h0=None, softplus=True):
        self.u, self.delta, self.A = _f64(u), _f64(delta), _f64(A)
        self.B, self.C, self.D = _f64(B), _f64(C), _f64(D)
        self.z, self.bias, self.h0 = _f64(z), _f64(bias), _f64(h0)
        bsz, dim, L = self.u.shape
        N = self.A.shape[1]
        if self.delta.shape != (bsz, dim, L) or self.A.shape != (dim, N):
            raise ValueError("shape mismatch for delta or A")
        if self.B.shape != (bsz, N, L) or self.C.shape != (bsz, N, L):
            raise ValueError("B and C must be [batch, dstate, seqlen]")
        if self.z is not None and self.z.shape != (bsz, dim, L):
            raise ValueError("z must be [batch, dim, seqlen]")
        if self.h0 is not None and self.h0.shape != (bsz, dim, N):
            raise ValueError("h0 must be [batch, dim, dstate]")
        self.shape = (bsz, dim, N, L)
        self.st = _In(bsz, dim, N, L, 1 if softplus else 0, *[
            _ptr(a) for a in (self.u, self.delta, self.A, self.B, self.C, self.D, self.z,
                              self.bias, self.h0)])


def fwd(u, delta, A, B, C, D=None, z=None, bias=None, h0=None, softplus=True,
        chunk_len=None, nthreads=None):
    """Sequential recurrent-mode forward.  Returns (out, final_state[, chunk_states])."""
    pb = _Problem(u, delta, A, B, C, D, z, bias, h0, softplus)
    bsz, dim, N, L = pb.shape
    out = np.empty((bsz, dim, L))
    fin = np.empty((bsz, dim, N))
    cs = None
    if chunk_len:
        cs = np.empty((bsz, dim, (L + chunk_len - 1) // chunk_len, N))
    rc = _load().oracle_fwd(ctypes.byref(pb.st), _ptr(out), _ptr(fin), int(chunk_len or 0),
                            _ptr(cs), int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"oracle_fwd failed: {rc}")
    return (out, fin, cs) if chunk_len else (out, fin)


def chunk_states_formula(u, delta, A, B, chunk_len, h0=None, bias=None, softplus=True,
                         nthreads=None):
    """Chunk states from per-chunk (transition, local end state) pairs and the link step."""
    bsz, dim, L = np.shape(u)
    zeros_c = np.zeros_like(np.asarray(B, dtype=np.float64))
    pb = _Problem(u, delta, A, B, zeros_c, None, None, bias, h0, softplus)
    N = pb.shape[2]
    cs = np.empty((bsz, dim, (L + chunk_len - 1) // chunk_len, N))
    fin = np.empty((bsz, dim, N))
    rc = _load().oracle_chunk_states_formula(ctypes.byref(pb.st), int(chunk_len), _ptr(cs),
                                             _ptr(fin), int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"oracle_chunk_states_formula failed: {rc}")
    return cs, fin


def bwd(u, delta, A, B, C, dout, D=None, z=None, bias=None, h0=None, softplus=True,
        nthreads=None):
    """Hand-derived backward with recomputed states.  Returns a dict of gradients."""
    pb = _Problem(u, delta, A, B, C, D, z, bias, h0, softplus)
    bsz, dim, N, L = pb.shape
    g = _f64(dout)
    if g.shape != (bsz, dim, L):
        raise ValueError("dout must be [batch, dim, seqlen]")
    r = {
        "du": np.empty((bsz, dim, L)), "ddelta": np.empty((bsz, dim, L)),
        "dz": np.empty((bsz, dim, L)) if pb.z is not None else None,
        "dA": np.empty((dim, N)), "dB": np.empty((bsz, N, L)), "dC": np.empty((bsz, N, L)),
        "dD": np.empty((dim,)), "ddelta_bias": np.empty((dim,)), "dh0": np.empty((bsz, dim, N)),
    }
    rc = _load().oracle_bwd(ctypes.byref(pb.st), _ptr(g), _ptr(r["du"]), _ptr(r["ddelta"]),
                            _ptr(r["dz"]), _ptr(r["dA"]), _ptr(r["dB"]), _ptr(r["dC"]),
                            _ptr(r["dD"]), _ptr(r["ddelta_bias"]), _ptr(r["dh0"]),
                            int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"oracle_bwd failed: {rc}")
    return r


from .twin import twin_fwd  # noqa: E402  (numpy restatement, no C)

__all__ = ["build", "fwd", "chunk_states_formula", "bwd", "twin_fwd", "default_threads"]
