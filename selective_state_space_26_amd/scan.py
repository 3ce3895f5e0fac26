"""Python binding of libmsel.so: the same three entry points, argument marshalling only.

PyTorch supplies device memory and the current HIP stream; every step of the scan runs in the
library's HIP kernels.  Tensors must already be on the GPU, contiguous, with the layouts of
include/msel.h:

    u, delta, z, out, dout, du, ddelta, dz : [batch, dim, seqlen]   float32 or bfloat16
    B, C                                   : [batch, dstate, seqlen] same dtype as u
    A                                      : [dim, dstate]           float32
    D, delta_bias                          : [dim]                   float32
    h0, final_state, dh0                   : [batch, dim, dstate]    float32
    chunk_states                           : [batch, dim, n_chunks, dstate] float32
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return _lib.MSEL_F32
    if dt == torch.bfloat16:
        return _lib.MSEL_BF16
    raise TypeError(f"activation dtype must be float32 or bfloat16, got {dt}")


def _need(t, name, shape, dtype, device):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def chunk_len() -> int:
    return int(_lib.load().msel_chunk_len())


def num_chunks(seqlen: int) -> int:
    return int(_lib.load().msel_num_chunks(int(seqlen)))


def _args(u, delta, A, B, C, D, z, delta_bias, h0, delta_softplus):
    if u.dim() != 3:
        raise ValueError("u must be [batch, dim, seqlen]")
    bsz, dim, L = u.shape
    N = A.shape[1] if A.dim() == 2 else -1
    dev, dt = u.device, u.dtype
    if dev.type != "cuda":
        raise ValueError("tensors must be on the GPU")
    _need(u, "u", (bsz, dim, L), dt, dev)
    _need(delta, "delta", (bsz, dim, L), dt, dev)
    _need(A, "A", (dim, N), torch.float32, dev)
    _need(B, "B", (bsz, N, L), dt, dev)
    _need(C, "C", (bsz, N, L), dt, dev)
    _need(z, "z", (bsz, dim, L), dt, dev)
    _need(D, "D", (dim,), torch.float32, dev)
    _need(delta_bias, "delta_bias", (dim,), torch.float32, dev)
    _need(h0, "h0", (bsz, dim, N), torch.float32, dev)
    a = _lib.ScanArgs()
    a.abi_version = _lib.ABI_VERSION
    a.batch, a.dim, a.dstate, a.seqlen = int(bsz), int(dim), int(N), int(L)
    a.dtype = _dtype_code(dt)
    a.delta_softplus = 1 if delta_softplus else 0
    a.reserved = 0
    a.u, a.delta, a.B, a.C, a.z = _ptr(u), _ptr(delta), _ptr(B), _ptr(C), _ptr(z)
    a.A, a.D, a.delta_bias, a.h0 = _ptr(A), _ptr(D), _ptr(delta_bias), _ptr(h0)
    return a, (bsz, dim, N, L)


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def msel_scan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True,
                  h0=None, return_final_state=True, return_chunk_states=False, out=None,
                  final_state=None, chunk_states=None):
    """Fused forward scan.  Returns (out, final_state or None, chunk_states or None)."""
    a, (bsz, dim, N, L) = _args(u, delta, A, B, C, D, z, delta_bias, h0, delta_softplus)
    dev = u.device
    out = torch.empty_like(u) if out is None else _need(out, "out", (bsz, dim, L), u.dtype, dev)
    if return_final_state and final_state is None:
        final_state = torch.empty((bsz, dim, N), device=dev, dtype=torch.float32)
    if return_chunk_states and chunk_states is None:
        chunk_states = torch.empty((bsz, dim, num_chunks(L), N), device=dev,
                                   dtype=torch.float32)
    _need(final_state, "final_state", (bsz, dim, N), torch.float32, dev)
    _need(chunk_states, "chunk_states", (bsz, dim, num_chunks(L), N), torch.float32, dev)
    a.out, a.final_state, a.chunk_states = _ptr(out), _ptr(final_state), _ptr(chunk_states)
    _lib.check("msel_scan_fwd", _lib.load().msel_scan_fwd(ctypes.byref(a), _stream(dev)))
    return out, final_state, chunk_states


def msel_scan_trap_fwd(u, delta, lam, A, B, C, D=None, z=None, delta_bias=None,
                       delta_softplus=True, h0=None, u_prev=None, B_prev=None,
                       return_final_state=True, return_chunk_states=False, out=None,
                       final_state=None, chunk_states=None):
    """Fused forward scan with the exponential-trapezoidal rule (lam: [batch, dim, seqlen] in
    [0, 1]; u_prev [batch, dim] and B_prev [batch, dstate]: the inputs of the step before the
    first).  Returns (out, final_state or None, chunk_states or None)."""
    a, (bsz, dim, N, L) = _args(u, delta, A, B, C, D, z, delta_bias, h0, delta_softplus)
    dev, dt = u.device, u.dtype
    _need(lam, "lam", (bsz, dim, L), dt, dev)
    _need(u_prev, "u_prev", (bsz, dim), dt, dev)
    _need(B_prev, "B_prev", (bsz, N), dt, dev)
    if lam is None:
        raise ValueError("lam is required")
    out = torch.empty_like(u) if out is None else _need(out, "out", (bsz, dim, L), dt, dev)
    if return_final_state and final_state is None:
        final_state = torch.empty((bsz, dim, N), device=dev, dtype=torch.float32)
    if return_chunk_states and chunk_states is None:
        chunk_states = torch.empty((bsz, dim, num_chunks(L), N), device=dev,
                                   dtype=torch.float32)
    _need(final_state, "final_state", (bsz, dim, N), torch.float32, dev)
    _need(chunk_states, "chunk_states", (bsz, dim, num_chunks(L), N), torch.float32, dev)
    a.out, a.final_state, a.chunk_states = _ptr(out), _ptr(final_state), _ptr(chunk_states)
    tr = _lib.TrapArgs()
    tr.lambda_, tr.u_prev, tr.B_prev = _ptr(lam), _ptr(u_prev), _ptr(B_prev)
    _lib.check("msel_scan_trap_fwd", _lib.load().msel_scan_trap_fwd(ctypes.byref(a),
                                                                    ctypes.byref(tr),
                                                                    _stream(dev)))
    return out, final_state, chunk_states


def msel_scan_complex_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None,
                          delta_softplus=True, h0=None, return_final_state=True,
                          return_chunk_states=False, out=None, final_state=None,
                          chunk_states=None):
    """Fused forward of the complex-valued (rotational) scan: states (2j, 2j+1) are the real
    and imaginary parts of one complex state, A[:, 2j] + i A[:, 2j+1] its rate (dstate even).
    Returns (out, final_state or None, chunk_states or None)."""
    a, (bsz, dim, N, L) = _args(u, delta, A, B, C, D, z, delta_bias, h0, delta_softplus)
    dev = u.device
    out = torch.empty_like(u) if out is None else _need(out, "out", (bsz, dim, L), u.dtype, dev)
    if return_final_state and final_state is None:
        final_state = torch.empty((bsz, dim, N), device=dev, dtype=torch.float32)
    if return_chunk_states and chunk_states is None:
        chunk_states = torch.empty((bsz, dim, num_chunks(L), N), device=dev,
                                   dtype=torch.float32)
    _need(final_state, "final_state", (bsz, dim, N), torch.float32, dev)
    _need(chunk_states, "chunk_states", (bsz, dim, num_chunks(L), N), torch.float32, dev)
    a.out, a.final_state, a.chunk_states = _ptr(out), _ptr(final_state), _ptr(chunk_states)
    _lib.check("msel_scan_complex_fwd",
               _lib.load().msel_scan_complex_fwd(ctypes.byref(a), _stream(dev)))
    return out, final_state, chunk_states


def msel_scan_chunk_carry(u, delta, A, B, delta_bias=None, delta_softplus=True, h0=None,
                          return_final_state=True, chunk_states=None, final_state=None):
    """Chunk-carry pass.  Returns (chunk_states, final_state or None)."""
    if u.dim() != 3 or A.dim() != 2:
        raise ValueError("u must be [batch, dim, seqlen] and A [dim, dstate]")
    bsz, dim, L = u.shape
    N = A.shape[1]
    dev = u.device
    _need(B, "B", (bsz, N, L), u.dtype, dev)
    a, _ = _args(u, delta, A, B, B, None, None, delta_bias, h0, delta_softplus)
    a.C = None
    if chunk_states is None:
        chunk_states = torch.empty((bsz, dim, num_chunks(L), N), device=dev,
                                   dtype=torch.float32)
    if return_final_state and final_state is None:
        final_state = torch.empty((bsz, dim, N), device=dev, dtype=torch.float32)
    _need(chunk_states, "chunk_states", (bsz, dim, num_chunks(L), N), torch.float32, dev)
    _need(final_state, "final_state", (bsz, dim, N), torch.float32, dev)
    a.chunk_states, a.final_state = _ptr(chunk_states), _ptr(final_state)
    _lib.check("msel_scan_chunk_carry",
               _lib.load().msel_scan_chunk_carry(ctypes.byref(a), _stream(dev)))
    return chunk_states, final_state


def _chunk_carry_out(u, A, chunk_states, final_state, return_final_state):
    bsz, dim, L = u.shape
    N = A.shape[1]
    dev = u.device
    if chunk_states is None:
        chunk_states = torch.empty((bsz, dim, num_chunks(L), N), device=dev,
                                   dtype=torch.float32)
    if return_final_state and final_state is None:
        final_state = torch.empty((bsz, dim, N), device=dev, dtype=torch.float32)
    _need(chunk_states, "chunk_states", (bsz, dim, num_chunks(L), N), torch.float32, dev)
    _need(final_state, "final_state", (bsz, dim, N), torch.float32, dev)
    return chunk_states, final_state


def msel_scan_trap_chunk_carry(u, delta, lam, A, B, delta_bias=None, delta_softplus=True,
                               h0=None, u_prev=None, B_prev=None, return_final_state=True,
                               chunk_states=None, final_state=None):
    """Chunk-carry pass of the exponential-trapezoidal rule.  Returns (chunk_states,
    final_state or None), those msel_scan_trap_fwd gives for the same inputs."""
    if u.dim() != 3 or A.dim() != 2:
        raise ValueError("u must be [batch, dim, seqlen] and A [dim, dstate]")
    bsz, dim, L = u.shape
    N = A.shape[1]
    dev, dt = u.device, u.dtype
    _need(B, "B", (bsz, N, L), dt, dev)
    _need(lam, "lam", (bsz, dim, L), dt, dev)
    _need(u_prev, "u_prev", (bsz, dim), dt, dev)
    _need(B_prev, "B_prev", (bsz, N), dt, dev)
    if lam is None:
        raise ValueError("lam is required")
    a, _ = _args(u, delta, A, B, B, None, None, delta_bias, h0, delta_softplus)
    a.C = None
    chunk_states, final_state = _chunk_carry_out(u, A, chunk_states, final_state,
                                                 return_final_state)
    a.chunk_states, a.final_state = _ptr(chunk_states), _ptr(final_state)
    tr = _lib.TrapArgs()
    tr.lambda_, tr.u_prev, tr.B_prev = _ptr(lam), _ptr(u_prev), _ptr(B_prev)
    _lib.check("msel_scan_trap_chunk_carry",
               _lib.load().msel_scan_trap_chunk_carry(ctypes.byref(a), ctypes.byref(tr),
                                                      _stream(dev)))
    return chunk_states, final_state


def msel_scan_complex_chunk_carry(u, delta, A, B, delta_bias=None, delta_softplus=True, h0=None,
                                  return_final_state=True, chunk_states=None, final_state=None):
    """Chunk-carry pass of the complex-valued scan (A interleaved (Re, Im), dstate even).
    Returns (chunk_states, final_state or None), those msel_scan_complex_fwd gives."""
    if u.dim() != 3 or A.dim() != 2:
        raise ValueError("u must be [batch, dim, seqlen] and A [dim, dstate]")
    bsz, dim, L = u.shape
    N = A.shape[1]
    _need(B, "B", (bsz, N, L), u.dtype, u.device)
    a, _ = _args(u, delta, A, B, B, None, None, delta_bias, h0, delta_softplus)
    a.C = None
    chunk_states, final_state = _chunk_carry_out(u, A, chunk_states, final_state,
                                                 return_final_state)
    a.chunk_states, a.final_state = _ptr(chunk_states), _ptr(final_state)
    _lib.check("msel_scan_complex_chunk_carry",
               _lib.load().msel_scan_complex_chunk_carry(ctypes.byref(a), _stream(u.device)))
    return chunk_states, final_state


def _shape_args(u, A, chunk_states_given):
    bsz, dim, L = u.shape
    a = _lib.ScanArgs()
    a.abi_version = _lib.ABI_VERSION
    a.batch, a.dim, a.dstate, a.seqlen = int(bsz), int(dim), int(A.shape[1]), int(L)
    a.dtype = _dtype_code(u.dtype)
    a.delta_softplus, a.reserved = 1, 0
    # the answer depends only on the shapes; non-null placeholders satisfy the argument checks
    for f in ("u", "delta", "B", "A"):
        setattr(a, f, 256)
    a.chunk_states = 256 if chunk_states_given else None
    return a


def bwd_workspace_bytes(u, A, chunk_states_given=False) -> int:
    """Bytes of workspace msel_scan_bwd needs for this problem (msel_scan_bwd_workspace_bytes)."""
    a = _shape_args(u, A, chunk_states_given)
    return int(_lib.load().msel_scan_bwd_workspace_bytes(ctypes.byref(a)))


def bwd_fused(u, A, chunk_states_given=True) -> bool:
    """Whether msel_scan_bwd takes its fused, deterministic plan for this problem
    (msel_scan_bwd_fused)."""
    a = _shape_args(u, A, chunk_states_given)
    return bool(_lib.load().msel_scan_bwd_fused(ctypes.byref(a)))


def set_bwd_fused(mode: int) -> None:
    """The backward's plan for later calls (msel_set_bwd_fused): 0 by size (the default),
    1 fused wherever it applies, -1 never."""
    _lib.load().msel_set_bwd_fused(int(mode))


def msel_scan_complex_bwd(u, delta, A, B, C, dout, chunk_states=None, D=None, z=None,
                          delta_bias=None, delta_softplus=True, h0=None, want_dA=True,
                          want_dB=True, want_dC=True, want_dD=True, want_ddelta_bias=True,
                          want_dh0=False, workspace=None):
    """Backward of msel_scan_complex_fwd (chunk_states: that forward's, or None: rebuilt by the
    library).  Returns a dict of gradients as msel_scan_bwd does (dA and dh0 interleaved
    (Re, Im))."""
    a, (bsz, dim, N, L) = _args(u, delta, A, B, C, D, z, delta_bias, h0, delta_softplus)
    dev = u.device
    _need(dout, "dout", (bsz, dim, L), u.dtype, dev)
    _need(chunk_states, "chunk_states", (bsz, dim, num_chunks(L), N), torch.float32, dev)
    a.chunk_states = _ptr(chunk_states)
    f32 = dict(device=dev, dtype=torch.float32)
    r = {
        "du": torch.empty_like(u), "ddelta": torch.empty_like(u),
        "dz": torch.empty_like(u) if z is not None else None,
        "dA": torch.empty((dim, N), **f32) if want_dA else None,
        "dB": torch.empty((bsz, N, L), **f32) if want_dB else None,
        "dC": torch.empty((bsz, N, L), **f32) if want_dC else None,
        "dD": torch.empty((dim,), **f32) if want_dD else None,
        "ddelta_bias": torch.empty((dim,), **f32) if want_ddelta_bias else None,
        "dh0": torch.empty((bsz, dim, N), **f32) if want_dh0 else None,
    }
    g = _lib.ScanGrads()
    g.dout = _ptr(dout)
    for k in ("du", "ddelta", "dz", "dA", "dB", "dC", "dD", "ddelta_bias", "dh0"):
        setattr(g, k, _ptr(r[k]))
    lib = _lib.load()
    need = int(lib.msel_scan_bwd_workspace_bytes(ctypes.byref(a)))
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(need, device=dev, dtype=torch.uint8)
    _lib.check("msel_scan_complex_bwd",
               lib.msel_scan_complex_bwd(ctypes.byref(a), ctypes.byref(g), _ptr(workspace),
                                         workspace.numel() * workspace.element_size(),
                                         _stream(dev)))
    return r


def msel_scan_trap_bwd(u, delta, lam, A, B, C, dout, chunk_states=None, D=None, z=None,
                       delta_bias=None, delta_softplus=True, h0=None, u_prev=None, B_prev=None,
                       want_dA=True, want_dB=True, want_dC=True, want_dD=True,
                       want_ddelta_bias=True, want_dh0=False, want_dprev=False,
                       workspace=None):
    """Backward of msel_scan_trap_fwd (chunk_states: that forward's, or None: rebuilt by the
    library).  Returns a dict of gradients as msel_scan_bwd does, plus "dlam" and, with
    want_dprev, "du_prev" [batch, dim] and "dB_prev" [batch, dstate] (fp32)."""
    a, (bsz, dim, N, L) = _args(u, delta, A, B, C, D, z, delta_bias, h0, delta_softplus)
    dev, dt = u.device, u.dtype
    _need(lam, "lam", (bsz, dim, L), dt, dev)
    _need(u_prev, "u_prev", (bsz, dim), dt, dev)
    _need(B_prev, "B_prev", (bsz, N), dt, dev)
    _need(dout, "dout", (bsz, dim, L), dt, dev)
    _need(chunk_states, "chunk_states", (bsz, dim, num_chunks(L), N), torch.float32, dev)
    if lam is None:
        raise ValueError("lam is required")
    a.chunk_states = _ptr(chunk_states)
    f32 = dict(device=dev, dtype=torch.float32)
    r = {
        "du": torch.empty_like(u), "ddelta": torch.empty_like(u), "dlam": torch.empty_like(u),
        "dz": torch.empty_like(u) if z is not None else None,
        "dA": torch.empty((dim, N), **f32) if want_dA else None,
        "dB": torch.empty((bsz, N, L), **f32) if want_dB else None,
        "dC": torch.empty((bsz, N, L), **f32) if want_dC else None,
        "dD": torch.empty((dim,), **f32) if want_dD else None,
        "ddelta_bias": torch.empty((dim,), **f32) if want_ddelta_bias else None,
        "dh0": torch.empty((bsz, dim, N), **f32) if want_dh0 else None,
        "du_prev": torch.empty((bsz, dim), **f32) if want_dprev else None,
        "dB_prev": torch.empty((bsz, N), **f32) if want_dprev else None,
    }
    g = _lib.ScanGrads()
    g.dout = _ptr(dout)
    for k in ("du", "ddelta", "dz", "dA", "dB", "dC", "dD", "ddelta_bias", "dh0"):
        setattr(g, k, _ptr(r[k]))
    tg = _lib.TrapGrads()
    tg.dlambda, tg.du_prev, tg.dB_prev = _ptr(r["dlam"]), _ptr(r["du_prev"]), _ptr(r["dB_prev"])
    tr = _lib.TrapArgs()
    tr.lambda_, tr.u_prev, tr.B_prev = _ptr(lam), _ptr(u_prev), _ptr(B_prev)
    lib = _lib.load()
    need = int(lib.msel_scan_bwd_workspace_bytes(ctypes.byref(a)))
    if need > 0 and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, device=dev, dtype=torch.uint8)
    ws_ptr = _ptr(workspace) if need > 0 else None
    ws_bytes = workspace.numel() * workspace.element_size() if need > 0 else 0
    _lib.check("msel_scan_trap_bwd",
               lib.msel_scan_trap_bwd(ctypes.byref(a), ctypes.byref(tr), ctypes.byref(g),
                                      ctypes.byref(tg), ws_ptr, ws_bytes, _stream(dev)))
    return r


def msel_scan_bwd(u, delta, A, B, C, dout, D=None, z=None, delta_bias=None,
                  delta_softplus=True, h0=None, chunk_states=None, want_dA=True, want_dB=True,
                  want_dC=True, want_dD=True, want_ddelta_bias=True, want_dh0=False,
                  workspace=None, main_events=None):
    """Backward with recomputation.  Returns a dict of gradients (absent ones are None).

    main_events: optional pair of torch.cuda.Event (enable_timing=True) that the library
    records on the current stream right before and after its gradient kernel
    (msel_scan_bwd_profiled); each must have been recorded once already so that it exists."""
    a, (bsz, dim, N, L) = _args(u, delta, A, B, C, D, z, delta_bias, h0, delta_softplus)
    dev, dt = u.device, u.dtype
    _need(dout, "dout", (bsz, dim, L), dt, dev)
    _need(chunk_states, "chunk_states", (bsz, dim, num_chunks(L), N), torch.float32, dev)
    a.chunk_states = _ptr(chunk_states)
    f32 = dict(device=dev, dtype=torch.float32)
    r = {
        "du": torch.empty_like(u), "ddelta": torch.empty_like(u),
        "dz": torch.empty_like(u) if z is not None else None,
        "dA": torch.empty((dim, N), **f32) if want_dA else None,
        "dB": torch.empty((bsz, N, L), **f32) if want_dB else None,
        "dC": torch.empty((bsz, N, L), **f32) if want_dC else None,
        "dD": torch.empty((dim,), **f32) if want_dD else None,
        "ddelta_bias": torch.empty((dim,), **f32) if want_ddelta_bias else None,
        "dh0": torch.empty((bsz, dim, N), **f32) if want_dh0 else None,
    }
    g = _lib.ScanGrads()
    g.dout = _ptr(dout)
    for k in ("du", "ddelta", "dz", "dA", "dB", "dC", "dD", "ddelta_bias", "dh0"):
        setattr(g, k, _ptr(r[k]))
    lib = _lib.load()
    need = int(lib.msel_scan_bwd_workspace_bytes(ctypes.byref(a)))
    if need > 0 and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, device=dev, dtype=torch.uint8)
    ws_ptr = _ptr(workspace) if need > 0 else None
    ws_bytes = workspace.numel() * workspace.element_size() if need > 0 else 0
    if main_events is None:
        _lib.check("msel_scan_bwd", lib.msel_scan_bwd(ctypes.byref(a), ctypes.byref(g), ws_ptr,
                                                      ws_bytes, _stream(dev)))
    else:
        ev = [ctypes.c_void_p(e.cuda_event) for e in main_events]
        if not all(e.value for e in ev):
            raise ValueError("main_events must have been recorded once before use")
        _lib.check("msel_scan_bwd_profiled",
                   lib.msel_scan_bwd_profiled(ctypes.byref(a), ctypes.byref(g), ws_ptr, ws_bytes,
                                              _stream(dev), ev[0], ev[1]))
    return r


def msel_scan_bwd_noalloc(u, delta, A, B, C, dout, D=None, z=None, delta_bias=None,
                          delta_softplus=True, h0=None, chunk_states=None, grads=None,
                          want_dA=True, want_dB=True, want_dC=True, want_dD=True,
                          want_ddelta_bias=True, want_dh0=False):
    """msel_scan_bwd with the library's static scratch as the workspace (for callers that
    cannot allocate; msel_scan_bwd_noalloc).  grads: optional dict of preallocated outputs
    (the keys msel_scan_bwd returns); missing ones are allocated here, on the caller's side of
    the C entry point, which itself allocates nothing.  Returns the dict of gradients."""
    a, (bsz, dim, N, L) = _args(u, delta, A, B, C, D, z, delta_bias, h0, delta_softplus)
    dev, dt = u.device, u.dtype
    _need(dout, "dout", (bsz, dim, L), dt, dev)
    _need(chunk_states, "chunk_states", (bsz, dim, num_chunks(L), N), torch.float32, dev)
    a.chunk_states = _ptr(chunk_states)
    f32 = dict(device=dev, dtype=torch.float32)
    given = dict(grads or {})
    shapes = {"du": (bsz, dim, L), "ddelta": (bsz, dim, L), "dz": (bsz, dim, L),
              "dA": (dim, N), "dB": (bsz, N, L), "dC": (bsz, N, L), "dD": (dim,),
              "ddelta_bias": (dim,), "dh0": (bsz, dim, N)}
    want = {"du": True, "ddelta": True, "dz": z is not None, "dA": want_dA, "dB": want_dB,
            "dC": want_dC, "dD": want_dD, "ddelta_bias": want_ddelta_bias, "dh0": want_dh0}
    r = {}
    for k, shp in shapes.items():
        if not want[k]:
            r[k] = None
            continue
        kdt = dt if k in ("du", "ddelta", "dz") else torch.float32
        if given.get(k) is not None:
            r[k] = _need(given[k], k, shp, kdt, dev)
        else:
            r[k] = torch.empty(shp, device=dev, dtype=kdt)
    g = _lib.ScanGrads()
    g.dout = _ptr(dout)
    for k in shapes:
        setattr(g, k, _ptr(r[k]))
    _lib.check("msel_scan_bwd_noalloc",
               _lib.load().msel_scan_bwd_noalloc(ctypes.byref(a), ctypes.byref(g), _stream(dev)))
    return r


def ring_timeouts() -> int:
    """Waits of the backward gradient kernels' LDS ring that gave up on the current device since
    the last call (0 in a correct run), then clears the count (msel_ring_timeouts).  Waits for
    the device to finish its work."""
    n = ctypes.c_ulonglong(0)
    _lib.check("msel_ring_timeouts", _lib.load().msel_ring_timeouts(ctypes.byref(n)))
    return int(n.value)


def set_ring_spin_limit(polls: int) -> None:
    """Poll limit of those waits for later calls (0: the default); for tests of the timeout
    path (msel_set_ring_spin_limit)."""
    _lib.load().msel_set_ring_spin_limit(int(polls))


BOUNDS_FILES = {1: "scan_fwd.hip", 2: "chunk_carry.hip", 3: "scan_bwd.hip", 4: "conv1d.hip",
                5: "scan_cplx.hip", 6: "scan_cplx_bwd.hip"}


def checked_build() -> bool:
    """Whether the loaded library is the checked build (msel_checked_build)."""
    return bool(_lib.load().msel_checked_build())


def bound_violations():
    """(count, file, line): out-of-range kernel indexes on the current device since the last
    call, and the source file and line of the first (msel_bound_violations; always (0, None, 0)
    in the release build).  Waits for the device to finish its work; clears the records."""
    n, f, ln = ctypes.c_ulonglong(0), ctypes.c_uint32(0), ctypes.c_uint32(0)
    _lib.check("msel_bound_violations",
               _lib.load().msel_bound_violations(ctypes.byref(n), ctypes.byref(f),
                                                 ctypes.byref(ln)))
    return int(n.value), BOUNDS_FILES.get(int(f.value)), int(ln.value)


def bounds_selftest(device=None) -> None:
    """Checked build: one kernel that forms an out-of-range index, which its check must count
    (msel_bounds_selftest).  Raises MselError (MSEL_ERR_UNSUPPORTED) in the release build."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else device
    _lib.check("msel_bounds_selftest", _lib.load().msel_bounds_selftest(_stream(dev)))
