"""ctypes view of include/msel.h and the loader of the in-tree libmsel.so.

There is no fallback of any kind: if the library is not built, every call raises.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmsel.so")
# the same sources built with every kernel index range-checked (msel_checked_build)
LIB_CHECKED_PATH = os.path.join(HERE, "libmsel_checked.so")

ABI_VERSION = 1
MSEL_F32, MSEL_BF16 = 0, 1
STATUS = {0: "MSEL_OK", 1: "MSEL_ERR_NULL", 2: "MSEL_ERR_SHAPE", 3: "MSEL_ERR_DTYPE",
          4: "MSEL_ERR_ALIGN", 5: "MSEL_ERR_UNSUPPORTED", 6: "MSEL_ERR_WORKSPACE",
          7: "MSEL_ERR_ALIAS", 8: "MSEL_ERR_HIP", 9: "MSEL_ERR_VERSION", 10: "MSEL_ERR_TOO_LARGE"}
NOALLOC_SCRATCH_BYTES = 64 << 20  # MSEL_NOALLOC_SCRATCH_BYTES

_P = ctypes.c_void_p


class ScanArgs(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_int32), ("batch", ctypes.c_int32),
                ("dim", ctypes.c_int32), ("dstate", ctypes.c_int32),
                ("seqlen", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("delta_softplus", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("u", _P), ("delta", _P), ("B", _P), ("C", _P), ("z", _P), ("A", _P),
                ("D", _P), ("delta_bias", _P), ("h0", _P), ("out", _P), ("final_state", _P),
                ("chunk_states", _P)]


class ScanGrads(ctypes.Structure):
    _fields_ = [("dout", _P), ("du", _P), ("ddelta", _P), ("dz", _P), ("dA", _P), ("dB", _P),
                ("dC", _P), ("dD", _P), ("ddelta_bias", _P), ("dh0", _P)]


class TrapArgs(ctypes.Structure):
    _fields_ = [("lambda_", _P), ("u_prev", _P), ("B_prev", _P)]


class TrapGrads(ctypes.Structure):
    _fields_ = [("dlambda", _P), ("du_prev", _P), ("dB_prev", _P)]


class ConvArgs(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_int32), ("batch", ctypes.c_int32),
                ("dim", ctypes.c_int32), ("seqlen", ctypes.c_int32), ("width", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("activation", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("x", _P), ("weight", _P), ("bias", _P),
                ("state_in", _P), ("out", _P), ("state_out", _P)]


class ConvGrads(ctypes.Structure):
    _fields_ = [("dout", _P), ("dx", _P), ("dweight", _P), ("dbias", _P), ("dstate_in", _P)]


class MselError(RuntimeError):
    def __init__(self, fn: str, code: int, text: str):
        super().__init__(f"{fn} returned {STATUS.get(code, code)}: {text}")
        self.code = code


_lib = None

EXPORTS = ["msel_abi_version", "msel_chunk_len", "msel_num_chunks", "msel_status_string",
           "msel_validate_fwd", "msel_validate_chunk_carry", "msel_validate_bwd",
           "msel_scan_fwd", "msel_scan_chunk_carry", "msel_scan_bwd_workspace_bytes",
           "msel_scan_bwd", "msel_scan_bwd_profiled", "msel_validate_conv_fwd",
           "msel_validate_conv_bwd", "msel_conv1d_fwd", "msel_conv1d_bwd",
           "msel_validate_trap_fwd", "msel_scan_trap_fwd", "msel_validate_complex_fwd",
           "msel_scan_complex_fwd", "msel_validate_trap_bwd", "msel_scan_trap_bwd",
           "msel_validate_complex_bwd", "msel_scan_complex_bwd", "msel_ring_timeouts",
           "msel_set_ring_spin_limit", "msel_scan_bwd_noalloc", "msel_validate_trap_chunk_carry",
           "msel_scan_trap_chunk_carry", "msel_validate_complex_chunk_carry",
           "msel_scan_complex_chunk_carry", "msel_checked_build", "msel_bound_violations",
           "msel_bounds_selftest", "msel_scan_bwd_fused", "msel_set_bwd_fused"]


def default_path() -> str:
    """The library load() uses: MSEL_LIBRARY=checked selects libmsel_checked.so, any other
    non-empty value is taken as a path; by default the in-tree libmsel.so."""
    v = os.environ.get("MSEL_LIBRARY", "")
    if v == "checked":
        return LIB_CHECKED_PATH
    return v or LIB_PATH


def load(path: str | None = None) -> ctypes.CDLL:
    """Load the library (once; default_path() unless `path` is given).  Raises if it is
    missing: the product has no other path."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or default_path()
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is not built; run `python -m selective_state_space_26_amd.build`"
                           " (or __graft_entry__.build())")
    lib = ctypes.CDLL(p)
    a, g = ctypes.POINTER(ScanArgs), ctypes.POINTER(ScanGrads)
    lib.msel_abi_version.restype = ctypes.c_int32
    lib.msel_abi_version.argtypes = []
    lib.msel_chunk_len.restype = ctypes.c_int32
    lib.msel_chunk_len.argtypes = []
    lib.msel_num_chunks.restype = ctypes.c_int32
    lib.msel_num_chunks.argtypes = [ctypes.c_int32]
    lib.msel_status_string.restype = ctypes.c_char_p
    lib.msel_status_string.argtypes = [ctypes.c_int]
    for fn in ("msel_validate_fwd", "msel_validate_chunk_carry"):
        getattr(lib, fn).restype = ctypes.c_int
        getattr(lib, fn).argtypes = [a]
    lib.msel_validate_bwd.restype = ctypes.c_int
    lib.msel_validate_bwd.argtypes = [a, g, _P, ctypes.c_size_t]
    lib.msel_scan_fwd.restype = ctypes.c_int
    lib.msel_scan_fwd.argtypes = [a, _P]
    lib.msel_scan_chunk_carry.restype = ctypes.c_int
    lib.msel_scan_chunk_carry.argtypes = [a, _P]
    lib.msel_scan_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.msel_scan_bwd_workspace_bytes.argtypes = [a]
    lib.msel_scan_bwd.restype = ctypes.c_int
    lib.msel_scan_bwd.argtypes = [a, g, _P, ctypes.c_size_t, _P]
    lib.msel_scan_bwd_noalloc.restype = ctypes.c_int
    lib.msel_scan_bwd_noalloc.argtypes = [a, g, _P]
    lib.msel_scan_bwd_profiled.restype = ctypes.c_int
    lib.msel_scan_bwd_profiled.argtypes = [a, g, _P, ctypes.c_size_t, _P, _P, _P]
    tap, tgp = ctypes.POINTER(TrapArgs), ctypes.POINTER(TrapGrads)
    lib.msel_validate_trap_bwd.restype = ctypes.c_int
    lib.msel_validate_trap_bwd.argtypes = [a, tap, g, tgp, _P, ctypes.c_size_t]
    lib.msel_scan_trap_bwd.restype = ctypes.c_int
    lib.msel_scan_trap_bwd.argtypes = [a, tap, g, tgp, _P, ctypes.c_size_t, _P]
    lib.msel_validate_complex_bwd.restype = ctypes.c_int
    lib.msel_validate_complex_bwd.argtypes = [a, g, _P, ctypes.c_size_t]
    lib.msel_scan_complex_bwd.restype = ctypes.c_int
    lib.msel_scan_complex_bwd.argtypes = [a, g, _P, ctypes.c_size_t, _P]
    lib.msel_validate_complex_fwd.restype = ctypes.c_int
    lib.msel_validate_complex_fwd.argtypes = [a]
    lib.msel_scan_complex_fwd.restype = ctypes.c_int
    lib.msel_scan_complex_fwd.argtypes = [a, _P]
    ta = ctypes.POINTER(TrapArgs)
    lib.msel_validate_trap_fwd.restype = ctypes.c_int
    lib.msel_validate_trap_fwd.argtypes = [a, ta]
    lib.msel_scan_trap_fwd.restype = ctypes.c_int
    lib.msel_scan_trap_fwd.argtypes = [a, ta, _P]
    lib.msel_validate_trap_chunk_carry.restype = ctypes.c_int
    lib.msel_validate_trap_chunk_carry.argtypes = [a, ta]
    lib.msel_scan_trap_chunk_carry.restype = ctypes.c_int
    lib.msel_scan_trap_chunk_carry.argtypes = [a, ta, _P]
    lib.msel_validate_complex_chunk_carry.restype = ctypes.c_int
    lib.msel_validate_complex_chunk_carry.argtypes = [a]
    lib.msel_scan_complex_chunk_carry.restype = ctypes.c_int
    lib.msel_scan_complex_chunk_carry.argtypes = [a, _P]
    ca, cg = ctypes.POINTER(ConvArgs), ctypes.POINTER(ConvGrads)
    lib.msel_validate_conv_fwd.restype = ctypes.c_int
    lib.msel_validate_conv_fwd.argtypes = [ca]
    lib.msel_validate_conv_bwd.restype = ctypes.c_int
    lib.msel_validate_conv_bwd.argtypes = [ca, cg]
    lib.msel_conv1d_fwd.restype = ctypes.c_int
    lib.msel_conv1d_fwd.argtypes = [ca, _P]
    lib.msel_conv1d_bwd.restype = ctypes.c_int
    lib.msel_conv1d_bwd.argtypes = [ca, cg, _P]
    lib.msel_ring_timeouts.restype = ctypes.c_int
    lib.msel_ring_timeouts.argtypes = [ctypes.POINTER(ctypes.c_ulonglong)]
    lib.msel_set_ring_spin_limit.restype = None
    lib.msel_set_ring_spin_limit.argtypes = [ctypes.c_uint32]
    lib.msel_checked_build.restype = ctypes.c_int
    lib.msel_checked_build.argtypes = []
    lib.msel_bound_violations.restype = ctypes.c_int
    lib.msel_bound_violations.argtypes = [ctypes.POINTER(ctypes.c_ulonglong),
                                          ctypes.POINTER(ctypes.c_uint32),
                                          ctypes.POINTER(ctypes.c_uint32)]
    lib.msel_bounds_selftest.restype = ctypes.c_int
    lib.msel_bounds_selftest.argtypes = [_P]
    lib.msel_scan_bwd_fused.restype = ctypes.c_int32
    lib.msel_scan_bwd_fused.argtypes = [a]
    lib.msel_set_bwd_fused.restype = None
    lib.msel_set_bwd_fused.argtypes = [ctypes.c_int32]
    if lib.msel_abi_version() != ABI_VERSION:
        raise RuntimeError("libmsel.so ABI version mismatch")
    if path is None:
        _lib = lib
    return lib


@contextlib.contextmanager
def using(path: str):
    """Inside the block every call of the binding goes to the library at `path` (for example
    LIB_CHECKED_PATH); the one loaded before is restored after it."""
    global _lib
    prev = _lib
    _lib = load(path)
    try:
        yield _lib
    finally:
        _lib = prev


def check(fn: str, code: int) -> None:
    if code != 0:
        raise MselError(fn, code, load().msel_status_string(code).decode())
