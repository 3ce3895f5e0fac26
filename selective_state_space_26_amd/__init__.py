"""MI355X (gfx950) selective SSM scan: a C-ABI HIP library (libmsel.so) and its thin binding.

    from selective_state_space_26_amd import msel_scan_fwd, msel_scan_bwd, msel_scan_chunk_carry
    from selective_state_space_26_amd import msel_conv1d_fwd, msel_conv1d_bwd

The kernels live in ``csrc/``; ``build.py`` compiles them in-tree.  Importing this package does
not load the library; the first call does, and raises if it is not built.
"""
from .conv import msel_conv1d_bwd, msel_conv1d_fwd  # noqa: F401
from .scan import (bwd_workspace_bytes, chunk_len, msel_scan_bwd,  # noqa: F401
                   msel_scan_chunk_carry, msel_scan_complex_bwd, msel_scan_complex_fwd, msel_scan_fwd,
                   msel_scan_bwd_noalloc, msel_scan_complex_chunk_carry,
                   msel_scan_trap_bwd, msel_scan_trap_chunk_carry, msel_scan_trap_fwd,
                   num_chunks, ring_timeouts, set_ring_spin_limit, checked_build,
                   bound_violations, bounds_selftest, bwd_fused, set_bwd_fused)

__all__ = ["msel_scan_fwd", "msel_scan_bwd", "msel_scan_chunk_carry", "chunk_len", "num_chunks",
           "bwd_workspace_bytes", "msel_conv1d_fwd", "msel_conv1d_bwd", "msel_scan_trap_fwd",
           "msel_scan_complex_fwd", "msel_scan_trap_bwd", "msel_scan_complex_bwd",
           "ring_timeouts", "set_ring_spin_limit", "msel_scan_bwd_noalloc",
           "msel_scan_trap_chunk_carry", "msel_scan_complex_chunk_carry", "checked_build",
           "bound_violations", "bounds_selftest", "bwd_fused", "set_bwd_fused"]
