"""Builds libmsel.so in-tree with hipcc for gfx950, and its checked twin libmsel_checked.so.

    python -m selective_state_space_26_amd.build        # from the repository root

Every HIP source is compiled with the packed-FP32 instructions disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``) and hardware fp32 atomics enabled.
The checked library is the same sources with ``-DMSEL_CHECKED``: every index a kernel forms
is compared with its buffer's extent (see msel_checked_build in include/msel.h).
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmsel.so")
LIB_CHECKED = os.path.join(HERE, "libmsel_checked.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["msel_api.cpp", "scan_fwd.hip", "chunk_carry.hip", "scan_bwd.hip", "conv1d.hip",
           "scan_cplx.hip", "scan_cplx_bwd.hip"]

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics", "-Wall", "-Wno-unused-function",
          "-I", os.path.join(os.path.dirname(HERE), "include")]


def _compile(src: str, checked: bool) -> str:
    out_dir = os.path.join(BUILD, "checked") if checked else BUILD
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    flags = COMMON + (["-DMSEL_CHECKED"] if checked else [])
    cmd = [HIPCC, *flags, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def _link(objs: list, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, lib)


def build(verbose: bool = True, checked: bool = True) -> str:
    """Builds libmsel.so and, unless checked is False, libmsel_checked.so; returns the first."""
    os.makedirs(os.path.join(BUILD, "checked"), exist_ok=True)
    jobs = [(src, False) for src in SOURCES] + ([(src, True) for src in SOURCES] if checked else [])
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    _link(objs[:len(SOURCES)], LIB)
    if verbose:
        print("built", LIB)
    if checked:
        _link(objs[len(SOURCES):], LIB_CHECKED)
        if verbose:
            print("built", LIB_CHECKED)
    return LIB


if __name__ == "__main__":
    build()
