"""The seeded random cases of the GPU parity tests (tests/test_gpu_random_shapes.py, and the
checked build's tests/test_gpu_checked.py): batch 1-3, dim 1-13 (most not a multiple of a
workgroup's channels), every dstate the variant allows, lengths from one step to a few chunks
with ragged tails, both dtypes, and random optional inputs.  Each case runs its variant's
forward, chunk-carry pass and backward (the convolution: forward and backward) through the
binding and checks them against the fp64 oracles: max|gpu - oracle| <= tol * max|oracle|
(1e-4 fp32, 1e-2 bf16 inputs; the convolution's fp32 sums at 1e-4).  Every other case's
backward runs with chunk states that the library rebuilds.  Imported by GPU tests only."""
import numpy as np
import torch

import msel_inputs
import oracle
import selective_state_space_26_amd as msel
from helpers import assert_close, host, log, to_device
from oracle import conv as oconv
from oracle import cplx as ocplx
from oracle import trap as otrap

LENGTHS = [1, 2, 7, 63, 64, 65, 511, 512, 513, 1000, 1024, 1025, 1500]


def _draw(kind, k):
    rng = np.random.default_rng([2026, k, {"scan": 0, "trap": 1, "cplx": 2, "conv": 3}[kind]])
    bsz = int(rng.integers(1, 4))
    dim = int(rng.integers(1, 14))
    N = 2 * int(rng.integers(1, 9)) if kind == "cplx" else int(rng.integers(1, 17))
    L = int(rng.choice(LENGTHS)) if rng.random() < 0.6 else int(rng.integers(1, 1501))
    dtype = "bf16" if rng.random() < 0.5 else "f32"
    flags = [bool(x) for x in rng.random(5) < 0.6]  # z, softplus, D/bias, h0, extra
    return (bsz, dim, N, L, dtype, *flags)


CASES = [("scan", k) for k in range(10)] + [("trap", k) for k in range(8)] + \
        [("cplx", k) for k in range(8)] + [("conv", k) for k in range(8)]


def ids(c):
    return f"{c[0]}-" + "x".join(map(str, _draw(*c)[:5]))


def _scan_inputs(t, dtype, sp):
    if not sp:  # without the softplus keep Delta = delta + bias positive and small
        v = np.abs(t.values("delta")) * np.float32(0.2)
        t["delta"] = msel_inputs.f32_to_bf16_bits(v) if dtype == "bf16" else v
        if t.get("bias") is not None:
            t["bias"] = (np.abs(t["bias"]) * np.float32(0.01)).astype(np.float32)
    return t


def _dev(t, dtype):
    d = to_device(t)
    act = torch.bfloat16 if dtype == "bf16" else torch.float32
    for k in ("lam", "u_prev", "B_prev"):
        if d.get(k) is not None and d[k].dtype != act:
            d[k] = d[k].to(act)
    return d


def _vals(t):
    return {k: (None if t.get(k) is None else t.values(k)) for k in t}


def _check_states(cs, ccs, cfin, rcs, rf, dtype):
    """The forward's chunk states and the chunk-carry pass's against the oracle's."""
    assert_close("chunk_states", host(cs), rcs, dtype)
    assert_close("chunk_carry chunk_states", host(ccs), rcs, dtype)
    assert_close("chunk_carry final_state", host(cfin), rf, dtype)


def run_case(case):
    """Runs one drawn case through the library and its oracle and asserts parity."""
    kind, k = case
    bsz, dim, N, L, dtype, with_z, sp, with_db, with_h0, extra = _draw(kind, k)
    log(f"random {kind} {k}: {(bsz, dim, N, L, dtype, with_z, sp, with_db, with_h0, extra)}")
    seed = 500 + k
    if kind == "conv":
        W = 1 + N % 4
        with_state = with_h0 and W > 1
        t = msel_inputs.make_conv(bsz, dim, L, W, dtype, seed, with_bias=with_db,
                                  with_state=with_state, with_dout=True)
        d = _dev(t, dtype)
        out, st = msel.msel_conv1d_fwd(d["x"], d["weight"], d["bias"], d["state"], with_z,
                                       return_state=W > 1)
        g = msel.msel_conv1d_bwd(d["x"], d["weight"], d["dout"], d["bias"], d["state"], with_z,
                                 want_dstate=W > 1)
        torch.cuda.synchronize()
        v = {n: t.values(n) for n in ("x", "weight", "bias", "state", "dout")}
        ro, rs = oconv.fwd(v["x"], v["weight"], v["bias"], v["state"], with_z)
        r = oconv.bwd(v["x"], v["weight"], v["dout"], v["bias"], v["state"], with_z)
        assert_close("out", host(out), ro, dtype)
        assert_close("dx", host(g["dx"]), r["dx"], dtype)
        for n in ("dweight", "dbias"):
            assert_close(n, host(g[n]), r[n], "f32")
        if W > 1:
            assert_close("state_out", host(st), rs, dtype)
            assert_close("dstate", host(g["dstate"]), r["dstate"], "f32")
        return

    common = dict(with_z=with_z, with_D=with_db, with_bias=with_db, with_h0=with_h0,
                  with_dout=True)
    if kind == "scan":
        t = _scan_inputs(msel_inputs.make(bsz, dim, N, L, dtype, seed, **common), dtype, sp)
        d = _dev(t, dtype)
        a = (d["u"], d["delta"], d["A"], d["B"], d["C"])
        o = (d["D"], d["z"], d["bias"], sp, d["h0"])
        out, fin, cs = msel.msel_scan_fwd(*a, *o, return_chunk_states=True)
        ccs, cfin = msel.msel_scan_chunk_carry(d["u"], d["delta"], d["A"], d["B"], d["bias"],
                                               sp, d["h0"])
        g = msel.msel_scan_bwd(*a, d["dout"], *o, chunk_states=cs if extra else None,
                               want_dh0=with_h0)
        torch.cuda.synchronize()
        v = _vals(t)
        ro, rf, rcs = oracle.fwd(v["u"], v["delta"], v["A"], v["B"], v["C"], v["D"], v["z"],
                                 v["bias"], v["h0"], softplus=sp, chunk_len=msel.chunk_len())
        r = oracle.bwd(v["u"], v["delta"], v["A"], v["B"], v["C"], v["dout"], v["D"], v["z"],
                       v["bias"], v["h0"], softplus=sp)
        _check_states(cs, ccs, cfin, rcs, rf, dtype)
        names = ["du", "ddelta", "dA", "dB", "dC", "dD", "ddelta_bias"]
    elif kind == "trap":
        t = _scan_inputs(msel_inputs.make(bsz, dim, N, L, dtype, seed, with_lam=True,
                                          with_prev=extra, **common), dtype, sp)
        d = _dev(t, dtype)
        a = (d["u"], d["delta"], d["lam"], d["A"], d["B"], d["C"])
        o = (d["D"], d["z"], d["bias"], sp, d["h0"], d.get("u_prev"), d.get("B_prev"))
        out, fin, cs = msel.msel_scan_trap_fwd(*a, *o, return_chunk_states=True)
        ccs, cfin = msel.msel_scan_trap_chunk_carry(d["u"], d["delta"], d["lam"], d["A"], d["B"],
                                                    d["bias"], sp, d["h0"], d.get("u_prev"),
                                                    d.get("B_prev"))
        g = msel.msel_scan_trap_bwd(*a, d["dout"], cs if k % 2 else None, *o, want_dh0=with_h0,
                                    want_dprev=extra)
        torch.cuda.synchronize()
        v = _vals(t)
        ro, rf, rcs = otrap.fwd(v["u"], v["delta"], v["lam"], v["A"], v["B"], v["C"], v["D"],
                              v["z"], v["bias"], v["h0"], v.get("u_prev"), v.get("B_prev"),
                              softplus=sp, chunk_len=msel.chunk_len())
        r = otrap.bwd(v["u"], v["delta"], v["lam"], v["A"], v["B"], v["C"], v["dout"], v["D"],
                      v["z"], v["bias"], v["h0"], v.get("u_prev"), v.get("B_prev"), softplus=sp)
        names = ["du", "ddelta", "dlam", "dA", "dB", "dC", "dD", "ddelta_bias"]
        _check_states(cs, ccs, cfin, rcs, rf, dtype)
        if extra:
            names += ["du_prev", "dB_prev"]
    else:
        t = _scan_inputs(msel_inputs.make(bsz, dim, N, L, dtype, seed, complex_A=True,
                                          **common), dtype, sp)
        d = _dev(t, dtype)
        a = (d["u"], d["delta"], d["A"], d["B"], d["C"])
        o = (d["D"], d["z"], d["bias"], sp, d["h0"])
        out, fin, cs = msel.msel_scan_complex_fwd(*a, *o, return_chunk_states=True)
        ccs, cfin = msel.msel_scan_complex_chunk_carry(d["u"], d["delta"], d["A"], d["B"],
                                                       d["bias"], sp, d["h0"])
        g = msel.msel_scan_complex_bwd(*a, d["dout"], cs if k % 2 else None, *o,
                                       want_dh0=with_h0)
        torch.cuda.synchronize()
        v = _vals(t)
        ro, rf, rcs = ocplx.fwd(v["u"], v["delta"], v["A"], v["B"], v["C"], v["D"], v["z"],
                              v["bias"], v["h0"], softplus=sp, chunk_len=msel.chunk_len())
        r = ocplx.bwd(v["u"], v["delta"], v["A"], v["B"], v["C"], v["dout"], v["D"], v["z"],
                      v["bias"], v["h0"], softplus=sp)
        names = ["du", "ddelta", "dA", "dB", "dC", "dD", "ddelta_bias"]
        _check_states(cs, ccs, cfin, rcs, rf, dtype)
    assert_close("out", host(out), ro, dtype)
    assert_close("final_state", host(fin), rf, dtype)
    if with_h0:
        names.append("dh0")
    if with_z:
        names.append("dz")
    for n in names:
        assert_close(n, host(g[n]), r[n], dtype)
