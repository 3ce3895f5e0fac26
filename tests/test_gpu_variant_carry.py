"""GPU parity of the chunk-carry passes of the two Mamba-3 variants (page 4, Appendix D, Speed:
the scan continues chunk by chunk from the intermediate state; page 5, the Mamba-3 post: the
exponential-trapezoidal rule and the complex-valued state), and of their backwards with the
chunk states rebuilt by the library instead of given by the forward.

* msel_scan_trap_chunk_carry and msel_scan_complex_chunk_carry against the chunk states and
  final state of their fp64 oracles (oracle/trap.py, oracle/cplx.py) over shapes with ragged
  chunks, both dtypes, the vector and scalar load paths, with and without h0, softplus, bias
  and the trapezoidal rule's previous-step inputs, and against their own forwards' chunk
  states;
* the reductions: lambda = 1 is the plain rule, and A_im = 0 the real scan with
  A[d, 2j+1] = A[d, 2j]: both must equal msel_scan_chunk_carry bit for bit;
* msel_scan_trap_bwd and msel_scan_complex_bwd with chunk_states=None against their oracles.

The bar: max|gpu - oracle| <= tol * max|oracle| per tensor (1e-4 fp32, 1e-2 bf16 inputs).
"""
import numpy as np
import pytest

import msel_inputs
from helpers import assert_close, host, log, to_device
from oracle import cplx as ocplx
from oracle import trap as otrap

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import selective_state_space_26_amd as msel  # noqa: E402

T = msel.chunk_len()

CASES = [
    # batch, dim, dstate, seqlen, dtype, softplus, bias, h0, previous-step inputs
    (2, 5, 16, 2500, "f32", True, True, True, True),     # 5 chunks, ragged tail
    (2, 5, 16, 2500, "bf16", True, True, True, False),   # scalar path (2500 % 8)
    (2, 3, 16, 4096, "bf16", True, True, False, True),   # whole chunks, vector path
    (3, 7, 6, 1000, "f32", False, False, True, True),    # no softplus, dstate 6
    (1, 1, 2, 777, "bf16", True, True, True, True),      # one channel, one complex state
    (1, 3, 16, 1, "f32", True, True, True, True),        # one step
    (2, 9, 10, 520, "f32", True, True, False, False),    # one chunk + 8 steps, odd channels
]


def _inputs(bsz, dim, N, L, dtype, sp, with_bias, with_h0, with_prev, seed=611,
            complex_A=False):
    t = msel_inputs.make(bsz, dim, N, L, dtype, seed, with_bias=with_bias, with_h0=with_h0,
                         with_lam=not complex_A, with_prev=with_prev and not complex_A,
                         with_dout=True, complex_A=complex_A)
    if not sp:
        v = np.abs(t.values("delta")) * np.float32(0.2)
        t["delta"] = msel_inputs.f32_to_bf16_bits(v) if dtype == "bf16" else v
    return t


def _vals(t):
    return {k: (None if t.get(k) is None else t.values(k)) for k in t}


def _ids(c):
    return "x".join(map(str, c[:5])) + ("" if c[5] else "-nosp") + ("-prev" if c[8] else "")


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_trap_chunk_carry_matches_oracle(case):
    bsz, dim, N, L, dtype, sp, with_bias, with_h0, with_prev = case
    log(f"trap chunk carry {case}")
    t = _inputs(*case)
    d = to_device(t)
    cs, fin = msel.msel_scan_trap_chunk_carry(d["u"], d["delta"], d["lam"], d["A"], d["B"],
                                              d["bias"], sp, d["h0"], d.get("u_prev"),
                                              d.get("B_prev"))
    _, ffin, fcs = msel.msel_scan_trap_fwd(d["u"], d["delta"], d["lam"], d["A"], d["B"], d["C"],
                                           d["D"], d["z"], d["bias"], sp, d["h0"],
                                           d.get("u_prev"), d.get("B_prev"),
                                           return_chunk_states=True)
    torch.cuda.synchronize()
    v = _vals(t)
    _, rf, rcs = otrap.fwd(v["u"], v["delta"], v["lam"], v["A"], v["B"], v["C"], v["D"],
                           v["z"], v["bias"], v["h0"], v.get("u_prev"), v.get("B_prev"),
                           softplus=sp, chunk_len=T)
    assert_close("chunk_states", host(cs), rcs, dtype)
    assert_close("final_state", host(fin), rf, dtype)
    assert_close("forward's chunk_states", host(cs), host(fcs), dtype)
    assert_close("forward's final_state", host(fin), host(ffin), dtype)


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_complex_chunk_carry_matches_oracle(case):
    bsz, dim, N, L, dtype, sp, with_bias, with_h0, _ = case
    log(f"complex chunk carry {case}")
    t = _inputs(*case, complex_A=True)
    d = to_device(t)
    cs, fin = msel.msel_scan_complex_chunk_carry(d["u"], d["delta"], d["A"], d["B"], d["bias"],
                                                 sp, d["h0"])
    _, ffin, fcs = msel.msel_scan_complex_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"],
                                              d["D"], d["z"], d["bias"], sp, d["h0"],
                                              return_chunk_states=True)
    torch.cuda.synchronize()
    v = _vals(t)
    _, rf, rcs = ocplx.fwd(v["u"], v["delta"], v["A"], v["B"], v["C"], v["D"], v["z"],
                           v["bias"], v["h0"], softplus=sp, chunk_len=T)
    assert_close("chunk_states", host(cs), rcs, dtype)
    assert_close("final_state", host(fin), rf, dtype)
    assert_close("forward's chunk_states", host(cs), host(fcs), dtype)
    assert_close("forward's final_state", host(fin), host(ffin), dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_variant_chunk_carry_reductions_are_exact(dtype):
    """lambda = 1 removes the trapezoidal terms exactly (c = (Delta - Delta) u = 0), and
    A_im = 0 the rotation (cos 0 = 1, sin 0 = 0): both passes then compute the plain pass's
    arithmetic in the same order."""
    log(f"variant chunk carry reductions {dtype}")
    t = msel_inputs.make(2, 5, 16, 2100, dtype, 612, with_h0=True)
    d = to_device(t)
    ref_cs, ref_fin = msel.msel_scan_chunk_carry(d["u"], d["delta"], d["A"], d["B"], d["bias"],
                                                 True, d["h0"])
    ones = torch.ones_like(d["u"])
    cs1, fin1 = msel.msel_scan_trap_chunk_carry(d["u"], d["delta"], ones, d["A"], d["B"],
                                                d["bias"], True, d["h0"])
    Ac = d["A"].clone()
    Ac[:, 1::2] = 0.0       # A_im = 0 ...
    Ar = d["A"].clone()
    Ar[:, 1::2] = Ar[:, 0::2]  # ... is the real scan with both states at A_re
    cs2, fin2 = msel.msel_scan_complex_chunk_carry(d["u"], d["delta"], Ac, d["B"], d["bias"],
                                                   True, d["h0"])
    ref2_cs, ref2_fin = msel.msel_scan_chunk_carry(d["u"], d["delta"], Ar, d["B"], d["bias"],
                                                   True, d["h0"])
    torch.cuda.synchronize()
    assert torch.equal(cs1, ref_cs) and torch.equal(fin1, ref_fin)
    assert torch.equal(cs2, ref2_cs) and torch.equal(fin2, ref2_fin)


BWD_CASES = [CASES[0], CASES[1], CASES[3], CASES[6]]


@pytest.mark.parametrize("case", BWD_CASES, ids=_ids)
def test_trap_bwd_with_rebuilt_states(case):
    bsz, dim, N, L, dtype, sp, with_bias, with_h0, with_prev = case
    log(f"trap bwd rebuilt states {case}")
    t = _inputs(*case)
    d = to_device(t)
    g = msel.msel_scan_trap_bwd(d["u"], d["delta"], d["lam"], d["A"], d["B"], d["C"], d["dout"],
                                None, d["D"], d["z"], d["bias"], sp, d["h0"], d.get("u_prev"),
                                d.get("B_prev"), want_dh0=True, want_dprev=True)
    torch.cuda.synchronize()
    v = _vals(t)
    r = otrap.bwd(v["u"], v["delta"], v["lam"], v["A"], v["B"], v["C"], v["dout"], v["D"],
                  v["z"], v["bias"], v["h0"], v.get("u_prev"), v.get("B_prev"), softplus=sp)
    for k in ("du", "ddelta", "dlam", "dz", "dA", "dB", "dC", "dD", "ddelta_bias", "dh0",
              "du_prev", "dB_prev"):
        assert_close(k, host(g[k]), r[k], dtype)


@pytest.mark.parametrize("case", BWD_CASES, ids=_ids)
def test_complex_bwd_with_rebuilt_states(case):
    bsz, dim, N, L, dtype, sp, with_bias, with_h0, _ = case
    log(f"complex bwd rebuilt states {case}")
    t = _inputs(*case, complex_A=True)
    d = to_device(t)
    g = msel.msel_scan_complex_bwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["dout"], None,
                                   d["D"], d["z"], d["bias"], sp, d["h0"], want_dh0=True)
    torch.cuda.synchronize()
    v = _vals(t)
    r = ocplx.bwd(v["u"], v["delta"], v["A"], v["B"], v["C"], v["dout"], v["D"], v["z"],
                  v["bias"], v["h0"], softplus=sp)
    for k in ("du", "ddelta", "dz", "dA", "dB", "dC", "dD", "ddelta_bias", "dh0"):
        assert_close(k, host(g[k]), r[k], dtype)
