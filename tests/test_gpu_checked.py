"""The checked build (libmsel_checked.so: every index a kernel forms into a global buffer or an
LDS array compared with the extent of what it indexes) on the GPU:

* its own check fires: the self-test kernel's out-of-range index is counted once, in its file;
* every seeded random case of the parity tests (every variant's forward, chunk-carry pass and
  backward, the convolution) meets no out-of-range index and still matches the fp64 oracles at
  the parity bar;
* the decode kernels (seqlen 1) of every variant meet none, and their outputs equal the release
  build's bit for bit;
* at the full sizes of the 2048- and 65536-step workloads, in the benchmark's launch
  configuration, the forward, the chunk-carry pass and the backward (chunk states given and
  rebuilt, and the allocation-free backward) meet no out-of-range index, and their outputs
  equal the release build's bit for bit (the atomic sums dA, dB, dC, dD, dbias to the parity
  bar: their order of addition varies between runs).
"""
import pytest

import msel_inputs
from helpers import assert_close, host, log, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import selective_state_space_26_amd as msel  # noqa: E402
from selective_state_space_26_amd import _lib  # noqa: E402

from random_cases import CASES, ids, run_case  # noqa: E402


@pytest.fixture
def checked():
    with _lib.using(_lib.LIB_CHECKED_PATH):
        assert msel.checked_build()
        msel.bound_violations()  # start from empty records
        yield
        count, f, line = msel.bound_violations()
        assert count == 0, f"{count} out-of-range indexes, the first at {f}:{line}"
        assert msel.ring_timeouts() == 0


def test_selftest_is_counted():
    with _lib.using(_lib.LIB_CHECKED_PATH):
        msel.bound_violations()
        msel.bounds_selftest()
        count, f, line = msel.bound_violations()
        assert (count, f) == (1, "scan_fwd.hip") and line > 0
        assert msel.bound_violations() == (0, None, 0)  # the read cleared it
    assert not msel.checked_build()
    assert msel.bound_violations() == (0, None, 0)  # the release build reports none


@pytest.mark.parametrize("case", CASES, ids=ids)
def test_random_case_in_range(checked, case):
    run_case(case)


def _step(d, given):
    a = (d["u"], d["delta"], d["A"], d["B"], d["C"])
    o = (d["D"], d["z"], d["bias"], True)
    out, fin, cs = msel.msel_scan_fwd(*a, *o, return_chunk_states=True)
    ccs, cfin = msel.msel_scan_chunk_carry(d["u"], d["delta"], d["A"], d["B"], d["bias"], True)
    g = msel.msel_scan_bwd(*a, d["dout"], *o, chunk_states=cs if given else None)
    r = {"out": out, "final_state": fin, "chunk_states": cs, "cc_states": ccs,
         "cc_final": cfin}
    r.update({k: v for k, v in g.items() if v is not None})
    if given:
        gn = msel.msel_scan_bwd_noalloc(*a, d["dout"], *o, chunk_states=cs)
        r.update({"noalloc_" + k: v for k, v in gn.items() if v is not None})
    torch.cuda.synchronize()
    return r


ATOMIC = ("dA", "dB", "dC", "dD", "ddelta_bias")


@pytest.mark.parametrize("wid,given", [(2, True), (2, False), (3, True)])
def test_full_workload_in_range_and_equal_to_release(wid, given):
    w = msel_inputs.WORKLOADS[wid]
    log(f"checked build, workload {wid} {w}, chunk states {'given' if given else 'rebuilt'}")
    d = to_device(msel_inputs.make_workload(w, with_dout=True))
    ref = _step(d, given)
    with _lib.using(_lib.LIB_CHECKED_PATH):
        msel.bound_violations()
        got = _step(d, given)
        count, f, line = msel.bound_violations()
        assert count == 0, f"{count} out-of-range indexes, the first at {f}:{line}"
        assert msel.ring_timeouts() == 0
    assert set(got) == set(ref)
    for k, v in ref.items():
        if k.replace("noalloc_", "") in ATOMIC:
            assert_close(k, host(got[k]), host(v), w.dtype)
        else:
            assert torch.equal(got[k], v), k


def _decode(kind, d):
    """One recurrent step (seqlen 1) of `kind` from a carried state."""
    if kind == "conv":
        out, st = msel.msel_conv1d_fwd(d["x"], d["weight"], d["bias"], d["state"], True,
                                       return_state=True)
        torch.cuda.synchronize()
        return {"out": out, "state": st}
    if kind == "trap":
        out, fin, _ = msel.msel_scan_trap_fwd(d["u"], d["delta"], d["lam"], d["A"], d["B"],
                                              d["C"], d["D"], d["z"], d["bias"], True, d["h0"],
                                              d["u_prev"], d["B_prev"])
    else:
        f = msel.msel_scan_complex_fwd if kind == "cplx" else msel.msel_scan_fwd
        out, fin, _ = f(d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"], d["bias"],
                        True, d["h0"])
    torch.cuda.synchronize()
    return {"out": out, "final_state": fin}


@pytest.mark.parametrize("kind", ["scan", "trap", "cplx", "conv"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_step_in_range_and_equal_to_release(kind, dtype):
    """The decode kernels (seqlen 1), which the random cases reach only for the plain scan."""
    log(f"checked build, decode step {kind} {dtype}")
    bsz, dim, N = 3, 37, 16
    if kind == "conv":
        t = msel_inputs.make_conv(bsz, dim, 1, 4, dtype, 41, with_state=True)
    else:
        t = msel_inputs.make(bsz, dim, N, 1, dtype, 42, with_h0=True, with_lam=kind == "trap",
                             with_prev=kind == "trap", complex_A=kind == "cplx")
    d = to_device(t)
    if kind == "trap":  # the step before the first, in the activation dtype
        act = torch.bfloat16 if dtype == "bf16" else torch.float32
        for k in ("lam", "u_prev", "B_prev"):
            d[k] = d[k].to(act)
    ref = _decode(kind, d)
    with _lib.using(_lib.LIB_CHECKED_PATH):
        msel.bound_violations()
        got = _decode(kind, d)
        count, f, line = msel.bound_violations()
        assert count == 0, f"{count} out-of-range indexes, the first at {f}:{line}"
    for k, v in ref.items():
        assert torch.equal(got[k], v), k
