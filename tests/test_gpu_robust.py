"""Failure handling on the GPU, with every kernel ending normally.

* Non-finite inputs propagate and never trap: a NaN in u of one channel and an infinite raw
  step in another poison those channels' outputs from that step on (and the sums over
  channels of their batch row), while every other output is what the clean inputs give:
  bit for bit where one thread writes each element, to 1e-6 of max|.| where fp32 atomics sum
  in a varying order.  The poisoned channel's outputs before the bad step are unchanged too
  (causality).
* The backward's LDS ring waits are bounded: with the poll limit forced down from the host
  (msel_set_ring_spin_limit) waits give up and msel_ring_timeouts counts them; with the default
  limit a run counts none and matches the oracle.
"""
import numpy as np
import pytest

import msel_inputs
import oracle
from helpers import assert_close, host, log, oracle_vals, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import selective_state_space_26_amd as msel  # noqa: E402

BAD_U = (0, 2, 700)      # (batch, channel, step) of the NaN in u
BAD_DELTA = (1, 4, 300)  # (batch, channel, step) of the +inf raw step


def _poison(d):
    p = {k: (None if v is None else v.clone()) for k, v in d.items()}
    p["u"][BAD_U] = float("nan")
    p["delta"][BAD_DELTA] = float("inf")
    return p


def _fwd(d):
    return msel.msel_scan_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"],
                              d["bias"], True, d["h0"], return_chunk_states=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_nonfinite_inputs_propagate(dtype):
    log(f"non-finite inputs {dtype}")
    t = msel_inputs.make(2, 6, 16, 1300, dtype, 401, with_h0=True, with_dout=True)
    clean = to_device(t)
    bad = _poison(clean)
    o1, f1, c1 = _fwd(clean)
    o2, f2, c2 = _fwd(bad)
    g1 = msel.msel_scan_bwd(clean["u"], clean["delta"], clean["A"], clean["B"], clean["C"],
                            clean["dout"], clean["D"], clean["z"], clean["bias"], True,
                            clean["h0"], chunk_states=c1, want_dh0=True)
    g2 = msel.msel_scan_bwd(bad["u"], bad["delta"], bad["A"], bad["B"], bad["C"], bad["dout"],
                            bad["D"], bad["z"], bad["bias"], True, bad["h0"], chunk_states=c2,
                            want_dh0=True)
    # and with the chunk states rebuilt by the backward itself
    g1r = msel.msel_scan_bwd(clean["u"], clean["delta"], clean["A"], clean["B"], clean["C"],
                             clean["dout"], clean["D"], clean["z"], clean["bias"], True,
                             clean["h0"], want_dh0=True)
    g3 = msel.msel_scan_bwd(bad["u"], bad["delta"], bad["A"], bad["B"], bad["C"], bad["dout"],
                            bad["D"], bad["z"], bad["bias"], True, bad["h0"], want_dh0=True)
    torch.cuda.synchronize()
    assert msel.ring_timeouts() == 0
    mask = torch.ones(2, 6, dtype=torch.bool, device=o1.device)  # untouched (batch, channel)
    for b, d_, s in (BAD_U, BAD_DELTA):
        mask[b, d_] = False
        # the poisoned channel: unchanged before the bad step, not finite from it on
        assert torch.equal(o1[b, d_, :s], o2[b, d_, :s])
        assert not torch.isfinite(o2[b, d_, s:].float()).all()
        assert not torch.isfinite(f2[b, d_]).all()
    assert torch.equal(o1[mask], o2[mask])
    assert torch.equal(f1[mask], f2[mask])
    assert torch.equal(c1[mask], c2[mask])
    for ref, g in ((g1, g2), (g1r, g3)):
        for k in ("du", "ddelta", "dz", "dh0"):
            assert torch.equal(ref[k][mask], g[k][mask]), k
        # the adjoint does not involve u, and exp(A * inf) = 0 ends it: dh0 stays finite; the
        # rest carries the NaN or the infinite step
        assert torch.isfinite(g["dh0"]).all()
        for k in ("du", "ddelta", "dz"):
            assert not torch.isfinite(g[k].float()).all(), k
        # dA, dD, dbias sum over batch and time per channel: channels 2 and 4 are poisoned
        keep = torch.tensor([0, 1, 3, 5], device=o1.device)
        for k in ("dA", "dD", "ddelta_bias"):
            assert_close(k, host(g[k][keep]), host(ref[k][keep]), "f32")
            assert not torch.isfinite(g[k]).all(), k
        # dB, dC sum over the channels of a batch row: both rows hold a poisoned channel
        for k in ("dB", "dC"):
            assert not torch.isfinite(g[k][0]).all() and not torch.isfinite(g[k][1]).all(), k


def _bwd_case(seed=402):
    t = msel_inputs.make(1, 96, 16, 1024, "f32", seed, with_h0=True, with_dout=True)
    return t, to_device(t)


def test_ring_wait_timeouts_are_counted():
    """A poll limit of 1 makes waits give up (counted, the kernels end); the default limit
    counts none, and the result matches the oracle."""
    log("ring wait timeouts")
    t, d = _bwd_case()
    msel.ring_timeouts()  # clear whatever earlier calls left
    args = (d["u"], d["delta"], d["A"], d["B"], d["C"], d["dout"], d["D"], d["z"], d["bias"],
            True, d["h0"])
    msel.set_ring_spin_limit(1)
    try:
        msel.msel_scan_bwd(*args)
        torch.cuda.synchronize()
        forced = msel.ring_timeouts()
    finally:
        msel.set_ring_spin_limit(0)
    assert forced > 0
    assert msel.ring_timeouts() == 0  # reading cleared the count
    g = msel.msel_scan_bwd(*args, want_dh0=True)
    torch.cuda.synchronize()
    assert msel.ring_timeouts() == 0
    v = oracle_vals(t)
    r = oracle.bwd(v["u"], v["delta"], v["A"], v["B"], v["C"], v["dout"], v["D"], v["z"],
                   v["bias"], v["h0"])
    for k in ("du", "ddelta", "dz", "dA", "dB", "dC", "dD", "ddelta_bias", "dh0"):
        assert_close(k, host(g[k]), r[k], "f32")


def test_complex_ring_wait_timeouts_are_counted():
    log("complex ring wait timeouts")
    t = msel_inputs.make(1, 96, 16, 1024, "f32", 403, with_h0=True, with_dout=True,
                         complex_A=True)
    d = to_device(t)
    msel.ring_timeouts()
    _, _, cs = msel.msel_scan_complex_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"],
                                          d["z"], d["bias"], True, d["h0"],
                                          return_chunk_states=True)
    args = (d["u"], d["delta"], d["A"], d["B"], d["C"], d["dout"], cs, d["D"], d["z"],
            d["bias"], True, d["h0"])
    msel.set_ring_spin_limit(1)
    try:
        msel.msel_scan_complex_bwd(*args)
        torch.cuda.synchronize()
        forced = msel.ring_timeouts()
    finally:
        msel.set_ring_spin_limit(0)
    assert forced > 0
    g = msel.msel_scan_complex_bwd(*args)
    torch.cuda.synchronize()
    assert msel.ring_timeouts() == 0
    from oracle import cplx as ocplx
    v = oracle_vals(t)
    r = ocplx.bwd(v["u"], v["delta"], v["A"], v["B"], v["C"], v["dout"], v["D"], v["z"],
                  v["bias"], v["h0"])
    for k in ("du", "ddelta", "dz", "dA", "dB", "dC", "dD", "ddelta_bias"):
        assert_close(k, host(g[k]), r[k], "f32")
    assert np.isfinite(host(g["du"])).all()
