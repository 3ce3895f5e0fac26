"""Every forward + backward pair only enqueues kernels (zero-fills included, no allocation
and no host synchronisation inside the library), so a whole training step of each variant can
be captured in a HIP graph.  Three replays, each after the outputs were overwritten with NaN
and followed by host work and a synchronisation, must match the eager step: bit for bit where
each output element is written by one thread, and to fp32 rounding where fp32 atomics sum
over channels or time (their order varies from run to run)."""
import numpy as np
import pytest

import msel_inputs
from helpers import host, log, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import selective_state_space_26_amd as msel  # noqa: E402

SHAPE = (2, 6, 16, 1100)  # three chunks, ragged tail


def _scan():
    t = msel_inputs.make(*SHAPE, "bf16", 31, with_dout=True)
    d = to_device(t)
    a = (d["u"], d["delta"], d["A"], d["B"], d["C"])
    o = (d["D"], d["z"], d["bias"], True)

    def step():
        out, fin, cs = msel.msel_scan_fwd(*a, *o, return_chunk_states=True)
        g = msel.msel_scan_bwd(*a, d["dout"], *o, chunk_states=cs)
        return dict(out=out, fin=fin, **g)
    return step, ("out", "fin", "du", "ddelta", "dz"), ("dA", "dB", "dC", "dD", "ddelta_bias")


def _trap():
    t = msel_inputs.make(*SHAPE, "bf16", 32, with_dout=True, with_lam=True, with_prev=True,
                         with_h0=True)
    d = to_device(t)
    a = (d["u"], d["delta"], d["lam"], d["A"], d["B"], d["C"])
    o = (d["D"], d["z"], d["bias"], True, d["h0"], d["u_prev"], d["B_prev"])

    def step():
        out, fin, cs = msel.msel_scan_trap_fwd(*a, *o, return_chunk_states=True)
        g = msel.msel_scan_trap_bwd(*a, d["dout"], cs, *o, want_dh0=True, want_dprev=True)
        return dict(out=out, fin=fin, **g)
    return (step, ("out", "fin", "du", "ddelta", "dz", "dlam", "dh0", "du_prev"),
            ("dA", "dB", "dC", "dD", "ddelta_bias", "dB_prev"))


def _complex():
    t = msel_inputs.make(*SHAPE, "bf16", 33, with_dout=True, complex_A=True)
    d = to_device(t)
    a = (d["u"], d["delta"], d["A"], d["B"], d["C"])
    o = (d["D"], d["z"], d["bias"], True)

    def step():
        out, fin, cs = msel.msel_scan_complex_fwd(*a, *o, return_chunk_states=True)
        g = msel.msel_scan_complex_bwd(*a, d["dout"], cs, *o)
        return dict(out=out, fin=fin, **g)
    return step, ("out", "fin", "du", "ddelta", "dz"), ("dA", "dB", "dC", "dD", "ddelta_bias")


def _noalloc():
    """The backward that allocates nothing (its workspace is the library's static array), with
    chunk states rebuilt: the path for callers under graph capture."""
    t = msel_inputs.make(*SHAPE, "bf16", 35, with_dout=True, with_h0=True)
    d = to_device(t)
    a = (d["u"], d["delta"], d["A"], d["B"], d["C"])
    o = (d["D"], d["z"], d["bias"], True, d["h0"])

    def step():
        out, fin, _ = msel.msel_scan_fwd(*a, *o)
        g = msel.msel_scan_bwd_noalloc(*a, d["dout"], *o, want_dh0=True)
        return dict(out=out, fin=fin, **g)
    return (step, ("out", "fin", "du", "ddelta", "dz", "dh0"),
            ("dA", "dB", "dC", "dD", "ddelta_bias"))


def _variants_rebuilt():
    """The trapezoidal and complex backwards with their chunk states rebuilt by their own
    chunk-carry passes inside the call."""
    t = msel_inputs.make(*SHAPE, "bf16", 36, with_dout=True, with_lam=True)
    d = to_device(t)
    tc = msel_inputs.make(*SHAPE, "bf16", 37, with_dout=True, complex_A=True)
    dc = to_device(tc)

    def step():
        g = msel.msel_scan_trap_bwd(d["u"], d["delta"], d["lam"], d["A"], d["B"], d["C"],
                                    d["dout"], None, d["D"], d["z"], d["bias"], True)
        gc = msel.msel_scan_complex_bwd(dc["u"], dc["delta"], dc["A"], dc["B"], dc["C"],
                                        dc["dout"], None, dc["D"], dc["z"], dc["bias"], True)
        r = {f"trap_{k}": v for k, v in g.items()}
        r.update({f"cplx_{k}": v for k, v in gc.items()})
        return r
    exact = ("trap_du", "trap_ddelta", "trap_dz", "trap_dlam", "cplx_du", "cplx_ddelta",
             "cplx_dz")
    summed = ("trap_dA", "trap_dB", "trap_dC", "cplx_dA", "cplx_dB", "cplx_dC")
    return step, exact, summed


def _conv():
    t = msel_inputs.make_conv(2, 6, 1100, 4, "bf16", 34, with_state=True, with_dout=True)
    d = to_device(t)

    def step():
        out, st = msel.msel_conv1d_fwd(d["x"], d["weight"], d["bias"], d["state"], True,
                                       return_state=True)
        g = msel.msel_conv1d_bwd(d["x"], d["weight"], d["dout"], d["bias"], d["state"], True,
                                 want_dstate=True)
        return dict(out=out, state_out=st, **g)
    return step, ("out", "state_out", "dx", "dstate"), ("dweight", "dbias")


def _fused():
    """The backward's fused plan (gradient kernel and reduce kernel; no atomics, so every
    output replays bit for bit)."""
    t = msel_inputs.make(*SHAPE, "bf16", 38, with_dout=True, with_h0=True)
    d = to_device(t)
    a = (d["u"], d["delta"], d["A"], d["B"], d["C"])
    o = (d["D"], d["z"], d["bias"], True, d["h0"])

    def step():
        out, fin, cs = msel.msel_scan_fwd(*a, *o, return_chunk_states=True)
        msel.set_bwd_fused(1)
        try:
            assert msel.bwd_fused(d["u"], d["A"])
            g = msel.msel_scan_bwd(*a, d["dout"], *o, chunk_states=cs, want_dh0=True)
        finally:
            msel.set_bwd_fused(0)
        return dict(out=out, fin=fin, **g)
    return step, ("out", "fin", "du", "ddelta", "dz", "dh0", "dA", "dB", "dC", "dD",
                  "ddelta_bias"), ()


STEPS = {"scan": _scan, "trap": _trap, "complex": _complex, "conv": _conv, "noalloc": _noalloc,
         "variants_rebuilt": _variants_rebuilt, "fused": _fused}


@pytest.mark.parametrize("variant", list(STEPS))
def test_training_step_replays_from_a_hip_graph(variant):
    log(f"graph {variant}")
    step, exact, summed = STEPS[variant]()
    eager = step()
    torch.cuda.synchronize()
    for n in exact + summed:
        assert eager[n] is not None, n
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        step()  # warm up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            cap = step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for k in range(3):
        for n in exact + summed:
            cap[n].fill_(float("nan"))  # every replay must write all of it again
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _ = host(cap[exact[0]]).sum()  # host work between replays
        for n in exact:
            assert torch.equal(cap[n], eager[n]), (k, n)
        for n in summed:
            a, b = host(cap[n]), host(eager[n])
            assert np.all(np.isfinite(a)), (k, n)
            assert np.max(np.abs(a - b)) <= 1e-5 * np.max(np.abs(b)), (k, n)
