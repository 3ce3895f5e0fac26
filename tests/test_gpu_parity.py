"""GPU parity of the HIP path against the fp64 oracle on small seeded problems.

Shapes span several tiles and chunks with ragged tails, both dtypes, with and without the gate,
softplus, D, bias and h0, and the degenerate sizes (seqlen 1, dstate 1, one channel).  The bar
is max|gpu - oracle| <= tol * max|oracle| per output tensor: tol = 1e-4 for fp32 inputs and
1e-2 for bf16 inputs (fp32 state and accumulation), on the same seeded inputs.
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

T = msel.chunk_len()

FWD_CASES = [
    # batch, dim, dstate, seqlen, dtype, z, softplus, D/bias, h0
    (1, 4, 4, 64, "f32", True, True, True, False),       # the tiny workload
    (2, 5, 16, 2500, "f32", True, True, True, True),     # 3 tiles, ragged tail
    (2, 5, 16, 2500, "bf16", True, True, True, True),    # unaligned bf16 rows
    (2, 3, 16, 4096, "bf16", False, True, True, False),  # aligned, whole tiles
    (3, 7, 5, 1000, "f32", False, False, False, True),   # odd dstate, no softplus/D/bias
    (1, 2, 16, 1, "f32", True, True, True, True),        # single step
    (1, 1, 1, 777, "bf16", True, True, True, False),     # dstate 1, one channel
    (2, 9, 16, 520, "f32", True, True, True, False),     # one chunk + 8 steps
    (1, 3, 8, 3 * 512, "bf16", True, False, True, True), # exact chunk multiple
    (2, 4, 16, 1000, "bf16", True, True, True, True),    # 16-byte rows, ragged last tile
]


def _case_inputs(bsz, dim, N, L, dtype, with_z, sp, with_db, with_h0, seed=123, dout=False):
    t = msel_inputs.make(bsz, dim, N, L, dtype, seed, with_z=with_z, with_D=with_db,
                         with_bias=with_db, with_h0=with_h0, with_dout=dout)
    if not sp:
        # without softplus keep Delta = delta + bias positive and small, as a learned step is
        v = np.abs(t.values("delta")) * np.float32(0.2)
        t["delta"] = msel_inputs.f32_to_bf16_bits(v) if dtype == "bf16" else v
        if t.get("bias") is not None:
            t["bias"] = (np.abs(t["bias"]) * np.float32(0.01)).astype(np.float32)
    return t


@pytest.mark.parametrize("case", FWD_CASES, ids=lambda c: "x".join(map(str, c[:5])))
def test_fwd_matches_oracle(case):
    bsz, dim, N, L, dtype, with_z, sp, with_db, with_h0 = case
    log(f"fwd {case}")
    t = _case_inputs(*case)
    dv = to_device(t)
    out, fin, cs = msel.msel_scan_fwd(dv["u"], dv["delta"], dv["A"], dv["B"], dv["C"], dv["D"],
                                      dv["z"], dv["bias"], sp, dv["h0"],
                                      return_chunk_states=True)
    torch.cuda.synchronize()
    v = oracle_vals(t)
    ro, rf, rcs = oracle.fwd(v["u"], v["delta"], v["A"], v["B"], v["C"], v["D"], v["z"],
                             v["bias"], v["h0"], softplus=sp, chunk_len=T)
    assert_close("out", host(out), ro, dtype)
    assert_close("final_state", host(fin), rf, dtype)
    assert_close("chunk_states", host(cs), rcs, dtype)


@pytest.mark.parametrize("case", FWD_CASES, ids=lambda c: "x".join(map(str, c[:5])))
def test_chunk_carry_matches_oracle(case):
    bsz, dim, N, L, dtype, with_z, sp, with_db, with_h0 = case
    log(f"chunk_carry {case}")
    t = _case_inputs(*case)
    dv = to_device(t)
    cs, fin = msel.msel_scan_chunk_carry(dv["u"], dv["delta"], dv["A"], dv["B"], dv["bias"], sp,
                                         dv["h0"])
    torch.cuda.synchronize()
    v = oracle_vals(t)
    rcs, rf = oracle.chunk_states_formula(v["u"], v["delta"], v["A"], v["B"], T, h0=v["h0"],
                                          bias=v["bias"], softplus=sp)
    assert_close("chunk_states", host(cs), rcs, dtype)
    assert_close("final_state", host(fin), rf, dtype)


BWD_CASES = [
    (1, 4, 4, 64, "f32", True, True, True, True),
    (2, 6, 16, 1100, "f32", True, True, True, True),
    (2, 6, 16, 1100, "bf16", True, True, True, True),
    (2, 5, 16, 2048, "bf16", False, True, True, False),
    (3, 3, 7, 700, "f32", False, False, False, True),
    (1, 3, 16, 1, "f32", True, True, True, True),
    (2, 9, 16, 1536, "f32", True, True, True, False),   # dim not a multiple of the workgroup
    (2, 13, 11, 700, "f32", True, True, True, True),    # dstate 11: the largest LDS need
    (1, 25, 10, 1030, "bf16", True, True, True, False), # two accumulator groups, ragged tail
    (2, 7, 16, 1000, "bf16", True, True, True, True),   # 16-byte rows, ragged last chunk
    (1, 1, 1, 777, "bf16", True, True, True, True),     # dstate 1, one channel: 12 ring groups
]


@pytest.mark.parametrize("given_states,want_dh0", [(False, True), (True, True), (True, False)])
@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "x".join(map(str, c[:5])))
def test_bwd_matches_oracle(case, given_states, want_dh0):
    """With the chunk states given and no dh0 asked for, the first chunk is not summarised."""
    bsz, dim, N, L, dtype, with_z, sp, with_db, with_h0 = case
    log(f"bwd {case} given_states={given_states} want_dh0={want_dh0}")
    t = _case_inputs(*case, dout=True)
    dv = to_device(t)
    cs = None
    if given_states:
        _, _, cs = msel.msel_scan_fwd(dv["u"], dv["delta"], dv["A"], dv["B"], dv["C"], dv["D"],
                                      dv["z"], dv["bias"], sp, dv["h0"],
                                      return_final_state=False, return_chunk_states=True)
    g = msel.msel_scan_bwd(dv["u"], dv["delta"], dv["A"], dv["B"], dv["C"], dv["dout"], dv["D"],
                           dv["z"], dv["bias"], sp, dv["h0"], chunk_states=cs,
                           want_dh0=want_dh0)
    torch.cuda.synchronize()
    v = oracle_vals(t)
    r = oracle.bwd(v["u"], v["delta"], v["A"], v["B"], v["C"], v["dout"], v["D"], v["z"],
                   v["bias"], v["h0"], softplus=sp)
    names = ["du", "ddelta", "dA", "dB", "dC", "dD", "ddelta_bias"]
    if want_dh0:
        names.append("dh0")
    else:
        assert g["dh0"] is None
    if with_z:
        names.append("dz")
    for k in names:
        assert_close(k, host(g[k]), r[k], dtype)
    if not with_z:
        assert g["dz"] is None


def test_fwd_is_deterministic():
    log("fwd determinism")
    t = _case_inputs(2, 5, 16, 2500, "bf16", True, True, True, True)
    dv = to_device(t)
    a = msel.msel_scan_fwd(dv["u"], dv["delta"], dv["A"], dv["B"], dv["C"], dv["D"], dv["z"],
                           dv["bias"], True, dv["h0"], return_chunk_states=True)
    b = msel.msel_scan_fwd(dv["u"], dv["delta"], dv["A"], dv["B"], dv["C"], dv["D"], dv["z"],
                           dv["bias"], True, dv["h0"], return_chunk_states=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_delta_zero_gives_exact_skip(dtype):
    """softplus off, delta = bias = 0: a = 1, dB x = 0, so out = D*u exactly and h stays 0."""
    log(f"delta=0 {dtype}")
    t = msel_inputs.make(2, 6, 16, 1300, dtype, 5, with_z=False, with_bias=False)
    dv = to_device(t)
    dv["delta"] = torch.zeros_like(dv["delta"])
    out, fin, _ = msel.msel_scan_fwd(dv["u"], dv["delta"], dv["A"], dv["B"], dv["C"], dv["D"],
                                     None, None, False)
    torch.cuda.synchronize()
    ref = (dv["D"][None, :, None] * dv["u"].float()).to(dv["u"].dtype)
    assert torch.equal(out, ref)
    assert torch.count_nonzero(fin).item() == 0


def test_state_reset_is_bitwise():
    """A step with Delta*A <= -750 zeroes exp(Delta A) in fp32: later outputs forget u before it."""
    log("state reset")
    L, t0 = 2300, 1111
    t = msel_inputs.make(1, 4, 16, L, "f32", 6, with_bias=False)
    dv = to_device(t)
    delta = dv["delta"].abs() * 0.2
    delta[:, :, t0] = 750.0
    args = (delta, dv["A"], dv["B"], dv["C"], dv["D"], dv["z"], None, False)
    o1, f1, _ = msel.msel_scan_fwd(dv["u"], *args)
    u2 = dv["u"].clone()
    u2[:, :, :t0] += torch.randn_like(u2[:, :, :t0])
    o2, f2, _ = msel.msel_scan_fwd(u2, *args)
    torch.cuda.synchronize()
    assert torch.equal(o1[:, :, t0:], o2[:, :, t0:])
    assert torch.equal(f1, f2)
    assert not torch.equal(o1[:, :, :t0], o2[:, :, :t0])


def test_causality_is_bitwise():
    log("causality")
    L, t1 = 3000, 1500
    t = msel_inputs.make(2, 3, 16, L, "bf16", 8)
    dv = to_device(t)
    args = (dv["delta"], dv["A"], dv["B"], dv["C"], dv["D"], dv["z"], dv["bias"], True)
    o1, _, _ = msel.msel_scan_fwd(dv["u"], *args)
    u2 = dv["u"].clone()
    u2[:, :, t1 + 1:] = 1.0
    o2, _, _ = msel.msel_scan_fwd(u2, *args)
    torch.cuda.synchronize()
    assert torch.equal(o1[:, :, :t1 + 1], o2[:, :, :t1 + 1])


def test_resume_from_final_state():
    """Two calls chained through h0 = final_state equal one call over the whole sequence."""
    log("resume")
    L, L1 = 3000, 1234
    t = msel_inputs.make(2, 4, 16, L, "f32", 9)
    dv = to_device(t)
    full, fin, _ = msel.msel_scan_fwd(dv["u"], dv["delta"], dv["A"], dv["B"], dv["C"], dv["D"],
                                      dv["z"], dv["bias"], True)
    s1, s2 = slice(0, L1), slice(L1, L)
    part = lambda x, s: x[:, :, s].contiguous()
    o1, f1, _ = msel.msel_scan_fwd(*(part(dv[k], s1) for k in ("u", "delta")), dv["A"],
                                   *(part(dv[k], s1) for k in ("B", "C")), dv["D"],
                                   part(dv["z"], s1), dv["bias"], True)
    o2, f2, _ = msel.msel_scan_fwd(*(part(dv[k], s2) for k in ("u", "delta")), dv["A"],
                                   *(part(dv[k], s2) for k in ("B", "C")), dv["D"],
                                   part(dv["z"], s2), dv["bias"], True, f1)
    torch.cuda.synchronize()
    assert_close("resumed out", host(torch.cat([o1, o2], 2)), host(full), "f32")
    assert_close("resumed final", host(f2), host(fin), "f32")


def test_fwd_chunk_states_agree_with_chunk_carry():
    log("fwd chunk states vs chunk carry")
    t = msel_inputs.make(2, 5, 16, 5000, "bf16", 10, with_h0=True)
    dv = to_device(t)
    _, fin, cs = msel.msel_scan_fwd(dv["u"], dv["delta"], dv["A"], dv["B"], dv["C"], dv["D"],
                                    dv["z"], dv["bias"], True, dv["h0"],
                                    return_chunk_states=True)
    cs2, fin2 = msel.msel_scan_chunk_carry(dv["u"], dv["delta"], dv["A"], dv["B"], dv["bias"],
                                           True, dv["h0"])
    torch.cuda.synchronize()
    assert_close("chunk_states", host(cs2), host(cs), "f32")
    assert_close("final", host(fin2), host(fin), "f32")


def test_binding_rejects_bad_inputs_before_launch():
    log("binding checks")
    x = torch.zeros(1, 2, 8, device="cuda")
    A = torch.zeros(2, 4, device="cuda")
    Bm = torch.zeros(1, 4, 8, device="cuda")
    with pytest.raises(ValueError):
        msel.msel_scan_fwd(x, x, A, Bm, Bm[:, :, :4])
    with pytest.raises(TypeError):
        msel.msel_scan_fwd(x.half(), x.half(), A, Bm.half(), Bm.half())
    with pytest.raises(Exception):
        msel.msel_scan_fwd(x, x, torch.zeros(2, 17, device="cuda"),
                           torch.zeros(1, 17, 8, device="cuda"),
                           torch.zeros(1, 17, 8, device="cuda"))


def test_bwd_profiled_matches_bwd_and_times_the_gradient_kernel():
    """msel_scan_bwd_profiled gives the same deterministic gradients as msel_scan_bwd and its
    events bracket a non-empty stretch of the stream."""
    log("bwd profiled")
    t = _case_inputs(2, 6, 16, 1100, "f32", True, True, True, True, dout=True)
    dv = to_device(t)
    args = (dv["u"], dv["delta"], dv["A"], dv["B"], dv["C"], dv["dout"], dv["D"], dv["z"],
            dv["bias"], True, dv["h0"])
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for e in ev:
        e.record()
    a = msel.msel_scan_bwd(*args, want_dh0=True)
    b = msel.msel_scan_bwd(*args, want_dh0=True, main_events=ev)
    torch.cuda.synchronize()
    for k in ("du", "ddelta", "dz", "dh0"):
        assert torch.equal(a[k], b[k]), k
    v = oracle_vals(t)
    r = oracle.bwd(v["u"], v["delta"], v["A"], v["B"], v["C"], v["dout"], v["D"], v["z"],
                   v["bias"], v["h0"])
    for k in ("dA", "dB", "dC", "dD", "ddelta_bias"):
        assert_close(k, host(b[k]), r[k], "f32")
    assert ev[0].elapsed_time(ev[1]) > 0.0


DECODE_CASES = [
    # batch, dim, dstate, dtype, z, softplus, D/bias, h0
    (8, 48, 16, "bf16", True, True, True, True),
    (3, 7, 5, "f32", False, False, False, True),
    (2, 5, 1, "bf16", True, True, True, False),
    (1, 33, 16, "f32", True, True, True, True),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: "x".join(map(str, c[:4])))
def test_decode_step_matches_oracle(case):
    """seqlen 1 runs the recurrent-mode step kernel: out, the next state and the one chunk
    state (the entering state) against the oracle."""
    bsz, dim, N, dtype, with_z, sp, with_db, with_h0 = case
    log(f"decode {case}")
    t = _case_inputs(bsz, dim, N, 1, dtype, with_z, sp, with_db, with_h0)
    dv = to_device(t)
    out, fin, cs = msel.msel_scan_fwd(dv["u"], dv["delta"], dv["A"], dv["B"], dv["C"], dv["D"],
                                      dv["z"], dv["bias"], sp, dv["h0"],
                                      return_chunk_states=True)
    torch.cuda.synchronize()
    v = oracle_vals(t)
    ro, rf, rcs = oracle.fwd(v["u"], v["delta"], v["A"], v["B"], v["C"], v["D"], v["z"],
                             v["bias"], v["h0"], softplus=sp, chunk_len=T)
    assert_close("out", host(out), ro, dtype)
    assert_close("final_state", host(fin), rf, dtype)
    assert_close("chunk_states", host(cs), rcs, dtype)


def test_decode_steps_update_the_state_in_place_and_follow_the_scan():
    """Six decode steps with final_state = h0 (one buffer) give the same outputs and final
    state as one forward scan over the six steps (within the fp32 tolerance) and as the
    oracle."""
    log("decode in place")
    bsz, dim, N, L = 2, 9, 16, 6
    t = _case_inputs(bsz, dim, N, L, "f32", True, True, True, True)
    dv = to_device(t)
    state = dv["h0"].clone()
    outs = []
    for s in range(L):
        sl = lambda x: None if x is None else x[..., s:s + 1].contiguous()
        o, f, _ = msel.msel_scan_fwd(sl(dv["u"]), sl(dv["delta"]), dv["A"], sl(dv["B"]),
                                     sl(dv["C"]), dv["D"], sl(dv["z"]), dv["bias"], True, state,
                                     final_state=state)
        assert f.data_ptr() == state.data_ptr()
        outs.append(o)
    torch.cuda.synchronize()
    got = torch.cat(outs, dim=-1)
    ref_out, ref_fin, _ = msel.msel_scan_fwd(dv["u"], dv["delta"], dv["A"], dv["B"], dv["C"],
                                             dv["D"], dv["z"], dv["bias"], True, dv["h0"])
    torch.cuda.synchronize()
    assert_close("steps vs scan out", host(got), host(ref_out).astype(np.float64), "f32")
    assert_close("steps vs scan state", host(state), host(ref_fin).astype(np.float64), "f32")
    v = oracle_vals(t)
    ro, rf = oracle.fwd(v["u"], v["delta"], v["A"], v["B"], v["C"], v["D"], v["z"], v["bias"],
                        v["h0"])
    assert_close("out", host(got), ro, "f32")
    assert_close("final_state", host(state), rf, "f32")


def test_decode_step_replays_from_a_hip_graph():
    """The decode step only enqueues a kernel, so it can be captured in a graph: three replays,
    each followed by host work and a synchronisation, match three eager steps bit for bit."""
    log("decode graph")
    bsz, dim, N = 4, 24, 16
    t = _case_inputs(bsz, dim, N, 1, "bf16", True, True, True, True)
    dv = to_device(t)
    args = (dv["u"], dv["delta"], dv["A"], dv["B"], dv["C"], dv["D"], dv["z"], dv["bias"], True)
    eager_state = dv["h0"].clone()
    eager_outs = []
    for _ in range(3):
        o, _, _ = msel.msel_scan_fwd(*args, eager_state, final_state=eager_state)
        eager_outs.append(o.clone())
    torch.cuda.synchronize()
    state = dv["h0"].clone()
    out = torch.empty_like(dv["u"])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            msel.msel_scan_fwd(*args, state, out=out, final_state=state)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    state.copy_(dv["h0"])
    torch.cuda.synchronize()
    for k in range(3):
        graph.replay()
        torch.cuda.synchronize()
        _ = host(out).sum()  # host work between replays
        assert torch.equal(out, eager_outs[k]), k
    assert torch.equal(state, eager_state)


@pytest.mark.parametrize("shape", [(1, 2, 0), (1, 0, 8), (0, 2, 8)])
def test_empty_problem_is_an_error(shape):
    """No steps, no channels or no batch rows: the library rejects the call before any launch
    (an empty problem is a shape error, not a silent no-op), and the binding raises."""
    log(f"empty {shape}")
    bsz, dim, L = shape
    N = 4
    dev = torch.device("cuda")
    u = torch.zeros(shape, device=dev)
    A = -torch.ones(dim, N, device=dev)
    Bm = torch.zeros(bsz, N, L, device=dev)
    with pytest.raises((ValueError, RuntimeError)):
        msel.msel_scan_fwd(u, u.clone(), A, Bm, Bm.clone(), None, None, None, True)
    with pytest.raises((ValueError, RuntimeError)):
        msel.msel_scan_bwd(u, u.clone(), A, Bm, Bm.clone(), u.clone(), None, None, None, True)
