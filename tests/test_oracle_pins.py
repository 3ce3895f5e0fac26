"""Pins of the fp64 CPU oracle to facts that do not come from the oracle itself.

Each test names the passage of the pages (or the mathematical fact) it relies on:

* convolutional mode: with time-invariant Delta, B and C the recurrence is a causal convolution
  with kernel C * dA^k * dB (page 1 and page 2, "convolutional mode" sentences), checked against
  ``numpy.convolve``;
* Delta -> 0 leaves only the skip term D*u (page 1 abstract: the selection lets the model
  ignore inputs depending on the token);
* state reset: a huge step drives exp(Delta*A) to exactly 0 and erases earlier history
  (page 1, "selective models can reset their state");
* chunking: the chunk formula (per-chunk transition and local state, then the link) gives the
  same states as the step-by-step loop (page 4, Appendix D, Speed paragraph);
* linearity and causality in u, closed forms for L=1, L=2 and N=1, resume from a final state;
* a second, independently written numpy oracle.
"""
import numpy as np
import pytest
from scipy.special import expit

import msel_inputs
import oracle


def _problem(bsz=1, dim=4, N=4, L=64, seed=0, **kw):
    t = msel_inputs.make(bsz, dim, N, L, "f32", seed, **kw)
    return {k: t.values(k) for k in ("u", "delta", "z", "B", "C", "A", "D", "bias", "h0", "dout")}


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


@pytest.mark.parametrize("shape", [(1, 4, 4, 64), (2, 8, 16, 256)])
def test_twin_oracle_agrees(shape):
    p = _problem(*shape, seed=7, with_h0=True)
    out_c, fin_c = oracle.fwd(p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"],
                              p["bias"], p["h0"])
    out_n, fin_n = oracle.twin_fwd(p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"],
                                   p["bias"], p["h0"])
    assert _rel(out_c, out_n) < 1e-12
    assert _rel(fin_c, fin_n) < 1e-12


@pytest.mark.parametrize("softplus", [True, False])
def test_convolutional_mode(softplus):
    """Time-invariant Delta, B, C: out = (K * u) + D u with K_k = sum_n C_n e^{k Delta A_n} Delta B_n."""
    rng = np.random.default_rng(11)
    dim, N, L = 3, 5, 80
    A = -rng.uniform(0.2, 3.0, size=(dim, N))
    raw = rng.uniform(0.01, 0.3, size=dim) if not softplus else rng.normal(-2.0, 0.5, size=dim)
    delta = np.repeat(raw[None, :, None], L, axis=2)
    Bn = rng.normal(size=N)
    Cn = rng.normal(size=N)
    B = np.repeat(Bn[None, :, None], L, axis=2)
    C = np.repeat(Cn[None, :, None], L, axis=2)
    u = rng.normal(size=(1, dim, L))
    D = rng.normal(size=dim)
    out, _ = oracle.fwd(u, delta, A, B, C, D=D, softplus=softplus, nthreads=1)
    dt = np.log1p(np.exp(raw)) if softplus else raw
    for d in range(dim):
        k = np.arange(L)
        kern = (Cn[None, :] * np.exp(k[:, None] * dt[d] * A[d][None, :]) * dt[d] * Bn[None, :]).sum(1)
        ref = np.convolve(u[0, d], kern)[:L] + D[d] * u[0, d]
        assert _rel(out[0, d], ref) < 1e-11


def test_delta_to_zero_gives_skip_only():
    p = _problem(seed=3)
    zero = np.zeros_like(p["delta"])
    out, fin = oracle.fwd(p["u"], zero, p["A"], p["B"], p["C"], p["D"], p["z"], None, None,
                          softplus=False, nthreads=1)
    z = p["z"].astype(np.float64)
    ref = p["D"].astype(np.float64)[None, :, None] * p["u"] * (z * expit(z))
    assert _rel(out, ref) < 1e-15
    assert np.all(fin == 0.0)


def test_state_reset_erases_history():
    p = _problem(seed=5)
    L, t0 = 64, 30
    delta = p["delta"].astype(np.float64).copy()
    delta[:, :, t0] = 750.0          # Delta*A_n <= -750 for every n: exp underflows to exactly 0
    args = dict(A=p["A"], B=p["B"], C=p["C"], D=p["D"], z=p["z"], bias=None, softplus=False,
                nthreads=1)
    out1, fin1 = oracle.fwd(p["u"], delta, **args)
    u2 = p["u"].astype(np.float64).copy()
    u2[:, :, :t0] += np.random.default_rng(1).normal(size=u2[:, :, :t0].shape)
    out2, fin2 = oracle.fwd(u2, delta, **args)
    assert np.array_equal(out1[:, :, t0:], out2[:, :, t0:])
    assert np.array_equal(fin1, fin2)
    assert not np.array_equal(out1[:, :, :t0], out2[:, :, :t0])


@pytest.mark.parametrize("T", [1, 7, 16, 64, 100])
def test_chunk_formula_matches_loop(T):
    p = _problem(bsz=2, dim=3, N=4, L=64, seed=9, with_h0=True)
    _, fin, cs = oracle.fwd(p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"],
                            p["bias"], p["h0"], chunk_len=T, nthreads=2)
    cs2, fin2 = oracle.chunk_states_formula(p["u"], p["delta"], p["A"], p["B"], T, h0=p["h0"],
                                            bias=p["bias"], nthreads=2)
    assert cs.shape == cs2.shape == (2, 3, -(-64 // T), 4)
    assert np.array_equal(cs[:, :, 0], p["h0"].astype(np.float64))
    assert _rel(cs2, cs) < 1e-12
    assert _rel(fin2, fin) < 1e-12


def test_linearity_and_causality_in_u():
    p = _problem(seed=13)
    args = dict(A=p["A"], B=p["B"], C=p["C"], D=p["D"], z=None, bias=p["bias"], nthreads=1)
    rng = np.random.default_rng(2)
    u1, u2 = rng.normal(size=p["u"].shape), rng.normal(size=p["u"].shape)
    o1, _ = oracle.fwd(u1, p["delta"], **args)
    o2, _ = oracle.fwd(u2, p["delta"], **args)
    o12, _ = oracle.fwd(2.5 * u1 - 0.75 * u2, p["delta"], **args)
    assert _rel(o12, 2.5 * o1 - 0.75 * o2) < 1e-12
    t1 = 40
    u3 = u1.copy()
    u3[:, :, t1 + 1:] += 1.0
    o3, _ = oracle.fwd(u3, p["delta"], **args)
    assert np.array_equal(o3[:, :, :t1 + 1], o1[:, :, :t1 + 1])


def test_closed_form_single_step():
    rng = np.random.default_rng(4)
    dim, N = 3, 6
    A = -rng.uniform(0.5, 4, size=(dim, N))
    u, delta, z = (rng.normal(size=(1, dim, 1)) for _ in range(3))
    B, C = rng.normal(size=(1, N, 1)), rng.normal(size=(1, N, 1))
    D, bias, h0 = rng.normal(size=dim), rng.normal(size=dim) * 0.1, rng.normal(size=(1, dim, N))
    out, fin = oracle.fwd(u, delta, A, B, C, D, z, bias, h0, nthreads=1)
    x = delta[0, :, 0] + bias
    dt = np.log(1.0 + np.exp(x))
    h1 = np.exp(dt[:, None] * A) * h0[0] + dt[:, None] * B[0, :, 0][None, :] * u[0, :, 0][:, None]
    y = (C[0, :, 0][None, :] * h1).sum(1) + D * u[0, :, 0]
    zz = z[0, :, 0]
    ref = y * zz / (1.0 + np.exp(-zz))
    assert _rel(out[0, :, 0], ref) < 1e-13
    assert _rel(fin[0], h1) < 1e-13


def test_closed_form_two_steps_distinguishes_B_from_C():
    """L=2, N=1: y_0 = C_0 D0 B_0 u_0 and y_1 = C_1 (e^{D1 A} D0 B_0 u_0 + D1 B_1 u_1)."""
    A = np.array([[-0.7]])
    d0, d1 = 0.3, 0.9
    delta = np.array([[[d0, d1]]])
    B = np.array([[[1.5, -2.0]]])
    C = np.array([[[0.25, 3.0]]])
    u = np.array([[[2.0, -1.0]]])
    out, fin = oracle.fwd(u, delta, A, B, C, softplus=False, nthreads=1)
    h0 = d0 * 1.5 * 2.0
    h1 = np.exp(d1 * -0.7) * h0 + d1 * -2.0 * -1.0
    assert _rel(out[0, 0], [0.25 * h0, 3.0 * h1]) < 1e-15
    assert _rel(fin[0, 0], [h1]) < 1e-15


def test_closed_form_geometric_series():
    """N=1, constant Delta, B, C, u: h_t = dB u (1 - a^{t+1}) / (1 - a)."""
    L = 50
    a_coef, dt, Bv, Cv, uv, Dv = -1.3, 0.2, 0.8, -1.1, 0.6, 0.4
    out, fin = oracle.fwd(np.full((1, 1, L), uv), np.full((1, 1, L), dt), np.array([[a_coef]]),
                          np.full((1, 1, L), Bv), np.full((1, 1, L), Cv), D=np.array([Dv]),
                          softplus=False, nthreads=1)
    a = np.exp(dt * a_coef)
    t = np.arange(L)
    h = dt * Bv * uv * (1 - a ** (t + 1)) / (1 - a)
    assert _rel(out[0, 0], Cv * h + Dv * uv) < 1e-13
    assert _rel(fin[0, 0], h[-1:]) < 1e-13


def test_resume_from_final_state():
    p = _problem(bsz=2, dim=3, N=4, L=64, seed=21, with_h0=True)
    args = dict(A=p["A"], D=p["D"], bias=p["bias"], nthreads=2)
    full, fin = oracle.fwd(p["u"], p["delta"], B=p["B"], C=p["C"], z=p["z"], h0=p["h0"], **args)
    L1 = 23
    sl = lambda a, s: None if a is None else a[:, :, s]
    o1, f1 = oracle.fwd(sl(p["u"], slice(0, L1)), sl(p["delta"], slice(0, L1)),
                        B=sl(p["B"], slice(0, L1)), C=sl(p["C"], slice(0, L1)),
                        z=sl(p["z"], slice(0, L1)), h0=p["h0"], **args)
    o2, f2 = oracle.fwd(sl(p["u"], slice(L1, None)), sl(p["delta"], slice(L1, None)),
                        B=sl(p["B"], slice(L1, None)), C=sl(p["C"], slice(L1, None)),
                        z=sl(p["z"], slice(L1, None)), h0=f1, **args)
    assert _rel(np.concatenate([o1, o2], axis=2), full) < 1e-13
    assert _rel(f2, fin) < 1e-13


def test_bf16_inputs_are_exact_values():
    """The oracle must see exactly the bf16 values the GPU reads: rounding is nearest-even."""
    x = np.array([1.0, 1.00390625, 1.005859375, 1.0078125, -3.0e38, 1e-40, np.inf],
                 dtype=np.float32)
    bits = msel_inputs.f32_to_bf16_bits(x)
    back = msel_inputs.bf16_bits_to_f32(bits)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa (1.0) wins; 1.005859375 = 1 + 1.5*2^-8
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == np.float32(1.0078125)
    assert back[3] == np.float32(1.0078125)
    assert np.isinf(back[6])
    t = msel_inputs.make(1, 2, 3, 16, "bf16", 0)
    assert t["u"].dtype == np.uint16
    assert np.all(msel_inputs.f32_to_bf16_bits(t.values("u")) == t["u"])


def test_golden_snapshot_of_tiny_workload():
    """Regression snapshot written by tests/golden/make_golden.py (oracle only)."""
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_f32_fwd_bwd.json")
    doc = json.load(open(path))
    t = msel_inputs.make(1, 4, 4, 64, "f32", 0, with_dout=True)
    v = {k: t.values(k) for k in ("u", "delta", "z", "B", "C", "A", "D", "bias", "dout")}
    out, fin = oracle.fwd(v["u"], v["delta"], v["A"], v["B"], v["C"], v["D"], v["z"], v["bias"],
                          nthreads=1)
    assert _rel(out.ravel(), doc["out"]) < 1e-13
    assert _rel(fin.ravel(), doc["final_state"]) < 1e-13
    g = oracle.bwd(v["u"], v["delta"], v["A"], v["B"], v["C"], v["dout"], v["D"], v["z"],
                   v["bias"], nthreads=1)
    for k, ref in doc["grads"].items():
        assert _rel(g[k].ravel(), ref) < 1e-13, k
