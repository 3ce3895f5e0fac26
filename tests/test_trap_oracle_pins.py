"""Pins of the fp64 oracle of the exponential-trapezoidal scan (oracle/trap.py).

* lambda = 1 is the zero-order-hold/Euler scan: the oracle must agree with the independently
  written C loop of oracle/msel_oracle.c (outputs, final state and chunk states);
* order of accuracy (page 5, the Mamba-3 post: the trapezoidal rule is the more accurate,
  second-order approximation): for the scalar system h' = A h + b x(t) with a smooth input, the
  error of the final state against the exact solution (closed form, cross-checked by scipy
  quadrature) must fall 4x per halving of the step for lambda = 1/2 and 2x for lambda = 1;
* impulse response: one input at step s gives y_s = C (Delta lambda B u) and
  y_{s+k} = C a^k Delta B u for k >= 1 (the two-tap convolution of the input, page 5);
* lambda = 0 on one step: h = a h0 + Delta a B_prev u_prev, y = C h + D u;
* continuing a sequence: two calls, the second started from the first's final state with
  u_prev, B_prev = the first's last inputs, equal one call;
* linearity in (u, u_prev) jointly, and causality.
"""
import numpy as np
import pytest

import msel_inputs
import oracle
from oracle import trap


def _problem(bsz=2, dim=3, N=4, L=50, seed=0, **kw):
    t = msel_inputs.make(bsz, dim, N, L, "f32", seed, with_lam=True, **kw)
    return {k: (None if t.get(k) is None else t.values(k).astype(np.float64)) for k in t}


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


@pytest.mark.parametrize("softplus", [True, False])
def test_lambda_one_is_the_euler_scan_of_the_c_oracle(softplus):
    p = _problem(bsz=2, dim=3, N=5, L=70, with_h0=True)
    lam1 = np.ones_like(p["lam"])
    # without the softplus keep Delta = delta + bias positive and small
    delta = p["delta"] if softplus else np.abs(p["delta"]) * 0.2
    bias = p["bias"] if softplus else np.abs(p["bias"]) * 0.01
    out, fin, cs = trap.fwd(p["u"], delta, lam1, p["A"], p["B"], p["C"], p["D"], p["z"],
                            bias, p["h0"], softplus=softplus, chunk_len=16)
    ro, rf = oracle.fwd(p["u"], delta, p["A"], p["B"], p["C"], p["D"], p["z"], bias,
                        p["h0"], softplus=softplus)
    assert _rel(out, ro) < 1e-12
    assert _rel(fin, rf) < 1e-12
    rcs, _ = oracle.chunk_states_formula(p["u"], delta, p["A"], p["B"], 16, p["h0"], bias,
                                         softplus=softplus)
    assert _rel(cs, rcs) < 1e-12


def _exact(A, b, h0, T, w, c):
    """h(T) for h' = A h + b (sin(w t) + c), h(0) = h0."""
    e = np.exp(A * T)
    sin_part = (-A * np.sin(w * T) - w * np.cos(w * T) + w * e) / (A * A + w * w)
    const_part = c * (e - 1.0) / A
    return e * h0 + b * (sin_part + const_part)


def _final_state(lam, n, A=-1.3, b=0.7, h0=0.4, T=2.0, w=3.0, c=0.5):
    dt = T / n
    tk = dt * np.arange(1, n + 1)                 # step j ends at t_{j+1}
    x = np.sin(w * tk) + c
    u = x.reshape(1, 1, n)
    delta = np.full((1, 1, n), dt)
    _, fin, _ = trap.fwd(u, delta, np.full((1, 1, n), lam), np.array([[A]]),
                         np.full((1, 1, n), b), np.zeros((1, 1, n)), h0=np.array([[[h0]]]),
                         u_prev=np.array([[np.sin(0.0) + c]]), B_prev=np.array([[b]]),
                         softplus=False)
    return fin[0, 0, 0], _exact(A, b, h0, T, w, c)


def test_exact_solution_matches_quadrature():
    from scipy.integrate import quad
    A, b, h0, T, w, c = -1.3, 0.7, 0.4, 2.0, 3.0, 0.5
    num = np.exp(A * T) * h0 + quad(lambda s: np.exp(A * (T - s)) * b * (np.sin(w * s) + c),
                                    0.0, T, epsabs=1e-14, epsrel=1e-14)[0]
    assert abs(num - _exact(A, b, h0, T, w, c)) < 1e-12


@pytest.mark.parametrize("lam,order", [(0.5, 2), (1.0, 1), (0.0, 1)])
def test_order_of_accuracy(lam, order):
    errs = []
    for n in (64, 128, 256, 512):
        got, want = _final_state(lam, n)
        errs.append(abs(got - want))
    ratios = [errs[i] / errs[i + 1] for i in range(len(errs) - 1)]
    for r in ratios:
        assert abs(r - 2 ** order) < 0.15 * 2 ** order, (lam, ratios)


def test_impulse_response():
    L, s, N = 12, 4, 3
    rng = np.random.default_rng(3)
    A = -rng.uniform(0.2, 1.5, size=(1, N))
    Bv, Cv = rng.standard_normal(N), rng.standard_normal(N)
    dt, lam, u0 = 0.3, 0.35, 1.7
    u = np.zeros((1, 1, L))
    u[0, 0, s] = u0
    out, _, _ = trap.fwd(u, np.full((1, 1, L), dt), np.full((1, 1, L), lam), A,
                         np.tile(Bv[None, :, None], (1, 1, L)), np.tile(Cv[None, :, None], (1, 1, L)),
                         softplus=False)
    a = np.exp(dt * A[0])
    want = np.zeros(L)
    want[s] = np.sum(Cv * dt * lam * Bv * u0)
    for k in range(1, L - s):
        want[s + k] = np.sum(Cv * a ** k * dt * Bv * u0)
    assert _rel(out[0, 0], want) < 1e-13
    assert np.all(out[0, 0, :s] == 0.0)


def test_lambda_zero_single_step():
    p = _problem(bsz=2, dim=3, N=4, L=1, with_h0=True, with_prev=True)
    lam0 = np.zeros_like(p["lam"])
    out, fin, _ = trap.fwd(p["u"], p["delta"], lam0, p["A"], p["B"], p["C"], p["D"], None,
                           p["bias"], p["h0"], p["u_prev"], p["B_prev"])
    x = p["delta"][:, :, 0] + p["bias"][None, :]
    dt = np.maximum(x, 0) + np.log1p(np.exp(-np.abs(x)))                 # [b, d]
    a = np.exp(dt[:, :, None] * p["A"][None])
    h = a * p["h0"] + dt[:, :, None] * a * p["B_prev"][:, None, :] * p["u_prev"][:, :, None]
    assert _rel(fin, h) < 1e-13
    y = np.sum(p["C"][:, None, :, 0] * h, axis=2) + p["D"][None, :] * p["u"][:, :, 0]
    assert _rel(out[:, :, 0], y) < 1e-13


@pytest.mark.parametrize("cut", [1, 17, 49])
def test_continuing_a_sequence(cut):
    p = _problem(bsz=2, dim=3, N=4, L=50, with_h0=True, with_prev=True)
    kw = dict(D=p["D"], z=p["z"], bias=p["bias"])
    full, ffin, _ = trap.fwd(p["u"], p["delta"], p["lam"], p["A"], p["B"], p["C"], h0=p["h0"],
                             u_prev=p["u_prev"], B_prev=p["B_prev"], **kw)
    sl = lambda k, a, b: p[k][:, :, a:b]
    o1, f1, _ = trap.fwd(sl("u", 0, cut), sl("delta", 0, cut), sl("lam", 0, cut), p["A"],
                         sl("B", 0, cut), sl("C", 0, cut), h0=p["h0"], u_prev=p["u_prev"],
                         B_prev=p["B_prev"], D=p["D"], z=sl("z", 0, cut), bias=p["bias"])
    o2, f2, _ = trap.fwd(sl("u", cut, 50), sl("delta", cut, 50), sl("lam", cut, 50), p["A"],
                         sl("B", cut, 50), sl("C", cut, 50), h0=f1, u_prev=p["u"][:, :, cut - 1],
                         B_prev=p["B"][:, :, cut - 1], D=p["D"], z=sl("z", cut, 50),
                         bias=p["bias"])
    assert _rel(np.concatenate([o1, o2], axis=2), full) < 1e-13
    assert _rel(f2, ffin) < 1e-13


def test_linearity_and_causality():
    p = _problem(bsz=1, dim=2, N=3, L=40, with_prev=True)
    q = _problem(bsz=1, dim=2, N=3, L=40, seed=9, with_prev=True)
    f = lambda u, up: trap.fwd(u, p["delta"], p["lam"], p["A"], p["B"], p["C"], p["D"],
                               u_prev=up, B_prev=p["B_prev"])[0]
    lhs = f(p["u"] + 2.0 * q["u"], p["u_prev"] + 2.0 * q["u_prev"])
    rhs = f(p["u"], p["u_prev"]) + 2.0 * f(q["u"], q["u_prev"])
    assert _rel(lhs, rhs) < 1e-12
    u2 = p["u"].copy()
    u2[:, :, 25:] += 1.0
    a, b = f(p["u"], p["u_prev"]), f(u2, p["u_prev"])
    np.testing.assert_array_equal(a[:, :, :25], b[:, :, :25])
    assert not np.allclose(a[:, :, 25:], b[:, :, 25:])


_GRADS = [("u", "du"), ("delta", "ddelta"), ("lam", "dlam"), ("A", "dA"), ("B", "dB"),
          ("C", "dC"), ("D", "dD"), ("z", "dz"), ("bias", "ddelta_bias"), ("h0", "dh0"),
          ("u_prev", "du_prev"), ("B_prev", "dB_prev")]


def _fwd_args(q, softplus=True):
    return (q["u"], q["delta"], q["lam"], q["A"], q["B"], q["C"], q["D"], q["z"], q["bias"],
            q["h0"], q["u_prev"], q["B_prev"])


@pytest.mark.parametrize("softplus", [True, False])
def test_bwd_matches_finite_differences(softplus):
    p = _problem(bsz=2, dim=2, N=3, L=7, with_h0=True, with_prev=True, with_dout=True)
    if not softplus:
        p["delta"] = np.abs(p["delta"]) * 0.2
        p["bias"] = np.abs(p["bias"]) * 0.01
    g = trap.bwd(*_fwd_args(p)[:6], p["dout"], *_fwd_args(p)[6:], softplus=softplus)

    def loss(**over):
        q = dict(p)
        q.update(over)
        out, _, _ = trap.fwd(*_fwd_args(q), softplus=softplus)
        return float(np.sum(p["dout"] * out))

    eps = 1e-6
    for name, gname in _GRADS:
        base = p[name]
        num = np.zeros_like(base)
        for idx in np.ndindex(*base.shape):
            hi, lo = base.copy(), base.copy()
            hi[idx] += eps
            lo[idx] -= eps
            num[idx] = (loss(**{name: hi}) - loss(**{name: lo})) / (2 * eps)
        assert g[gname].shape == base.shape, name
        assert _rel(g[gname], num) < 1e-6, name


def test_bwd_matches_torch_autograd():
    torch = pytest.importorskip("torch")
    p = _problem(bsz=2, dim=3, N=4, L=23, with_h0=True, with_prev=True, with_dout=True)
    t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=k != "dout") for k, v in p.items()}
    x = t["delta"] + t["bias"][None, :, None]
    dt = torch.nn.functional.softplus(x)
    h, up, Bp = t["h0"], t["u_prev"], t["B_prev"]
    ys = []
    for s in range(23):
        a = torch.exp(dt[:, :, s, None] * t["A"][None])
        right = t["lam"][:, :, s, None] * t["B"][:, None, :, s] * t["u"][:, :, s, None]
        left = (1 - t["lam"][:, :, s, None]) * a * Bp[:, None, :] * up[:, :, None]
        h = a * h + dt[:, :, s, None] * (right + left)
        ys.append((t["C"][:, None, :, s] * h).sum(dim=2))
        up, Bp = t["u"][:, :, s], t["B"][:, :, s]
    y = torch.stack(ys, dim=2) + t["D"][None, :, None] * t["u"]
    out = y * torch.nn.functional.silu(t["z"])
    (out * t["dout"]).sum().backward()
    g = trap.bwd(*_fwd_args(p)[:6], p["dout"], *_fwd_args(p)[6:])
    for name, gname in _GRADS:
        assert _rel(g[gname], t[name].grad.numpy()) < 1e-12, name
