"""Pins of the fp64 oracle of the complex-valued (rotational) scan (oracle/cplx.py).

* no rotation: with A_im = 0 every pair is two real states decaying at A_re, so the oracle
  must equal the independently written C loop of oracle/msel_oracle.c with A[d, 2j+1] set to
  A[d, 2j] (outputs, final state and chunk states);
* pure rotation: with A_re = 0 and no input, a pair turns by A_im * sum(Delta): h = (cos, sin)
  of that angle, exactly;
* parity (page 5, the Mamba-3 post: the complex state lets the model track parity, which the
  real one cannot): with Delta_t = bit_t, A = 0 + i pi, no input, h0 = (1, 0) and C = (1, 0),
  y_t = (-1)^(number of ones up to t), for random bit strings;
* the norm of a pair decays exactly as exp(A_re sum(Delta)) without input;
* continuing a sequence from its final state equals one call; linearity in u.
"""
import numpy as np
import pytest

import msel_inputs
import oracle
from oracle import cplx


def _problem(bsz=2, dim=3, N=4, L=50, seed=0, **kw):
    t = msel_inputs.make(bsz, dim, N, L, "f32", seed, complex_A=True, **kw)
    return {k: (None if t.get(k) is None else t.values(k).astype(np.float64)) for k in t}


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


@pytest.mark.parametrize("softplus", [True, False])
def test_no_rotation_is_the_real_scan_of_the_c_oracle(softplus):
    p = _problem(bsz=2, dim=3, N=6, L=70, with_h0=True)
    A = p["A"].copy()
    A[:, 1::2] = 0.0
    delta = p["delta"] if softplus else np.abs(p["delta"]) * 0.2
    bias = p["bias"] if softplus else np.abs(p["bias"]) * 0.01
    out, fin, cs = cplx.fwd(p["u"], delta, A, p["B"], p["C"], p["D"], p["z"], bias, p["h0"],
                            softplus=softplus, chunk_len=16)
    Ar = A.copy()
    Ar[:, 1::2] = A[:, 0::2]
    ro, rf = oracle.fwd(p["u"], delta, Ar, p["B"], p["C"], p["D"], p["z"], bias, p["h0"],
                        softplus=softplus)
    assert _rel(out, ro) < 1e-12
    assert _rel(fin, rf) < 1e-12
    rcs, _ = oracle.chunk_states_formula(p["u"], delta, Ar, p["B"], 16, p["h0"], bias,
                                         softplus=softplus)
    assert _rel(cs, rcs) < 1e-12


def test_pure_rotation():
    L, theta = 40, 2.3
    rng = np.random.default_rng(1)
    dt = rng.uniform(0.01, 0.2, size=(1, 1, L))
    A = np.array([[0.0, theta]])
    h0 = np.array([[[1.0, 0.0]]])
    _, fin, _ = cplx.fwd(np.zeros((1, 1, L)), dt, A, np.zeros((1, 2, L)), np.zeros((1, 2, L)),
                         h0=h0, softplus=False)
    ang = theta * dt.sum()
    np.testing.assert_allclose(fin[0, 0], [np.cos(ang), np.sin(ang)], atol=1e-13)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_parity(seed):
    L = 200
    bits = np.random.default_rng(seed).integers(0, 2, size=L).astype(np.float64)
    A = np.array([[0.0, np.pi]])
    C = np.zeros((1, 2, L))
    C[0, 0, :] = 1.0
    out, _, _ = cplx.fwd(np.zeros((1, 1, L)), bits.reshape(1, 1, L), A, np.zeros((1, 2, L)), C,
                         h0=np.array([[[1.0, 0.0]]]), softplus=False)
    want = (-1.0) ** np.cumsum(bits)
    np.testing.assert_allclose(out[0, 0], want, atol=1e-12)


def test_norm_decay_without_input():
    p = _problem(bsz=1, dim=2, N=8, L=60, with_h0=True)
    _, fin, _ = cplx.fwd(np.zeros_like(p["u"]), p["delta"], p["A"], p["B"], p["C"],
                         bias=p["bias"], h0=p["h0"])
    x = p["delta"] + p["bias"][None, :, None]
    sdt = (np.maximum(x, 0) + np.log1p(np.exp(-np.abs(x)))).sum(axis=2)      # [b, d]
    norm0 = np.hypot(p["h0"][..., 0::2], p["h0"][..., 1::2])
    norm = np.hypot(fin[..., 0::2], fin[..., 1::2])
    want = norm0 * np.exp(sdt[:, :, None] * p["A"][None, :, 0::2])
    assert _rel(norm, want) < 1e-12


@pytest.mark.parametrize("cut", [1, 23])
def test_continuing_a_sequence(cut):
    p = _problem(bsz=2, dim=3, N=4, L=50, with_h0=True)
    full, ffin, _ = cplx.fwd(p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"],
                             p["bias"], p["h0"])
    sl = lambda k, a, b: p[k][:, :, a:b]
    o1, f1, _ = cplx.fwd(sl("u", 0, cut), sl("delta", 0, cut), p["A"], sl("B", 0, cut),
                         sl("C", 0, cut), p["D"], sl("z", 0, cut), p["bias"], p["h0"])
    o2, f2, _ = cplx.fwd(sl("u", cut, 50), sl("delta", cut, 50), p["A"], sl("B", cut, 50),
                         sl("C", cut, 50), p["D"], sl("z", cut, 50), p["bias"], f1)
    assert _rel(np.concatenate([o1, o2], axis=2), full) < 1e-13
    assert _rel(f2, ffin) < 1e-13


def test_linearity_in_u():
    p = _problem(bsz=1, dim=2, N=4, L=30)
    q = _problem(bsz=1, dim=2, N=4, L=30, seed=5)
    f = lambda u: cplx.fwd(u, p["delta"], p["A"], p["B"], p["C"], p["D"])[0]
    assert _rel(f(p["u"] + 3.0 * q["u"]), f(p["u"]) + 3.0 * f(q["u"])) < 1e-12


def test_odd_dstate_is_rejected():
    with pytest.raises(ValueError):
        cplx.fwd(np.zeros((1, 1, 2)), np.zeros((1, 1, 2)), np.zeros((1, 3)), np.zeros((1, 3, 2)),
                 np.zeros((1, 3, 2)))


_GRADS = [("u", "du"), ("delta", "ddelta"), ("A", "dA"), ("B", "dB"), ("C", "dC"), ("D", "dD"),
          ("z", "dz"), ("bias", "ddelta_bias"), ("h0", "dh0")]


@pytest.mark.parametrize("softplus", [True, False])
def test_bwd_matches_finite_differences(softplus):
    p = _problem(bsz=2, dim=2, N=4, L=7, with_h0=True, with_dout=True)
    if not softplus:
        p["delta"] = np.abs(p["delta"]) * 0.2
        p["bias"] = np.abs(p["bias"]) * 0.01
    args = lambda q: (q["u"], q["delta"], q["A"], q["B"], q["C"])
    g = cplx.bwd(*args(p), p["dout"], p["D"], p["z"], p["bias"], p["h0"], softplus=softplus)

    def loss(**over):
        q = dict(p)
        q.update(over)
        out, _, _ = cplx.fwd(*args(q), q["D"], q["z"], q["bias"], q["h0"], softplus=softplus)
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


def test_bwd_matches_torch_autograd_of_the_rotation_form():
    """The same recurrence written with real 2x2 scale-rotations (the page's formulation),
    differentiated by torch on the CPU in fp64."""
    torch = pytest.importorskip("torch")
    p = _problem(bsz=2, dim=3, N=6, L=21, with_h0=True, with_dout=True)
    t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=k != "dout") for k, v in p.items()}
    dt = torch.nn.functional.softplus(t["delta"] + t["bias"][None, :, None])
    Ar, Ai = t["A"][:, 0::2], t["A"][:, 1::2]
    hr, hi = t["h0"][..., 0::2], t["h0"][..., 1::2]
    ys = []
    for s in range(21):
        e = torch.exp(dt[:, :, s, None] * Ar[None])
        ang = dt[:, :, s, None] * Ai[None]
        c, sn = e * torch.cos(ang), e * torch.sin(ang)
        pin = (dt[:, :, s] * t["u"][:, :, s])[:, :, None]
        hr, hi = (c * hr - sn * hi + pin * t["B"][:, None, 0::2, s],
                  sn * hr + c * hi + pin * t["B"][:, None, 1::2, s])
        ys.append((t["C"][:, None, 0::2, s] * hr + t["C"][:, None, 1::2, s] * hi).sum(dim=2))
    y = torch.stack(ys, dim=2) + t["D"][None, :, None] * t["u"]
    out = y * torch.nn.functional.silu(t["z"])
    (out * t["dout"]).sum().backward()
    g = cplx.bwd(p["u"], p["delta"], p["A"], p["B"], p["C"], p["dout"], p["D"], p["z"],
                 p["bias"], p["h0"])
    for name, gname in _GRADS:
        assert _rel(g[gname], t[name].grad.numpy()) < 1e-12, name
