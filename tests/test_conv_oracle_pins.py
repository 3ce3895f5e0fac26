"""Pins of the fp64 oracle of the short causal convolution to facts outside the oracle.

* impulse response: a unit input at step t0 produces the taps in reverse order at steps
  t0 .. t0+W-1 and nothing before t0 (causality and the orientation of the taps);
* a library routine: with the state at zero, the convolution equals torch's grouped
  (depthwise) conv1d padded by W-1 on the left and cut to L; with a state, the valid grouped
  conv1d over [state, x];
* SiLU: a(0) = 0, a(p) - a(-p) = p and a(ln 3) = 0.75 ln 3 (sigmoid(ln 3) = 3/4);
* streaming: a sequence cut in two pieces, the second started from the state the first left
  (the convolutional states kept in the cache, page 1 "A Secret Weapon For mamba paper"),
  gives the same outputs as one call, also when a piece is shorter than W-1; one step at a time
  (the recurrent use of the cache) gives the same as well;
* gradients: central finite differences in fp64, and torch autograd through torch's conv1d and
  SiLU on the CPU in fp64, for dx, dw, dbias and the state's gradient.
"""
import numpy as np
import pytest

import msel_inputs
from oracle import conv


def _problem(bsz=2, dim=3, L=20, W=4, seed=0, **kw):
    t = msel_inputs.make_conv(bsz, dim, L, W, "f32", seed, **kw)
    return {k: t.values(k) for k in ("x", "weight", "bias", "state", "dout")}


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


@pytest.mark.parametrize("W", [1, 2, 3, 4])
@pytest.mark.parametrize("t0", [0, 5, 11])
def test_impulse_response(W, t0):
    L, dim = 12, 2
    rng = np.random.default_rng(W * 100 + t0)
    w = rng.standard_normal((dim, W))
    x = np.zeros((1, dim, L))
    x[0, :, t0] = 1.0
    out, _ = conv.fwd(x, w, silu=False)
    want = np.zeros((1, dim, L))
    for j in range(W):
        if t0 + j < L:
            want[0, :, t0 + j] = w[:, W - 1 - j]
    np.testing.assert_array_equal(out, want)


@pytest.mark.parametrize("W", [1, 2, 3, 4])
@pytest.mark.parametrize("with_state", [False, True])
def test_matches_torch_grouped_conv1d(W, with_state):
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    p = _problem(bsz=2, dim=5, L=37, W=W, with_state=with_state)
    x = torch.tensor(p["x"], dtype=torch.float64)
    w = torch.tensor(p["weight"], dtype=torch.float64).unsqueeze(1)  # [D, 1, W]
    b = torch.tensor(p["bias"], dtype=torch.float64)
    if with_state:
        xe = torch.cat([torch.tensor(p["state"], dtype=torch.float64), x], dim=2)
        ref = F.conv1d(xe, w, b, groups=5)
    else:
        ref = F.conv1d(x, w, b, padding=W - 1, groups=5)[:, :, :37]
    pre = conv.preactivation(p["x"], p["weight"], p["bias"], p["state"])
    assert _rel(pre, ref.numpy()) < 1e-14
    out, _ = conv.fwd(p["x"], p["weight"], p["bias"], p["state"], silu=True)
    assert _rel(out, F.silu(ref).numpy()) < 1e-14


def test_silu_values():
    # with one tap of weight 1 and no bias the output is the activation of the input itself
    x = np.array([[[0.0, np.log(3.0), -np.log(3.0), 2.5, -2.5, 30.0]]])
    out, _ = conv.fwd(x, np.ones((1, 1)), silu=True)
    o = out[0, 0]
    assert o[0] == 0.0
    assert abs(o[1] - 0.75 * np.log(3.0)) < 1e-15
    assert abs((o[1] - o[2]) - np.log(3.0)) < 1e-15
    assert abs((o[3] - o[4]) - 2.5) < 1e-15
    assert abs(o[5] - 30.0) < 1e-11


@pytest.mark.parametrize("W", [2, 3, 4])
@pytest.mark.parametrize("cut", [1, 2, 9])
def test_streaming_in_two_pieces(W, cut):
    p = _problem(bsz=2, dim=3, L=16, W=W, with_state=True)
    full, fs = conv.fwd(p["x"], p["weight"], p["bias"], p["state"])
    a, sa = conv.fwd(p["x"][:, :, :cut], p["weight"], p["bias"], p["state"])
    b, sb = conv.fwd(p["x"][:, :, cut:], p["weight"], p["bias"], sa)
    assert _rel(np.concatenate([a, b], axis=2), full) < 1e-15
    np.testing.assert_array_equal(sb, fs)
    # the final state is the last W-1 inputs
    np.testing.assert_array_equal(fs, p["x"][:, :, 16 - (W - 1):])


def test_short_sequence_state_mixes_old_and_new_inputs():
    p = _problem(bsz=1, dim=2, L=2, W=4, with_state=True)
    _, fs = conv.fwd(p["x"], p["weight"], p["bias"], p["state"])
    np.testing.assert_array_equal(fs[:, :, 0], p["state"][:, :, 2])
    np.testing.assert_array_equal(fs[:, :, 1:], p["x"])


def test_one_step_at_a_time():
    p = _problem(bsz=2, dim=3, L=10, W=4, with_state=True)
    full, fs = conv.fwd(p["x"], p["weight"], p["bias"], p["state"])
    s = p["state"]
    for t in range(10):
        o, s = conv.fwd(p["x"][:, :, t:t + 1], p["weight"], p["bias"], s)
        assert _rel(o[:, :, 0], full[:, :, t]) < 1e-15
    np.testing.assert_array_equal(s, fs)


def _loss(p, silu, **over):
    q = dict(p)
    q.update(over)
    out, _ = conv.fwd(q["x"], q["weight"], q["bias"], q["state"], silu=silu)
    return float(np.sum(np.asarray(q["dout"], np.float64) * out))


@pytest.mark.parametrize("silu", [True, False])
@pytest.mark.parametrize("W", [1, 3, 4])
def test_gradients_match_finite_differences(silu, W):
    p = _problem(bsz=2, dim=2, L=7, W=W, with_state=True, with_dout=True)
    p = {k: (None if v is None else np.asarray(v, np.float64)) for k, v in p.items()}
    g = conv.bwd(p["x"], p["weight"], p["dout"], p["bias"], p["state"], silu=silu)
    eps = 1e-6
    for name, gname in (("x", "dx"), ("weight", "dweight"), ("bias", "dbias"),
                        ("state", "dstate")):
        base = p[name]
        num = np.zeros_like(base)
        for idx in np.ndindex(*base.shape):
            hi, lo = base.copy(), base.copy()
            hi[idx] += eps
            lo[idx] -= eps
            num[idx] = (_loss(p, silu, **{name: hi}) - _loss(p, silu, **{name: lo})) / (2 * eps)
        if base.size:
            assert _rel(g[gname], num) < 1e-7, name
        assert g[gname].shape == base.shape


@pytest.mark.parametrize("W", [2, 4])
def test_gradients_match_torch_autograd(W):
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    p = _problem(bsz=2, dim=4, L=19, W=W, with_state=True, with_dout=True)
    t = {k: torch.tensor(np.asarray(v, np.float64), requires_grad=k != "dout")
         for k, v in p.items()}
    xe = torch.cat([t["state"], t["x"]], dim=2)
    out = F.silu(F.conv1d(xe, t["weight"].unsqueeze(1), t["bias"], groups=4))
    (out * t["dout"]).sum().backward()
    g = conv.bwd(p["x"], p["weight"], p["dout"], p["bias"], p["state"])
    assert _rel(g["dx"], t["x"].grad.numpy()) < 1e-13
    assert _rel(g["dweight"], t["weight"].grad.numpy()) < 1e-13
    assert _rel(g["dbias"], t["bias"].grad.numpy()) < 1e-13
    assert _rel(g["dstate"], t["state"].grad.numpy()) < 1e-13
