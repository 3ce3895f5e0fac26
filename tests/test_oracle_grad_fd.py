"""The oracle's hand-derived backward against central finite differences of its forward.

The backward recomputes the states from the inputs (page 1 and page 4 Appendix D, Memory
paragraph); its formulas are derived by hand, so they are pinned here element by element on a
problem of the tiny workload's size (batch 1, dim 4, dstate 4, seqlen 64): every element of every
input, in double precision, step 1e-6, relative error at most 1e-6 of the largest gradient.
"""
import numpy as np
import pytest

import msel_inputs
import oracle

EPS = 1e-6


def _loss(p, dout, softplus):
    out, _ = oracle.fwd(p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"], p["bias"],
                        p["h0"], softplus=softplus, nthreads=1)
    return float(np.sum(out * dout))


def _fd(p, dout, name, softplus):
    base = p[name]
    g = np.zeros_like(base)
    flat = base.reshape(-1)
    gf = g.reshape(-1)
    for i in range(flat.size):
        keep = flat[i]
        flat[i] = keep + EPS
        lp = _loss(p, dout, softplus)
        flat[i] = keep - EPS
        lm = _loss(p, dout, softplus)
        flat[i] = keep
        gf[i] = (lp - lm) / (2 * EPS)
    return g


@pytest.mark.parametrize("softplus,with_z", [(True, True), (False, False)])
def test_backward_matches_finite_differences(softplus, with_z):
    t = msel_inputs.make(1, 4, 4, 64, "f32", seed=0, with_z=with_z, with_h0=True,
                         with_dout=True)
    p = {k: (None if t.get(k) is None else t.values(k).astype(np.float64).copy())
         for k in ("u", "delta", "z", "B", "C", "A", "D", "bias", "h0")}
    if not softplus:
        # keep Delta positive without the softplus so that exp(Delta*A) stays a decay
        p["delta"] = np.abs(p["delta"]) * 0.2
        p["bias"] = np.abs(p["bias"]) * 0.0 + 0.01
    dout = t.values("dout").astype(np.float64)
    g = oracle.bwd(p["u"], p["delta"], p["A"], p["B"], p["C"], dout, p["D"], p["z"],
                   p["bias"], p["h0"], softplus=softplus, nthreads=1)
    pairs = [("u", "du"), ("delta", "ddelta"), ("B", "dB"), ("C", "dC"), ("A", "dA"),
             ("D", "dD"), ("bias", "ddelta_bias"), ("h0", "dh0")]
    if with_z:
        pairs.append(("z", "dz"))
    for name, gname in pairs:
        fd = _fd(p, dout, name, softplus)
        an = g[gname]
        err = np.max(np.abs(fd - an)) / max(np.max(np.abs(fd)), 1e-30)
        assert err < 1e-6, (name, err)


def test_gradient_identities():
    """dD = sum over (b, t) of dy*u and dbias = sum over (b, t) of ddelta (fixed by the chain rule)."""
    t = msel_inputs.make(2, 3, 4, 40, "f32", seed=1, with_dout=True)
    v = {k: t.values(k) for k in ("u", "delta", "z", "B", "C", "A", "D", "bias", "dout")}
    g = oracle.bwd(v["u"], v["delta"], v["A"], v["B"], v["C"], v["dout"], v["D"], v["z"],
                   v["bias"], nthreads=2)
    z = v["z"].astype(np.float64)
    dy = v["dout"] * z / (1.0 + np.exp(-z))
    assert np.allclose(g["dD"], (dy * v["u"]).sum(axis=(0, 2)), rtol=1e-12, atol=1e-12)
    assert np.allclose(g["ddelta_bias"], g["ddelta"].sum(axis=(0, 2)), rtol=1e-12, atol=1e-12)


def test_thread_count_does_not_change_results_beyond_rounding():
    t = msel_inputs.make(2, 5, 4, 33, "f32", seed=3, with_dout=True)
    v = {k: t.values(k) for k in ("u", "delta", "z", "B", "C", "A", "D", "bias", "dout")}
    g1 = oracle.bwd(v["u"], v["delta"], v["A"], v["B"], v["C"], v["dout"], v["D"], v["z"],
                    v["bias"], nthreads=1)
    g4 = oracle.bwd(v["u"], v["delta"], v["A"], v["B"], v["C"], v["dout"], v["D"], v["z"],
                    v["bias"], nthreads=4)
    for k in g1:
        if g1[k] is not None:
            assert np.allclose(g1[k], g4[k], rtol=1e-13, atol=1e-13), k
