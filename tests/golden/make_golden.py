"""Writes tests/golden/tiny_f32_fwd_bwd.json from the fp64 oracle only.

The pages print no worked numerical example of the scan, so this fixture is a regression
snapshot of the oracle itself on the tiny workload (batch 1, dim 4, dstate 4, seqlen 64, seed 0,
softplus on, gate on), taken after the oracle passed its pins (convolutional mode, Delta -> 0,
state reset, chunk formula, closed forms, numpy twin, finite differences).  It guards the oracle
against silent changes; it is not an independent pin.

Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import msel_inputs  # noqa: E402
import oracle  # noqa: E402


def main():
    w = msel_inputs.WORKLOADS[0]
    t = msel_inputs.make(w.batch, w.dim, w.dstate, w.seqlen, w.dtype, w.seed, with_dout=True)
    v = {k: t.values(k) for k in ("u", "delta", "z", "B", "C", "A", "D", "bias", "dout")}
    out, fin = oracle.fwd(v["u"], v["delta"], v["A"], v["B"], v["C"], v["D"], v["z"], v["bias"],
                          nthreads=1)
    g = oracle.bwd(v["u"], v["delta"], v["A"], v["B"], v["C"], v["dout"], v["D"], v["z"],
                   v["bias"], nthreads=1)
    doc = {
        "workload": "batch 1, dim 4, dstate 4, seqlen 64, f32, seed 0 (msel_inputs.make)",
        "source": "fp64 oracle (oracle.fwd / oracle.bwd), regression snapshot",
        "out": out.ravel().tolist(),
        "final_state": fin.ravel().tolist(),
        "grads": {k: g[k].ravel().tolist() for k in ("du", "ddelta", "dz", "dA", "dB", "dC",
                                                     "dD", "ddelta_bias")},
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_f32_fwd_bwd.json")
    with open(path, "w") as f:
        json.dump(doc, f, indent=0)
    print("wrote", path)


if __name__ == "__main__":
    main()
