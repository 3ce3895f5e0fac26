"""Benchmark of the selective scan on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2] [--no-cpu]

A step is one pass of the whole hot path over one batch of synthetic input resident in HBM:
the fused forward scan (out, final state and the state at every chunk boundary), then the
backward with recomputation (all gradients): it rebuilds every state inside the chunks from
those boundary states and runs the chunk carry backward for the adjoint.  The standalone
chunk-carry entry point is timed separately.  The
default workload is batch 8, d_model 768 x expand 2 = 1536 channels, dstate 16, seqlen 2048,
bf16 activations with fp32 state -- the workload that runs both the forward and the backward.

Prints one JSON line: the whole-step throughput in token*channels/s, the roofline of the
dominant kernel (from HIP events on the launch stream over the timed steps), per-kernel
figures, and the fp64 CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
VALU_PEAK_TOPS = 39.32         # 256 CUs x 64 fp32 lanes/clk x 2.4 GHz, in 1e12 lane-ops/s
METRIC = "selective-scan fwd/bwd tokens·channels/s and achieved HBM GB/s (% of peak)"


def algorithmic_bytes(w, nchunks):
    s = 2 if w.dtype == "bf16" else 4
    tc = w.batch * w.dim * w.seqlen
    bnl = w.batch * w.dstate * w.seqlen
    dn, d = w.dim * w.dstate, w.dim
    fwd = 4 * tc * s + 2 * bnl * s + w.batch * w.dim * w.dstate * 4 + dn * 4 + 2 * d * 4
    cc = 2 * tc * s + bnl * s + w.batch * w.dim * nchunks * w.dstate * 4 + dn * 4 + d * 4
    bwd = 7 * tc * s + 2 * bnl * s + 2 * bnl * 4 + 2 * dn * 4 + 4 * d * 4
    return {"fwd": fwd, "chunk_carry": cc, "bwd": bwd}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-channels", type=int, default=192,
                    help="channels per batch row in the CPU-baseline sample")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import msel_inputs
    import selective_state_space_26_amd as msel

    w = msel_inputs.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t = msel_inputs.make_workload(w, with_dout=True)
    act = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def put(v, dt):
        if v is None:
            return None
        if v.dtype == np.uint16:
            return torch.from_numpy(v.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(v)).to(device=dev, dtype=dt)

    d = {k: put(v, act if k in ("u", "delta", "z", "B", "C", "dout") else torch.float32)
         for k, v in t.items()}
    nch = msel.num_chunks(w.seqlen)
    names = ("fwd", "bwd")
    ws = torch.empty(msel.bwd_workspace_bytes(d["u"], d["A"], True), device=dev,
                     dtype=torch.uint8)

    def step(ev=None):
        """fwd (out, final state, one state per chunk) then bwd, which recomputes every state
        inside the chunks and runs the chunk carry backward for the adjoint."""
        if ev is not None:
            ev[0].record()
        out, fin, cs = msel.msel_scan_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"],
                                          d["z"], d["bias"], True, return_chunk_states=True)
        if ev is not None:
            ev[1].record()
        g = msel.msel_scan_bwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["dout"], d["D"],
                               d["z"], d["bias"], True, chunk_states=cs, workspace=ws)
        if ev is not None:
            ev[2].record()
        return out, fin, g

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    per = {n: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs]))
           for i, n in enumerate(names)}

    tc = w.batch * w.dim * w.seqlen
    alg = algorithmic_bytes(w, nch)
    # the standalone chunk-carry pass, timed on its own after the steps
    cc_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for _ in range(3):
        msel.msel_scan_chunk_carry(d["u"], d["delta"], d["A"], d["B"], d["bias"], True)
    cc_ev[0].record()
    for _ in range(args.steps):
        msel.msel_scan_chunk_carry(d["u"], d["delta"], d["A"], d["B"], d["bias"], True)
    cc_ev[1].record()
    torch.cuda.synchronize()
    per["chunk_carry"] = cc_ev[0].elapsed_time(cc_ev[1]) / args.steps
    kernels = {}
    for n in ("fwd", "chunk_carry", "bwd"):
        gbs = alg[n] / (per[n] * 1e-3) / 1e9
        kernels[n] = {"ms": round(per[n], 4), "alg_bytes": alg[n], "GB/s": round(gbs, 1),
                      "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                      "tc_per_s": float(f"{tc / (per[n] * 1e-3):.4g}")}
    kernels["bwd"]["note"] = ("msel_scan_bwd call: convert + summary + link + main kernels and "
                              "zero-fills")
    dom = max(names, key=lambda n: per[n])
    ach = alg[dom] / (per[dom] * 1e-3) / 1e9
    roofline = {"kernel": dom, "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None}

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(w, t, args.cpu_channels)

    line = {
        "metric": METRIC, "value": float(f"{tc / (ms_per_step * 1e-3):.5g}"),
        "unit": "token*channels/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "dim": w.dim, "dstate": w.dstate,
                   "seqlen": w.seqlen, "step": "fwd (with chunk-boundary states) + bwd"},
        "roofline": roofline, "kernels": kernels, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(w, t, channels):
    """The fp64 oracle, as it stands, on the first `channels` channels of every batch row:
    forward + backward, timed on this host's cores."""
    import numpy as np

    import oracle
    ch = min(channels, w.dim)
    v = {k: (None if t.get(k) is None else t.values(k)) for k in t}
    sl = lambda x: None if x is None else np.ascontiguousarray(x[:, :ch])
    sub = dict(u=sl(v["u"]), delta=sl(v["delta"]), z=sl(v["z"]), dout=sl(v["dout"]),
               A=v["A"][:ch], D=v["D"][:ch], bias=v["bias"][:ch], B=v["B"], C=v["C"])
    nthreads = oracle.default_threads()
    s = time.perf_counter()
    oracle.fwd(sub["u"], sub["delta"], sub["A"], sub["B"], sub["C"], sub["D"], sub["z"],
               sub["bias"], nthreads=nthreads)
    oracle.bwd(sub["u"], sub["delta"], sub["A"], sub["B"], sub["C"], sub["dout"], sub["D"],
               sub["z"], sub["bias"], nthreads=nthreads)
    el = time.perf_counter() - s
    tcs = w.batch * ch * w.seqlen
    return {"value": float(f"{tcs / el:.4g}"), "unit": "token*channels/s", "cores": nthreads,
            "kind": "oracle", "seconds": round(el, 3),
            "sample": f"fwd+bwd (chunk states recomputed inside the loop) on channels 0..{ch - 1}"
                      f" of all {w.batch} batch rows, full seqlen {w.seqlen}"}


if __name__ == "__main__":
    main()
