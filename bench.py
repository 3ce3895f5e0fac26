"""Benchmark of the selective scan on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2] [--no-cpu]

A step is one pass of the whole hot path over one batch of synthetic input resident in HBM:
the fused forward scan (out, final state and the state at every chunk boundary), then the
backward with recomputation (all gradients): it rebuilds every state inside the chunks from
those boundary states and runs the chunk carry backward for the adjoint.  The standalone
chunk-carry entry point is timed separately, and so are the recurrent (decode) step and
the short causal convolution + SiLU that produces the scan's input (forward, backward and its
decode step, width 4, at the same batch, channels, length and dtype).  The
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
FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X fp32 vector: 256 CUs x 256 flop/clk x 2.4 GHz
METRIC = "selective-scan fwd/bwd tokens·channels/s and achieved HBM GB/s (% of peak)"
# fp32 flops per (batch, channel, time, state) update, FMA = 2, exp2 = 1 (the arithmetic of
# the recurrence itself; the parallel scan's replay and combine steps are not counted)
FLOPS_FWD = 7      # Delta*A, exp2, (Delta u)*B, h = a h + p, y += C h
FLOPS_BWD = 20     # recompute h (5), adjoint (3), g = lam h a (2), dA, dDelta, du, dB, dC (10)
FLOPS_BWD_Z = 2    # y += C h, rebuilt for dz when there is a gate
FLOPS_TRAP = 10    # Delta*A, exp2, c*B_prev, (gamma u)*B, p = a*(c B_prev) + .., h, y
FLOPS_TRAP_BWD = 31  # the backward's 20 + the previous/next-step input terms of the rule
# per complex state (a pair of real states) and step: Delta*A_re, Delta*A_im, exp2, sin, cos,
# the two products of the transition, (Delta u)*B for both parts, h = a h + p (4 fma), y (2 fma)
FLOPS_COMPLEX_PAIR = 21
# its backward per complex state and step: recompute h (17), the adjoint conj(a) G + C dy (12),
# X = conj(G) a h (12), the dDelta, dA, du, dB and dC terms (18)
FLOPS_COMPLEX_BWD_PAIR = 59
# rocprofv3 FETCH_SIZE / WRITE_SIZE summaries, per kernel, of the default workload
TRAFFIC_FILE = "profiles/{kernel}_d768x2_bf16_traffic.txt"
CONV_WIDTH = 4     # taps of the short causal convolution before the scan
CONV_SETS = 4      # input copies the convolution timing cycles through (> last-level cache)


def algorithmic_bytes(w, nchunks):
    """Bytes each pass must move at least once between HBM and the chip."""
    s = 2 if w.dtype == "bf16" else 4
    tc = w.batch * w.dim * w.seqlen
    bnl = w.batch * w.dstate * w.seqlen
    states = w.batch * w.dim * nchunks * w.dstate * 4
    dn, d = w.dim * w.dstate, w.dim
    fwd = 4 * tc * s + 2 * bnl * s + states + w.batch * w.dim * w.dstate * 4 + dn * 4 + 2 * d * 4
    cc = 2 * tc * s + bnl * s + states + dn * 4 + d * 4
    # the gradient kernel: u, delta, dout, z in; du, ddelta, dz out; B, C in; dB, dC out
    # (fp32); chunk-start states and adjoint carries in; A, D, bias in; dA, dD, dbias out
    bwd_main = 7 * tc * s + 2 * bnl * s + 2 * bnl * 4 + 2 * states + 2 * (dn + 2 * d) * 4
    # the whole msel_scan_bwd call: the same tensors once (its summary pass reads delta, dout
    # and z a second time; that re-read is not counted)
    bwd = 7 * tc * s + 2 * bnl * s + 2 * bnl * 4 + 2 * dn * 4 + 4 * d * 4
    return {"fwd": fwd, "chunk_carry": cc, "bwd_main": bwd_main, "bwd": bwd}


def measured_traffic(workload_name, kernel="bwd_main_kernel"):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    summary, or None when there is none for this workload or the kernel's sources have changed
    since the counters were taken."""
    path = os.path.join(ROOT, TRAFFIC_FILE.format(kernel=kernel))
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if "=" in line and not line.lstrip().startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    from selective_state_space_26_amd.profsum import source_digest, sources_of
    if (kv.get("workload") != workload_name or kv.get("kernel") != kernel
            or kv.get("source_sha256") != source_digest(sources_of(kernel))):
        return None
    try:
        return int(float(kv["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the oracle over the whole workload for at least this long")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="before the steps, copy a buffer of this many MiB once (a plain copy "
                         "kernel of known size that scales the HBM byte counters)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path; its sharding is "
              "a design, not code (run with --gpus 1).", file=sys.stderr)
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
    ws = torch.empty(msel.bwd_workspace_bytes(d["u"], d["A"], True), device=dev,
                     dtype=torch.uint8)

    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, device=dev, dtype=torch.float32)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def new_events(k):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(k)]
        for e in ev:   # the library records the gradient-kernel events itself: create them
            e.record()
        return ev

    def step(ev=None):
        """fwd (out, final state, one state per chunk) then bwd, which recomputes every state
        inside the chunks and runs the chunk carry backward for the adjoint.  All launches go
        to torch's current stream, on which the events are recorded."""
        if ev is not None:
            ev[0].record()
        out, fin, cs = msel.msel_scan_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"],
                                          d["z"], d["bias"], True, return_chunk_states=True)
        if ev is not None:
            ev[1].record()
        g = msel.msel_scan_bwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["dout"], d["D"],
                               d["z"], d["bias"], True, chunk_states=cs, workspace=ws,
                               main_events=None if ev is None else (ev[3], ev[4]))
        if ev is not None:
            ev[2].record()
        return out, fin, g

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [new_events(5) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    per = {
        "fwd": float(np.mean([e[0].elapsed_time(e[1]) for e in evs])),
        "bwd": float(np.mean([e[1].elapsed_time(e[2]) for e in evs])),
        "bwd_main": float(np.mean([e[3].elapsed_time(e[4]) for e in evs])),
    }

    tc = w.batch * w.dim * w.seqlen
    upd = tc * w.dstate
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

    # the recurrent (decode) step at the same batch and channels: seqlen 1, state in place
    st = {k: (None if v is None else (v[..., :1].contiguous() if k in ("u", "delta", "z", "B", "C")
                                        else v)) for k, v in d.items()}
    state = torch.zeros(w.batch, w.dim, w.dstate, device=dev, dtype=torch.float32)
    dec_out = torch.empty_like(st["u"])
    def decode():
        msel.msel_scan_fwd(st["u"], st["delta"], st["A"], st["B"], st["C"], st["D"], st["z"],
                           st["bias"], True, state, out=dec_out, final_state=state)
    dec_per_graph, dec_reps = 32, 10
    per["decode_step"] = graph_time(decode, dec_per_graph, dec_reps)

    # the exponential-trapezoidal forward at the same shape: one more input stream (lambda);
    # calls alternate between two copies of the streamed inputs (~400 MB, more than the
    # last-level cache)
    lam = put(msel_inputs.make(w.batch, w.dim, w.dstate, w.seqlen, w.dtype, w.seed,
                               with_lam=True)["lam"], act)
    tsets = [{k: (d[k] if i == 0 else d[k].clone()) for k in ("u", "delta", "z")} |
             {"lam": lam if i == 0 else lam.clone(), "out": torch.empty_like(d["u"])}
             for i in range(2)]
    trap_cs = torch.empty(w.batch, w.dim, nch, w.dstate, device=dev, dtype=torch.float32)
    trap_fin = torch.empty(w.batch, w.dim, w.dstate, device=dev, dtype=torch.float32)

    def trap_fwd(i):
        c = tsets[i % 2]
        msel.msel_scan_trap_fwd(c["u"], c["delta"], c["lam"], d["A"], d["B"], d["C"], d["D"],
                                c["z"], d["bias"], True, out=c["out"], final_state=trap_fin,
                                chunk_states=trap_cs)
    for i in range(4):
        trap_fwd(i)
    tev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    tev[0].record()
    for i in range(args.steps):
        trap_fwd(i)
    tev[1].record()
    torch.cuda.synchronize()
    per["trap_fwd"] = tev[0].elapsed_time(tev[1]) / args.steps
    # its backward, from the chunk states of copy 0 (the call streams ~550 MB: no rotation)
    trap_fwd(0)
    trap_ws = torch.empty(msel.bwd_workspace_bytes(d["u"], d["A"], True), device=dev,
                          dtype=torch.uint8)

    def trap_bwd():
        c = tsets[0]
        msel.msel_scan_trap_bwd(c["u"], c["delta"], c["lam"], d["A"], d["B"], d["C"], d["dout"],
                                trap_cs, d["D"], c["z"], d["bias"], True, workspace=trap_ws)
    for _ in range(3):
        trap_bwd()
    tev[0].record()
    for _ in range(args.steps):
        trap_bwd()
    tev[1].record()
    torch.cuda.synchronize()
    per["trap_bwd"] = tev[0].elapsed_time(tev[1]) / args.steps
    del tsets, trap_ws

    # the complex-valued (rotational) forward at the same shape: dstate 16 = 8 complex states,
    # rates -1/2 + i pi j; calls alternate between the two input copies above
    cA = put(msel_inputs.make(1, w.dim, w.dstate, 1, "f32", w.seed, complex_A=True)["A"],
             torch.float32)
    csets = [{k: (d[k] if i == 0 else d[k].clone()) for k in ("u", "delta", "z")} |
             {"out": torch.empty_like(d["u"])} for i in range(2)]

    def complex_fwd(i):
        c = csets[i % 2]
        msel.msel_scan_complex_fwd(c["u"], c["delta"], cA, d["B"], d["C"], d["D"], c["z"],
                                   d["bias"], True, out=c["out"], final_state=trap_fin,
                                   chunk_states=trap_cs)
    for i in range(4):
        complex_fwd(i)
    cev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    cev[0].record()
    for i in range(args.steps):
        complex_fwd(i)
    cev[1].record()
    torch.cuda.synchronize()
    per["complex_fwd"] = cev[0].elapsed_time(cev[1]) / args.steps
    # its backward, from the chunk states of copy 0
    complex_fwd(0)
    cws = torch.empty(msel.bwd_workspace_bytes(d["u"], d["A"], True), device=dev,
                      dtype=torch.uint8)

    def complex_bwd():
        c = csets[0]
        msel.msel_scan_complex_bwd(c["u"], c["delta"], cA, d["B"], d["C"], d["dout"], trap_cs,
                                   d["D"], c["z"], d["bias"], True, workspace=cws)
    for _ in range(3):
        complex_bwd()
    cev[0].record()
    for _ in range(args.steps):
        complex_bwd()
    cev[1].record()
    torch.cuda.synchronize()
    per["complex_bwd"] = cev[0].elapsed_time(cev[1]) / args.steps
    del csets, cws

    # the short causal convolution + SiLU that makes the scan's input, at the same batch,
    # channels, length and dtype, width 4, with bias and incoming state: forward, backward
    # (zero-fill + one kernel) and the decode step (seqlen 1, state updated in place)
    cv = {k: put(v, act if k in ("x", "state", "dout") else torch.float32)
          for k, v in msel_inputs.make_conv(w.batch, w.dim, w.seqlen, CONV_WIDTH, w.dtype,
                                            w.seed, with_state=True, with_dout=True).items()}
    # consecutive calls cycle through CONV_SETS copies of the streamed tensors, more than the
    # chip's 256 MB last-level cache holds, so that each call reads its inputs from HBM
    sets = [{"x": cv["x"] if i == 0 else cv["x"].clone(),
             "dout": cv["dout"] if i == 0 else cv["dout"].clone(),
             "out": torch.empty_like(cv["x"]), "state_out": torch.empty_like(cv["state"])}
            for i in range(CONV_SETS)]

    def conv_fwd(i):
        c = sets[i % CONV_SETS]
        msel.msel_conv1d_fwd(c["x"], cv["weight"], cv["bias"], cv["state"], out=c["out"],
                             state_out=c["state_out"])

    def conv_bwd(i):
        c = sets[i % CONV_SETS]
        msel.msel_conv1d_bwd(c["x"], cv["weight"], c["dout"], cv["bias"], cv["state"],
                             want_dstate=True)

    for name, fn in (("conv_fwd", conv_fwd), ("conv_bwd", conv_bwd)):
        for i in range(CONV_SETS):
            fn(i)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for i in range(args.steps):
            fn(i)
        ev[1].record()
        torch.cuda.synchronize()
        per[name] = ev[0].elapsed_time(ev[1]) / args.steps
    del sets
    cx1 = cv["x"][..., :1].contiguous()
    cache = cv["state"].clone()
    conv_dec_out = torch.empty_like(cx1)

    def conv_decode():
        msel.msel_conv1d_fwd(cx1, cv["weight"], cv["bias"], cache, out=conv_dec_out,
                             state_out=cache)
    per["conv_decode_step"] = graph_time(conv_decode, dec_per_graph, dec_reps)

    fl_bwd = FLOPS_BWD + (FLOPS_BWD_Z if d.get("z") is not None else 0)
    flops = {"fwd": FLOPS_FWD * upd, "bwd_main": fl_bwd * upd, "trap_fwd": FLOPS_TRAP * upd,
             "complex_fwd": FLOPS_COMPLEX_PAIR * upd // 2}
    alg["trap_fwd"] = alg["fwd"] + tc * (2 if w.dtype == "bf16" else 4)  # + lambda
    alg["complex_fwd"] = alg["fwd"]
    # + lambda in, dlambda out
    alg["trap_bwd"] = alg["bwd"] + 2 * tc * (2 if w.dtype == "bf16" else 4)
    alg["complex_bwd"] = alg["bwd"]
    flops["complex_bwd"] = FLOPS_COMPLEX_BWD_PAIR * upd // 2
    flops["trap_bwd"] = (FLOPS_TRAP_BWD + (FLOPS_BWD_Z if d.get("z") is not None else 0)) * upd
    kernels = {}
    for n in ("fwd", "chunk_carry", "bwd_main", "bwd", "trap_fwd", "trap_bwd", "complex_fwd",
              "complex_bwd"):
        sec = per[n] * 1e-3
        gbs = alg[n] / sec / 1e9
        kernels[n] = {"ms": round(per[n], 4), "alg_bytes": alg[n], "GB/s": round(gbs, 1),
                      "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                      "tc_per_s": float(f"{tc / sec:.4g}")}
        if n in flops:
            kernels[n]["TFLOP/s"] = round(flops[n] / sec / 1e12, 2)
    kernels["fwd"]["what"] = "scan_fwd_kernel (one launch)"
    kernels["complex_bwd"]["what"] = ("the msel_scan_complex_bwd call (zero-fills, summary, link "
                                      "and the pair-per-wavefront gradient kernel), timed apart "
                                      "from the step")
    kernels["trap_bwd"]["what"] = ("the msel_scan_trap_bwd call (zero-fills, summary, link and "
                                   "the trapezoidal gradient kernel), timed apart from the step")
    kernels["complex_fwd"]["what"] = ("scan_cplx_fwd_kernel: the complex-valued (rotational) "
                                      "forward, dstate 16 as 8 complex states, one launch, "
                                      "timed apart from the step")
    kernels["trap_fwd"]["what"] = ("scan_fwd_kernel with the exponential-trapezoidal rule "
                                   "(msel_scan_trap_fwd, lambda as one more input), one launch, "
                                   "timed apart from the step")
    kernels["chunk_carry"]["what"] = "chunk_carry_kernel (one launch), timed apart from the step"
    kernels["bwd_main"]["what"] = "bwd_main_kernel, the chunk-parallel gradient kernel"
    kernels["bwd"]["what"] = ("the msel_scan_bwd call: zero-fills, summary, link and "
                              "bwd_main_kernel")
    s_ = 2 if w.dtype == "bf16" else 4
    dec_bytes = (2 * w.batch * w.dim * w.dstate * 4 + 4 * w.batch * w.dim * s_ +
                 2 * w.batch * w.dstate * s_ + w.dim * w.dstate * 4 + 2 * w.dim * 4)
    dsec = per["decode_step"] * 1e-3
    kernels["decode_step"] = {
        "ms": round(per["decode_step"], 4), "alg_bytes": dec_bytes,
        "GB/s": round(dec_bytes / dsec / 1e9, 1),
        "hbm_frac": round(dec_bytes / dsec / 1e9 / HBM_PEAK_GBS, 4),
        "tc_per_s": float(f"{w.batch * w.dim / dsec:.4g}"),
        "what": "scan_step_kernel: one recurrent step (seqlen 1) of every channel, state "
                "updated in place; steps replayed from a HIP graph"}

    rows = w.batch * w.dim
    H = CONV_WIDTH - 1
    conv_bytes = {
        # x in, out out; state in and out; taps and bias in
        "conv_fwd": 2 * tc * s_ + 2 * rows * H * s_ + w.dim * (CONV_WIDTH + 1) * 4,
        # x, dout in, dx out; state in, its fp32 gradient out; taps, bias in, their grads out
        "conv_bwd": 3 * tc * s_ + rows * H * (s_ + 4) + 2 * w.dim * (CONV_WIDTH + 1) * 4,
        "conv_decode_step": 2 * rows * s_ + 2 * rows * H * s_ + w.dim * (CONV_WIDTH + 1) * 4,
    }
    what = {"conv_fwd": "conv_fwd_kernel: causal depthwise conv (width 4) + bias + SiLU, "
                        "state in and out (one launch)",
            "conv_bwd": "the msel_conv1d_bwd call: zero-fill of the tap/bias gradients and "
                        "conv_bwd_kernel (recomputes the activation)",
            "conv_decode_step": "conv_step_kernel: msel_conv1d_fwd at seqlen 1 with the state "
                                "updated in place; steps replayed from a HIP graph"}
    for n, nb in conv_bytes.items():
        sec = per[n] * 1e-3
        toks = rows if n == "conv_decode_step" else tc
        kernels[n] = {"ms": round(per[n], 4), "alg_bytes": nb, "GB/s": round(nb / sec / 1e9, 1),
                      "hbm_frac": round(nb / sec / 1e9 / HBM_PEAK_GBS, 4),
                      "tc_per_s": float(f"{toks / sec:.4g}"), "what": what[n]}
        if n in ("conv_fwd", "conv_bwd"):
            kernels[n]["traffic"] = measured_traffic(w.name, n + "_kernel")

    # the dominant kernel: the gradient kernel, bound by VALU arithmetic (an exp2 per update
    # and ~20 flops), measured with the library's events on the launch stream
    sec = per["bwd_main"] * 1e-3
    ach = flops["bwd_main"] / sec / 1e12
    roofline = {
        "kernel": "bwd_main_kernel", "bound": "alu", "achieved": round(ach, 2),
        "peak": FP32_VECTOR_PEAK_TFLOPS, "unit": "TFLOP/s",
        "frac": round(ach / FP32_VECTOR_PEAK_TFLOPS, 4),
        "traffic": measured_traffic(w.name),
        "flops_per_launch": flops["bwd_main"],
        "flops_per_update": fl_bwd, "updates_per_launch": upd,
        "alg_bytes_per_launch": alg["bwd_main"],
        "hbm_GBs": kernels["bwd_main"]["GB/s"], "hbm_frac": kernels["bwd_main"]["hbm_frac"],
        "ms_per_launch": round(per["bwd_main"], 4),
    }

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(w, t, args.cpu_seconds)

    line = {
        "metric": METRIC, "value": float(f"{tc / (ms_per_step * 1e-3):.5g}"),
        "unit": "token*channels/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        # dtype: the arithmetic type of every step (state, transitions, sums); the activations
        # are stored in io_dtype
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "dim": w.dim, "dstate": w.dstate,
                   "seqlen": w.seqlen, "io_dtype": w.dtype,
                   "step": "fwd (with chunk-boundary states) + bwd"},
        "roofline": roofline, "kernels": kernels, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def graph_time(fn, per_graph, reps):
    """ms per call of `fn` (which only enqueues kernels): one call costs more host time than
    GPU time, so `per_graph` calls are captured in a HIP graph that is replayed `reps` times."""
    import torch
    for _ in range(5):
        fn()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for _ in range(per_graph):
                fn()
    torch.cuda.current_stream().wait_stream(side)
    graph.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(reps):
        graph.replay()
    ev[1].record()
    torch.cuda.synchronize()
    return ev[0].elapsed_time(ev[1]) / (per_graph * reps)


def cpu_baseline(w, t, min_seconds):
    """The fp64 oracle, as it stands: forward then backward over the whole workload, repeated
    until at least `min_seconds` have passed, on at most 16 of this host's cores."""
    import oracle
    v = {k: (None if t.get(k) is None else t.values(k)) for k in t}
    nthreads = min(16, oracle.default_threads())
    reps, el = 0, 0.0
    s = time.perf_counter()
    while el < min_seconds:
        oracle.fwd(v["u"], v["delta"], v["A"], v["B"], v["C"], v["D"], v["z"], v["bias"],
                   nthreads=nthreads)
        oracle.bwd(v["u"], v["delta"], v["A"], v["B"], v["C"], v["dout"], v["D"], v["z"],
                   v["bias"], nthreads=nthreads)
        reps += 1
        el = time.perf_counter() - s
    tcs = reps * w.batch * w.dim * w.seqlen
    return {"value": float(f"{tcs / el:.4g}"), "unit": "token*channels/s", "cores": nthreads,
            "kind": "oracle", "seconds": round(el, 3),
            "sample": f"{reps} x (fwd + bwd) over the whole workload: all {w.batch} batch rows, "
                      f"{w.dim} channels, seqlen {w.seqlen}, fp64"}


if __name__ == "__main__":
    main()
