"""Benchmark of the selective scan on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2] [--no-cpu] [--no-extra]

A step is one pass of the whole hot path over one batch of synthetic input resident in HBM:
the fused forward scan (out, final state and the state at every chunk boundary), then the
backward with recomputation (all gradients): it rebuilds every state inside the chunks from
those boundary states and runs the chunk carry backward for the adjoint.  Consecutive steps
take consecutive copies of the inputs, from a ring of copies larger than the chip's 256 MB
last-level cache (MALL), so that each step's forward reads its inputs from HBM.  The timed
steps follow an untimed clock ramp (--ramp-ms, 300 ms of the same step) and the W warmup
steps, all back to back, so that they run at the clocks the chip holds under sustained load
(after the setup's idle time the first steps run ~10% slower).  The K timed steps carry no
events; K more steps with HIP events around each pass give the per-kernel times.  The default
workload is batch 8, d_model 768 x expand 2 = 1536 channels, dstate 16, seqlen 2048, bf16
activations with fp32 state -- the workload that runs both the forward and the backward.

Besides the step it measures, each with a cold last-level cache (a 512 MiB copy before every
launch) and reported as median / p10 / p90 over the launches:
  * the forward, the gradient kernel and the chunk-carry pass of the step's workload alone;
  * the same passes at the other workloads' full sizes: the selective-copying shape (fp32
    forward), the 64k-step bf16 forward (chunk carry across 128 chunks) and the fp32 backward
    with recomputed chunk states;
  * the variants at the step's shape: the recurrent (decode) step, the exponential-trapezoidal
    and complex forwards and backwards, and the short causal convolution + SiLU (width 4).

Prints one JSON line: the whole-step throughput in token*channels/s, the HBM roofline of the
dominant kernel (from HIP events on its launch stream over the timed steps), per-kernel
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
# VALU issue of the chip: one wave64 instruction per SIMD every 4 clocks (16 lanes per clock),
# 1024 SIMDs at 2.4 GHz = 39.3 T lane-instructions/s; the scan kernels issue VALU
# instructions one at a time (their dual-issue share is ~13% by the SQ counters)
VALU_ISSUE_PEAK = 1024 * 16 * 2.4e9
METRIC = "selective-scan fwd/bwd tokens·channels/s and achieved HBM GB/s (% of peak)"
# The least VALU work per (batch, channel, time, state) update that the recurrence itself
# needs, in instructions (each exp is one instruction): the forward Delta*A, exp, (Delta u)*B,
# h = a h + p, y += C h; the backward recomputes h (4), runs the adjoint lam = a lam + C dy (2),
# forms g = lam h a (2), and adds into dA, dDelta, sum(lam B), dB, dC (5), plus y += C h for
# the gate's dz (1).
VALU_FLOOR_FWD = 5
VALU_FLOOR_BWD = 13
VALU_FLOOR_BWD_Z = 1
CONV_WIDTH = 4     # taps of the short causal convolution before the scan
CACHE_BYTES = 256 << 20   # MI355X last-level cache (MALL)
FLUSH_MIB = 512           # a copy of this size before every cold launch evicts it
COLD_REPS = 10
# rocprofv3 FETCH_SIZE / WRITE_SIZE summaries, per kernel, of the default workload
TRAFFIC_FILE = "profiles/{kernel}_d768x2_bf16_traffic.txt"


def algorithmic_bytes(w, nchunks, dtype_bytes=None, fused=False):
    """Bytes each pass must move at least once between HBM and the chip.  fused: the backward
    takes its fused plan (its gradient kernel reads the chunk states, not the adjoint carries
    of a link pass)."""
    s = dtype_bytes or (2 if w.dtype == "bf16" else 4)
    tc = w.batch * w.dim * w.seqlen
    bnl = w.batch * w.dstate * w.seqlen
    states = w.batch * w.dim * nchunks * w.dstate * 4
    dn, d = w.dim * w.dstate, w.dim
    # u, delta, z in, out out; B, C in; final state out; A, D, bias in.  The chunk states the
    # forward also writes are implementation overhead (0.4-3% of it) and are not counted.
    fwd = 4 * tc * s + 2 * bnl * s + w.batch * w.dim * w.dstate * 4 + dn * 4 + 2 * d * 4
    # u, delta in; B in; A, bias in; chunk states out (the pass's product)
    cc = 2 * tc * s + bnl * s + states + dn * 4 + d * 4
    # the whole backward: u, delta, dout, z in; du, ddelta, dz out; B, C in; dB, dC out
    # (fp32); A, D, bias in; dA, dD, dbias out.  The gradient kernel alone moves the same
    # tensors, plus the chunk-start states (and with the chunk-parallel plan the adjoint
    # carries) it reads, counted for it.  The fused plan's partial sums are not counted.
    bwd = 7 * tc * s + 2 * bnl * s + 2 * bnl * 4 + 2 * dn * 4 + 4 * d * 4
    bwd_main = bwd + (1 if fused else 2) * states
    return {"fwd": fwd, "chunk_carry": cc, "bwd_main": bwd_main, "bwd": bwd}


def measured_traffic(workload_name, kernel):
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
    ap.add_argument("--ramp-ms", type=float, default=300.0,
                    help="run the step untimed for this long before the warmup steps, so that "
                         "the GPU's clocks reach their level under sustained load")
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extra", action="store_true",
                    help="time only the step (no cold per-kernel, variant or other-workload "
                         "timings): for profiler runs")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the oracle over the whole workload for at least this long")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="before the steps, copy a buffer of this many MiB once (a plain copy "
                         "kernel of known size that scales the HBM byte counters)")
    return ap.parse_args()


def summary(ms):
    """mean / median / p10 / p90 of a list of per-launch times in ms."""
    import numpy as np
    a = np.asarray(ms, dtype=np.float64)
    return {"mean": float(a.mean()), "median": float(np.median(a)),
            "p10": float(np.percentile(a, 10)), "p90": float(np.percentile(a, 90)),
            "n": int(a.size)}


def entry(st, alg_bytes, tcs, what, updates=None, valu_floor=None, basis="median"):
    """A kernels[...] record: times, and the algorithmic GB/s and tc/s at the `basis` time."""
    ms = st[basis]
    sec = ms * 1e-3
    gbs = alg_bytes / sec / 1e9
    e = {"ms": round(ms, 4), "ms_basis": basis,
         "ms_stats": {k: (round(v, 4) if isinstance(v, float) else v) for k, v in st.items()},
         "alg_bytes": int(alg_bytes), "GB/s": round(gbs, 1),
         "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "tc_per_s": float(f"{tcs / sec:.4g}"),
         "what": what}
    if updates is not None and valu_floor is not None:
        floor_s = updates * valu_floor / VALU_ISSUE_PEAK
        e["valu_issue"] = {"floor_instr_per_update": valu_floor, "floor_ms": round(floor_s * 1e3, 4),
                           "frac": round(floor_s / sec, 4)}
    return e


class Ctx:
    """Device, dtype and the helpers every timing below uses."""

    def __init__(self, torch, np, dev):
        self.torch, self.np, self.dev = torch, np, dev
        n = FLUSH_MIB * (1 << 20) // 4
        self.flush_src = torch.ones(n, device=dev, dtype=torch.float32)
        self.flush_dst = torch.empty_like(self.flush_src)

    def put(self, v, dt):
        torch, np = self.torch, self.np
        if v is None:
            return None
        if v.dtype == np.uint16:
            return torch.from_numpy(v.view(np.int16)).to(self.dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(v)).to(device=self.dev, dtype=dt)

    def device_inputs(self, t, dtype):
        torch = self.torch
        act = torch.bfloat16 if dtype == "bf16" else torch.float32
        return {k: self.put(v, act if k in ("u", "delta", "z", "B", "C", "dout", "lam")
                            else torch.float32) for k, v in t.items()}

    def flush(self):
        """Evict the last-level cache: a 512 MiB copy (reads and writes twice its size)."""
        self.flush_dst.copy_(self.flush_src)

    def cold(self, fn, reps=COLD_REPS, events=None):
        """Per-launch ms of fn() (which enqueues on the current stream), each launch after a
        cache flush.  events(): optional pair of events fn records itself (the gradient
        kernel's), else the events bracket the whole call."""
        torch = self.torch
        fn()  # warm the code path
        out = []
        for _ in range(reps):
            self.flush()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            if events is None:
                ev[0].record()
                fn()
                ev[1].record()
            else:
                for e in ev:
                    e.record()
                fn(ev)
            torch.cuda.synchronize()
            out.append(ev[0].elapsed_time(ev[1]))
        return summary(out)


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
    cx = Ctx(torch, np, dev)
    t = msel_inputs.make_workload(w, with_dout=True)
    d0 = cx.device_inputs(t, w.dtype)
    nch = msel.num_chunks(w.seqlen)
    s_ = 2 if w.dtype == "bf16" else 4
    tc = w.batch * w.dim * w.seqlen
    upd = tc * w.dstate
    fused = msel.bwd_fused(d0["u"], d0["A"], True)  # the plan the step's backward takes
    alg = algorithmic_bytes(w, nch, fused=fused)

    # a ring of input copies, together more than twice the last-level cache
    streamed = ("u", "delta", "z", "dout", "B", "C")
    set_bytes = sum(d0[k].numel() * d0[k].element_size() for k in streamed if d0[k] is not None)
    nsets = max(2, min(8, -(-3 * CACHE_BYTES // set_bytes)))
    sets = [d0] + [{k: (v.clone() if k in streamed and v is not None else v)
                    for k, v in d0.items()} for _ in range(nsets - 1)]
    for s in sets:
        s["out"] = torch.empty_like(d0["u"])
        s["fin"] = torch.empty(w.batch, w.dim, w.dstate, device=dev, dtype=torch.float32)
        s["cs"] = torch.empty(w.batch, w.dim, nch, w.dstate, device=dev, dtype=torch.float32)
    ws = torch.empty(msel.bwd_workspace_bytes(d0["u"], d0["A"], True), device=dev,
                     dtype=torch.uint8)

    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, device=dev, dtype=torch.float32)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def fwd(s):
        return msel.msel_scan_fwd(s["u"], s["delta"], s["A"], s["B"], s["C"], s["D"], s["z"],
                                  s["bias"], True, out=s["out"], final_state=s["fin"],
                                  chunk_states=s["cs"], return_chunk_states=True)

    def bwd(s, main_events=None, states=True):
        return msel.msel_scan_bwd(s["u"], s["delta"], s["A"], s["B"], s["C"], s["dout"], s["D"],
                                  s["z"], s["bias"], True, chunk_states=s["cs"] if states else None,
                                  workspace=ws, main_events=main_events)

    def new_events(k):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(k)]
        for e in ev:   # the library records the gradient-kernel events itself: create them
            e.record()
        return ev

    def step(k, ev=None):
        """fwd (out, final state, one state per chunk) then bwd, which recomputes every state
        inside the chunks and runs the chunk carry backward for the adjoint, on input copy
        k mod nsets.  All launches go to torch's current stream, on which the events are
        recorded."""
        s = sets[k % nsets]
        if ev is not None:
            ev[0].record()
        fwd(s)
        if ev is not None:
            ev[1].record()
        g = bwd(s, None if ev is None else (ev[3], ev[4]))
        if ev is not None:
            ev[2].record()
        return g

    # Clock ramp: the GPU's power management raises its clocks only under sustained load; a
    # step started from idle (setup above, or a few ms of host work between steps) runs about
    # 10% slower than the same step among back-to-back ones.  So the step first runs untimed
    # for ramp_ms, then the W warmup steps, then the K timed ones, all back to back.
    ramp_steps = 0
    t_ramp = time.perf_counter()
    while (time.perf_counter() - t_ramp) * 1e3 < args.ramp_ms:
        for _ in range(8):
            step(ramp_steps)
            ramp_steps += 1
        torch.cuda.synchronize()
    for k in range(args.warmup):
        step(ramp_steps + k)
    # The timed steps: the host clock around K back-to-back steps with nothing else on the
    # stream.  Then the same K steps again with HIP events around each pass and the gradient
    # kernel, for the per-kernel figures and the roofline: each event record costs the stream
    # ~3 us between kernels, so the events stay out of the headline steps.
    k0 = ramp_steps + args.warmup
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(k0 + k)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    evs = [new_events(5) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for k in range(args.steps):
        step(k0 + args.steps + k, evs[k])
    torch.cuda.synchronize()
    ms_per_step_events = (time.perf_counter() - t2) * 1e3 / args.steps
    step_ms = {
        "fwd": summary([e[0].elapsed_time(e[1]) for e in evs]),
        "bwd": summary([e[1].elapsed_time(e[2]) for e in evs]),
        "bwd_main": summary([e[3].elapsed_time(e[4]) for e in evs]),
    }
    vf_bwd = VALU_FLOOR_BWD + (VALU_FLOOR_BWD_Z if d0.get("z") is not None else 0)
    kernels = {
        "fwd": entry(step_ms["fwd"], alg["fwd"], tc, "scan_fwd_kernel in the step (one launch)",
                     upd, VALU_FLOOR_FWD),
        "bwd": entry(step_ms["bwd"], alg["bwd"], tc, "the msel_scan_bwd call in the step: " +
                     ("the fused bwd_main_kernel and bwd_reduce_kernel" if fused else
                      "zero-fills, summary, link and bwd_main_kernel")),
        "bwd_main": entry(step_ms["bwd_main"], alg["bwd_main"], tc,
                          "bwd_main_kernel in the step, " +
                          ("the fused gradient kernel (chunks walked last to first)" if fused
                           else "the chunk-parallel gradient kernel"), upd, vf_bwd),
    }
    for k in ("fwd", "bwd_main"):
        kernels[k]["traffic"] = measured_traffic(
            w.name, "scan_fwd_kernel" if k == "fwd" else "bwd_main_kernel")

    # the dominant kernel of the step: its HBM roofline from the timed steps' mean launch
    # duration (the figure rocprofv3's kernel-trace average is compared with)
    dom = max(("fwd", "bwd_main"), key=lambda k: step_ms[k]["mean"])
    dsec = step_ms[dom]["mean"] * 1e-3
    dbytes = alg[dom]
    ach = dbytes / dsec / 1e9
    vfloor = VALU_FLOOR_FWD if dom == "fwd" else vf_bwd
    roofline = {
        "kernel": "scan_fwd_kernel" if dom == "fwd" else "bwd_main_kernel",
        "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(ach / HBM_PEAK_GBS, 4),
        "traffic": kernels[dom]["traffic"],
        "alg_bytes_per_launch": dbytes, "ms_per_launch_mean": round(step_ms[dom]["mean"], 4),
        "ms_per_launch_median": round(step_ms[dom]["median"], 4),
        "valu_issue": {"floor_instr_per_update": vfloor, "updates_per_launch": upd,
                       "peak_lane_instr_per_s": VALU_ISSUE_PEAK,
                       "frac": round(upd * vfloor / VALU_ISSUE_PEAK / dsec, 4)},
    }

    extra = {}
    if not args.no_extra:
        extra = extra_timings(cx, msel, msel_inputs, w, sets, nsets, alg, tc, upd, vf_bwd, ws,
                              fwd, bwd, args)
    else:  # the chunk-carry pass alone, a few launches (profiler runs count its bytes too)
        s0 = sets[0]
        extra["chunk_carry_cold"] = entry(
            cx.cold(lambda: msel.msel_scan_chunk_carry(s0["u"], s0["delta"], s0["A"], s0["B"],
                                                       s0["bias"], True, chunk_states=s0["cs"],
                                                       final_state=s0["fin"]), reps=3),
            alg["chunk_carry"], tc, "chunk_carry_kernel (one launch) after a cache flush")
    for k in ("chunk_carry_cold",):
        if k in extra:
            extra[k]["traffic"] = measured_traffic(w.name, "chunk_carry_kernel")
    kernels.update(extra)

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(w, t, args.cpu_seconds)

    line = {
        "metric": METRIC, "value": float(f"{tc / (ms_per_step * 1e-3):.5g}"),
        "unit": "token*channels/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "clock_ramp": {"ms": args.ramp_ms, "steps": ramp_steps},
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        # the same steps timed again with the per-kernel HIP events on the stream
        "ms_per_step_with_events": round(ms_per_step_events, 4),
        # dtype: the arithmetic type of every step (state, transitions, sums); the activations
        # are stored in io_dtype
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "dim": w.dim, "dstate": w.dstate,
                   "seqlen": w.seqlen, "io_dtype": w.dtype,
                   "step": "fwd (with chunk-boundary states) + bwd",
                   "bwd_plan": "fused" if fused else "chunk-parallel",
                   "input_copies": nsets, "input_copy_bytes": int(set_bytes)},
        "roofline": roofline, "kernels": kernels, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def extra_timings(cx, msel, msel_inputs, w, sets, nsets, alg, tc, upd, vf_bwd, ws, fwd, bwd,
                  args):
    """Cold-cache per-kernel timings of the step's passes, the other workloads and the
    variants."""
    torch, np = cx.torch, cx.np
    dev = cx.dev
    s_ = 2 if w.dtype == "bf16" else 4
    nch = msel.num_chunks(w.seqlen)
    k = {}
    s = sets[0]
    k["fwd_cold"] = entry(cx.cold(lambda: fwd(s)), alg["fwd"], tc,
                          "scan_fwd_kernel, one launch after a 512 MiB cache flush", upd,
                          VALU_FLOOR_FWD)
    k["bwd_main_cold"] = entry(cx.cold(lambda ev=None: bwd(s, None if ev is None else ev),
                                       events=True),
                               alg["bwd_main"], tc, "bwd_main_kernel, one launch after a "
                               "512 MiB cache flush", upd, vf_bwd)
    k["chunk_carry_cold"] = entry(
        cx.cold(lambda: msel.msel_scan_chunk_carry(s["u"], s["delta"], s["A"], s["B"], s["bias"],
                                                   True, chunk_states=s["cs"],
                                                   final_state=s["fin"])),
        alg["chunk_carry"], tc, "chunk_carry_kernel (one launch) after a cache flush")

    # the other workloads at their full sizes
    for wid, passes in ((1, ("fwd", "chunk_carry", "bwd")), (3, ("fwd", "chunk_carry", "bwd")),
                        (4, ("fwd", "bwd"))):
        if wid == args.workload:
            continue
        ow = msel_inputs.WORKLOADS[wid]
        od = device_workload(torch, ow, dev)
        onch = msel.num_chunks(ow.seqlen)
        otc = ow.batch * ow.dim * ow.seqlen
        oupd = otc * ow.dstate
        # the backward as that workload's description asks: chunk states rebuilt by the
        # backward (workload 4: "no stored intermediate states"), else the forward's
        given = wid != 4
        oalg = algorithmic_bytes(ow, onch, fused=given and msel.bwd_fused(od["u"], od["A"], True))
        od["out"] = torch.empty_like(od["u"])
        od["fin"] = torch.empty(ow.batch, ow.dim, ow.dstate, device=dev, dtype=torch.float32)
        od["cs"] = torch.empty(ow.batch, ow.dim, onch, ow.dstate, device=dev,
                               dtype=torch.float32)
        ows = torch.empty(max(msel.bwd_workspace_bytes(od["u"], od["A"], False),
                              msel.bwd_workspace_bytes(od["u"], od["A"], True)), device=dev,
                          dtype=torch.uint8)
        tag = f"w{wid}"
        shape = f"{ow.batch}x{ow.dim}x{ow.dstate}x{ow.seqlen} {ow.dtype}"

        def ofwd():
            msel.msel_scan_fwd(od["u"], od["delta"], od["A"], od["B"], od["C"], od["D"],
                               od["z"], od["bias"], True, out=od["out"], final_state=od["fin"],
                               chunk_states=od["cs"], return_chunk_states=True)
        k[f"fwd_{tag}"] = entry(cx.cold(ofwd), oalg["fwd"], otc,
                                f"scan_fwd_kernel at workload {wid} ({ow.name}, {shape}), "
                                "cold cache", oupd, VALU_FLOOR_FWD)
        k[f"fwd_{tag}"]["workload"] = ow.name
        if "chunk_carry" in passes:
            k[f"chunk_carry_{tag}"] = entry(
                cx.cold(lambda: msel.msel_scan_chunk_carry(
                    od["u"], od["delta"], od["A"], od["B"], od["bias"], True,
                    chunk_states=od["cs"], final_state=od["fin"])),
                oalg["chunk_carry"], otc, f"chunk_carry_kernel at workload {wid}, cold cache")
        ofwd()

        def obwd(ev=None):
            msel.msel_scan_bwd(od["u"], od["delta"], od["A"], od["B"], od["C"], od["dout"],
                               od["D"], od["z"], od["bias"], True,
                               chunk_states=od["cs"] if given else None, workspace=ows,
                               main_events=ev)
        vfb = VALU_FLOOR_BWD + VALU_FLOOR_BWD_Z
        k[f"bwd_main_{tag}"] = entry(cx.cold(obwd, events=True), oalg["bwd_main"], otc,
                                     f"bwd_main_kernel at workload {wid}, cold cache", oupd, vfb)
        k[f"bwd_{tag}"] = entry(cx.cold(obwd), oalg["bwd"], otc,
                                f"the msel_scan_bwd call at workload {wid}, chunk states "
                                f"{'from the forward' if given else 'rebuilt (none stored)'}, "
                                "cold cache")
        del od, ows
        torch.cuda.empty_cache()

    # the recurrent (decode) step at the same batch and channels: seqlen 1, state in place
    d = sets[0]
    st = {k_: (None if v is None else (v[..., :1].contiguous() if k_ in ("u", "delta", "z", "B", "C")
                                        else v)) for k_, v in d.items()
          if k_ not in ("out", "fin", "cs")}
    state = torch.zeros(w.batch, w.dim, w.dstate, device=dev, dtype=torch.float32)
    dec_out = torch.empty_like(st["u"])

    def decode():
        msel.msel_scan_fwd(st["u"], st["delta"], st["A"], st["B"], st["C"], st["D"], st["z"],
                           st["bias"], True, state, out=dec_out, final_state=state)
    dec_ms = graph_time(torch, decode, 32, 10)
    dec_bytes = (2 * w.batch * w.dim * w.dstate * 4 + 4 * w.batch * w.dim * s_ +
                 2 * w.batch * w.dstate * s_ + w.dim * w.dstate * 4 + 2 * w.dim * 4)
    k["decode_step"] = entry({"mean": dec_ms, "median": dec_ms, "p10": dec_ms, "p90": dec_ms,
                              "n": 320}, dec_bytes, w.batch * w.dim,
                             "scan_step_kernel: one recurrent step (seqlen 1) of every channel, "
                             "state updated in place; mean over 320 steps replayed from HIP "
                             "graphs")

    # the exponential-trapezoidal and complex variants at the same shape, cold cache
    lam = cx.put(msel_inputs.make(w.batch, w.dim, w.dstate, w.seqlen, w.dtype, w.seed,
                                  with_lam=True)["lam"],
                 torch.bfloat16 if w.dtype == "bf16" else torch.float32)
    cs2 = torch.empty_like(d["cs"])
    fin2 = torch.empty_like(d["fin"])
    out2 = torch.empty_like(d["u"])
    vws = torch.empty(msel.bwd_workspace_bytes(d["u"], d["A"], True), device=dev,
                      dtype=torch.uint8)

    def trap_fwd():
        msel.msel_scan_trap_fwd(d["u"], d["delta"], lam, d["A"], d["B"], d["C"], d["D"], d["z"],
                                d["bias"], True, out=out2, final_state=fin2, chunk_states=cs2)

    def trap_bwd():
        msel.msel_scan_trap_bwd(d["u"], d["delta"], lam, d["A"], d["B"], d["C"], d["dout"], cs2,
                                d["D"], d["z"], d["bias"], True, workspace=vws)
    k["trap_fwd"] = entry(cx.cold(trap_fwd), alg["fwd"] + tc * s_, tc,
                          "scan_fwd_kernel with the exponential-trapezoidal rule "
                          "(msel_scan_trap_fwd, lambda as one more input), cold cache")
    trap_fwd()
    k["trap_bwd"] = entry(cx.cold(trap_bwd), alg["bwd"] + 2 * tc * s_, tc,
                          "the msel_scan_trap_bwd call (zero-fills, summary, link and the "
                          "trapezoidal gradient kernel), cold cache")
    cA = cx.put(msel_inputs.make(1, w.dim, w.dstate, 1, "f32", w.seed, complex_A=True)["A"],
                torch.float32)

    def complex_fwd():
        msel.msel_scan_complex_fwd(d["u"], d["delta"], cA, d["B"], d["C"], d["D"], d["z"],
                                   d["bias"], True, out=out2, final_state=fin2,
                                   chunk_states=cs2)

    def complex_bwd():
        msel.msel_scan_complex_bwd(d["u"], d["delta"], cA, d["B"], d["C"], d["dout"], cs2,
                                   d["D"], d["z"], d["bias"], True, workspace=vws)
    k["complex_fwd"] = entry(cx.cold(complex_fwd), alg["fwd"], tc,
                             "scan_cplx_fwd_kernel: the complex-valued (rotational) forward, "
                             "dstate 16 as 8 complex states, cold cache")
    complex_fwd()
    k["complex_bwd"] = entry(cx.cold(complex_bwd), alg["bwd"], tc,
                             "the msel_scan_complex_bwd call (zero-fills, summary, link and the "
                             "pair-ring gradient kernel), cold cache")
    del vws, out2

    # the short causal convolution + SiLU that makes the scan's input, at the same batch,
    # channels, length and dtype, width 4, with bias and incoming state
    cv = {k_: cx.put(v, (torch.bfloat16 if w.dtype == "bf16" else torch.float32)
                     if k_ in ("x", "state", "dout") else torch.float32)
          for k_, v in msel_inputs.make_conv(w.batch, w.dim, w.seqlen, CONV_WIDTH, w.dtype,
                                             w.seed, with_state=True, with_dout=True).items()}
    cout = torch.empty_like(cv["x"])
    cst = torch.empty_like(cv["state"])
    rows = w.batch * w.dim
    H = CONV_WIDTH - 1

    def conv_fwd():
        msel.msel_conv1d_fwd(cv["x"], cv["weight"], cv["bias"], cv["state"], out=cout,
                             state_out=cst)

    def conv_bwd():
        msel.msel_conv1d_bwd(cv["x"], cv["weight"], cv["dout"], cv["bias"], cv["state"],
                             want_dstate=True)
    conv_bytes = {
        "conv_fwd": 2 * tc * s_ + 2 * rows * H * s_ + w.dim * (CONV_WIDTH + 1) * 4,
        "conv_bwd": 3 * tc * s_ + rows * H * (s_ + 4) + 2 * w.dim * (CONV_WIDTH + 1) * 4,
        "conv_decode_step": 2 * rows * s_ + 2 * rows * H * s_ + w.dim * (CONV_WIDTH + 1) * 4,
    }
    k["conv_fwd"] = entry(cx.cold(conv_fwd), conv_bytes["conv_fwd"], tc,
                          "conv_fwd_kernel: causal depthwise conv (width 4) + bias + SiLU, "
                          "state in and out (one launch), cold cache")
    k["conv_bwd"] = entry(cx.cold(conv_bwd), conv_bytes["conv_bwd"], tc,
                          "the msel_conv1d_bwd call: zero-fill of the tap/bias gradients and "
                          "conv_bwd_kernel (recomputes the activation), cold cache")
    for n in ("conv_fwd", "conv_bwd"):
        k[n]["traffic"] = measured_traffic(w.name, n + "_kernel")
    cx1 = cv["x"][..., :1].contiguous()
    cache = cv["state"].clone()
    conv_dec_out = torch.empty_like(cx1)

    def conv_decode():
        msel.msel_conv1d_fwd(cx1, cv["weight"], cv["bias"], cache, out=conv_dec_out,
                             state_out=cache)
    cd_ms = graph_time(torch, conv_decode, 32, 10)
    k["conv_decode_step"] = entry({"mean": cd_ms, "median": cd_ms, "p10": cd_ms, "p90": cd_ms,
                                   "n": 320}, conv_bytes["conv_decode_step"], rows,
                                  "conv_step_kernel: msel_conv1d_fwd at seqlen 1 with the state "
                                  "updated in place; mean over 320 steps replayed from HIP "
                                  "graphs")
    return k


def device_workload(torch, w, dev):
    """A workload's inputs drawn on the device with a seeded torch generator, in the input
    recipe's distributions (u, z, dout, B, C, D ~ N(0,1); delta = 0.5 N(0,1); bias =
    log(expm1(U[1e-3, 1e-1])); A[d, n] = -(n+1)), rounded to nearest-even bf16 where the
    workload is bf16.  For timing only: the kernels' work does not depend on the values, and
    drawing the 64k-step workload on the host would take half a minute."""
    g = torch.Generator(device=dev)
    g.manual_seed(1000 + w.seed)
    act = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    f32 = dict(device=dev, dtype=torch.float32, generator=g)

    def normal(shape, scale=1.0):
        return (torch.randn(shape, **f32) * scale).to(act)
    x = {"u": normal((w.batch, w.dim, w.seqlen)), "delta": normal((w.batch, w.dim, w.seqlen), 0.5),
         "z": normal((w.batch, w.dim, w.seqlen)), "dout": normal((w.batch, w.dim, w.seqlen)),
         "B": normal((w.batch, w.dstate, w.seqlen)), "C": normal((w.batch, w.dstate, w.seqlen))}
    x["D"] = torch.randn(w.dim, **f32)
    x["bias"] = torch.log(torch.expm1(torch.rand(w.dim, **f32) * (1e-1 - 1e-3) + 1e-3))
    x["A"] = (-(torch.arange(w.dstate, device=dev, dtype=torch.float32) + 1.0)).expand(
        w.dim, w.dstate).contiguous()
    return x


def graph_time(torch, fn, per_graph, reps):
    """ms per call of `fn` (which only enqueues kernels): one call costs more host time than
    GPU time, so `per_graph` calls are captured in a HIP graph that is replayed `reps` times."""
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


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, t, min_seconds):
    """The fp64 oracle, as it stands: forward then backward over the whole workload, repeated
    until at least `min_seconds` have passed, on the host threads this process may use (at most
    16, the host share of one GPU on the GPU hosts); and the same on one thread over a slice of
    the workload (one batch row, a sixteenth of its channels), scaled by token*channels."""
    import oracle
    v = {k: (None if t.get(k) is None else t.values(k)) for k in t}
    nthreads = min(16, oracle.default_threads())

    def run(vv, threads, secs):
        reps, el = 0, 0.0
        s = time.perf_counter()
        while el < secs:
            oracle.fwd(vv["u"], vv["delta"], vv["A"], vv["B"], vv["C"], vv["D"], vv["z"],
                       vv["bias"], nthreads=threads)
            oracle.bwd(vv["u"], vv["delta"], vv["A"], vv["B"], vv["C"], vv["dout"], vv["D"],
                       vv["z"], vv["bias"], nthreads=threads)
            reps += 1
            el = time.perf_counter() - s
        return reps, el

    reps, el = run(v, nthreads, min_seconds)
    tcs = reps * w.batch * w.dim * w.seqlen
    nd = max(1, w.dim // 16)
    sl = {k: (None if x is None else x) for k, x in v.items()}
    for k in ("u", "delta", "z", "dout"):
        sl[k] = v[k][:1, :nd]
    for k in ("B", "C"):
        sl[k] = v[k][:1]
    for k in ("A", "D", "bias"):
        sl[k] = None if v[k] is None else v[k][:nd]
    r1, e1 = run(sl, 1, min(3.0, min_seconds))
    tc1 = r1 * nd * w.seqlen
    return {"value": float(f"{tcs / el:.4g}"), "unit": "token*channels/s", "cores": nthreads,
            "kind": "oracle", "seconds": round(el, 3),
            "sample": f"{reps} x (fwd + bwd) over the whole workload: all {w.batch} batch rows, "
                      f"{w.dim} channels, seqlen {w.seqlen}, fp64",
            "host_cpus_visible": os.cpu_count(), "cpu_model": _cpu_model(),
            "one_thread": {"value": float(f"{tc1 / e1:.4g}"), "unit": "token*channels/s",
                           "seconds": round(e1, 3),
                           "sample": f"{r1} x (fwd + bwd) over batch row 0, channels 0..{nd - 1},"
                                     f" seqlen {w.seqlen}, fp64, one thread"}}


if __name__ == "__main__":
    main()
