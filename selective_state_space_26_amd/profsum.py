"""Summaries of rocprofv3 output for the scan kernels (part of the measurement harness).

    python -m selective_state_space_26_amd.profsum stats KERNEL_STATS_CSV OUT.md --command "..."
    python -m selective_state_space_26_amd.profsum traffic FETCH_CSV WRITE_CSV OUT.txt \\
        --kernel bwd_main_kernel [--match "bwd_main_kernel<msel::bf16_t, ..., false>"] \\
        --copy-mib 512 --workload NAME --command-fetch "..." --command-write "..."

`stats` turns a `--kernel-trace --stats` kernel_stats.csv into a short markdown table (with
`--trace KERNEL_TRACE_CSV`, also the busiest kernels split by launch grid).

`counters` turns `--pmc SQ_...` counter_collection.csv files (one per pass) into a per-kernel
table: the mean per dispatch of each counter and the ratios that say what bounds a kernel.

`traffic` reads two `--pmc FETCH_SIZE` / `--pmc WRITE_SIZE` counter_collection.csv files (KiB
per dispatch), takes the largest `copyBuffer` dispatch of the run (a plain device-to-device
copy of --copy-mib MiB that the bench makes before its steps) as the calibration of each
counter, and writes the HBM bytes per launch of --kernel: counter KiB x 1024 x (copy bytes /
copy counter bytes).  The file records the SHA-256 of the kernel's sources, so that readers
can tell when the counters no longer describe the code.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import os
import statistics
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BWD_SOURCES = ("selective_state_space_26_amd/csrc/scan_bwd.hip",
               "selective_state_space_26_amd/csrc/msel_device.hpp",
               "selective_state_space_26_amd/csrc/msel_kernels.hpp")
CONV_SOURCES = ("selective_state_space_26_amd/csrc/conv1d.hip",
                "selective_state_space_26_amd/csrc/msel_device.hpp",
                "selective_state_space_26_amd/csrc/msel_kernels.hpp")


FWD_SOURCES = ("selective_state_space_26_amd/csrc/scan_fwd.hip",
               "selective_state_space_26_amd/csrc/msel_device.hpp",
               "selective_state_space_26_amd/csrc/msel_kernels.hpp")
CC_SOURCES = ("selective_state_space_26_amd/csrc/chunk_carry.hip",
              "selective_state_space_26_amd/csrc/msel_device.hpp",
              "selective_state_space_26_amd/csrc/msel_kernels.hpp")


def sources_of(kernel: str):
    """The sources a kernel is built from (their digest goes into its traffic file)."""
    if kernel.startswith("conv_"):
        return CONV_SOURCES
    if kernel.startswith("scan_fwd"):
        return FWD_SOURCES
    if kernel.startswith("chunk_carry"):
        return CC_SOURCES
    return BWD_SOURCES


def source_digest(files=BWD_SOURCES) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def short_name(name: str) -> str:
    n = name.replace("(anonymous namespace)::", "")
    if n.startswith("void "):
        n = n[5:]
    return n.split("(")[0]


def stats(csv_path: str, out: str, command: str, trace_csv: str | None = None,
          top: int = 12) -> None:
    """The --stats table; with the kernel trace of the same run, also each of the `top`
    busiest kernels split by launch grid (one kernel serves several problem sizes in one run,
    and its per-size durations are what per-launch timings compare with)."""
    rows = list(csv.DictReader(open(csv_path)))
    lines = [f"# rocprofv3 kernel statistics: {os.path.basename(out)}", "",
             "Command (from the repository root on the GPU host):", "", "```", command, "```",
             "", "| kernel | calls | avg us | min us | max us | % of GPU time |",
             "|---|---:|---:|---:|---:|---:|"]
    for r in rows:
        lines.append(f"| `{short_name(r['Name'])}` | {r['Calls']} | "
                     f"{float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                     f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.2f} |")
    if trace_csv is not None:
        busiest = [r["Name"] for r in rows[:top]]
        groups = defaultdict(list)
        for r in csv.DictReader(open(trace_csv)):
            if r["Kernel_Name"] not in busiest:
                continue
            key = (r["Kernel_Name"], int(r["Grid_Size_X"]), int(r["Workgroup_Size_X"]))
            groups[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3)
        lines += ["", "The same run from its kernel trace, split by launch grid (threads in x, "
                  "workgroup size): one line per kernel and problem size.", "",
                  "| kernel | grid x | workgroup | calls | avg us | median us | min us | max us |",
                  "|---|---:|---:|---:|---:|---:|---:|---:|"]
        for name in busiest:
            for (n, gx, wx), us in sorted((k, v) for k, v in groups.items() if k[0] == name):
                lines.append(f"| `{short_name(n)}` | {gx} | {wx} | {len(us)} | "
                             f"{statistics.mean(us):.1f} | {statistics.median(us):.1f} | "
                             f"{min(us):.1f} | {max(us):.1f} |")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def _per_dispatch(csv_path: str, counter: str):
    """{kernel name: [value per dispatch]} for one counter (rows summed per dispatch)."""
    by = defaultdict(float)
    names = {}
    for r in csv.DictReader(open(csv_path)):
        if r["Counter_Name"] != counter:
            continue
        key = r["Dispatch_Id"]
        by[key] += float(r["Counter_Value"])
        names[key] = r["Kernel_Name"]
    out = defaultdict(list)
    for k, v in by.items():
        out[names[k]].append(v)
    return out


def traffic(fetch_csv, write_csv, out, kernel, copy_mib, workload, cmd_fetch, cmd_write,
            match=None):
    copy_bytes = copy_mib * (1 << 20)
    res = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        d = _per_dispatch(path, counter)
        copies = [v for name, vs in d.items() if "copyBuffer" in name for v in vs]
        if not copies:
            raise SystemExit(f"no copyBuffer dispatch in {path}")
        cal_kib = max(copies)
        factor = copy_bytes / (cal_kib * 1024.0)
        sel = match or kernel
        mine = [v for name, vs in d.items() if sel in name for v in vs]
        if not mine:
            raise SystemExit(f"no {kernel} dispatch in {path}")
        kib = statistics.mean(mine)
        res[counter] = dict(kib=kib, n=len(mine), cal_kib=cal_kib, factor=factor,
                            bytes=kib * 1024.0 * factor)
    total = res["FETCH_SIZE"]["bytes"] + res["WRITE_SIZE"]["bytes"]
    lines = [
        f"# HBM traffic of {kernel} on workload {workload}, from two rocprofv3 --pmc passes",
        f"# fetch pass: {cmd_fetch}",
        f"# write pass: {cmd_write}",
        "# counter KiB are per dispatch (mean over the dispatches of the kernel); each counter",
        f"# is scaled by a plain {copy_mib} MiB device copy read by the same counter",
        f"workload = {workload}",
        f"kernel = {kernel}",
        f"dispatch_name_contains = {match or kernel}",
        f"source_sha256 = {source_digest(sources_of(kernel))}",
    ]
    for c, r in res.items():
        lc = c.lower()
        lines += [f"{lc}_kib_per_dispatch = {r['kib']:.1f}",
                  f"{lc}_dispatches = {r['n']}",
                  f"{lc}_copy_kib = {r['cal_kib']:.1f}",
                  f"{lc}_copy_factor = {r['factor']:.4f}",
                  f"{lc}_bytes_per_launch = {r['bytes']:.0f}"]
    lines.append(f"traffic_bytes_per_launch = {total:.0f}")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def counters(csv_paths, out, selects, commands, clock_ghz=2.4, simds=1024):
    """Per selected kernel: mean per dispatch of every counter, and derived ratios.  SQ cycle
    counters are in quad-cycles (4 clocks), summed over the wavefronts; `simds` and
    `clock_ghz` turn them into a share of the SIMDs' time over the dispatch's duration."""
    vals = {n: defaultdict(lambda: defaultdict(float)) for n, _ in selects}
    durs = {n: {} for n, _ in selects}
    for path in csv_paths:
        for r in csv.DictReader(open(path)):
            name = next((n for n, sub in selects if sub in r["Kernel_Name"]), None)
            if name is None:
                continue
            key = (path, r["Dispatch_Id"])
            vals[name][r["Counter_Name"]][key] += float(r["Counter_Value"])
            durs[name][key] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    lines = [f"# rocprofv3 SQ counters: {os.path.basename(out)}", "",
             "Commands (from the repository root on the GPU host), one pass each:", "", "```",
             *commands, "```", "",
             "Mean per dispatch.  Cycle counters are quad-cycles summed over the wavefronts; "
             f"the SIMD shares assume {simds} SIMDs at {clock_ghz} GHz over the profiled "
             "dispatch's duration (which the profiler lengthens a little).", ""]
    for name, sub in selects:
        v = {c: statistics.mean(d.values()) for c, d in vals[name].items()}
        if not v:
            continue
        dur = statistics.mean(durs[name].values())
        lines += [f"## {name}", "", f"dispatches matching `{sub}`, mean duration "
                  f"{dur * 1e6:.1f} us", "", "| counter | per dispatch |", "|---|---:|"]
        lines += [f"| {c} | {x:.4g} |" for c, x in sorted(v.items())]
        waves = v.get("SQ_WAVES")
        quad = simds * dur * clock_ghz * 1e9 / 4.0
        derived = []
        if waves and "SQ_INSTS_VALU" in v:
            derived.append(("VALU instructions per wavefront", v["SQ_INSTS_VALU"] / waves))
        if "SQ_ACTIVE_INST_VALU" in v and "SQ_INSTS_VALU" in v:
            derived.append(("quad-cycles per VALU instruction",
                            v["SQ_ACTIVE_INST_VALU"] / v["SQ_INSTS_VALU"]))
        if "SQ_ACTIVE_INST_VALU" in v:
            derived.append(("share of SIMD time issuing VALU", v["SQ_ACTIVE_INST_VALU"] / quad))
        if "SQ_ACTIVE_INST_VALU2" in v:
            derived.append(("share of SIMD time dual-issuing VALU",
                            v["SQ_ACTIVE_INST_VALU2"] / quad))
        for c in ("SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_LDS"):
            if c in v and v.get("SQ_WAVE_CYCLES"):
                derived.append((f"{c} / SQ_WAVE_CYCLES", v[c] / v["SQ_WAVE_CYCLES"]))
        if derived:
            lines += ["", "| derived | value |", "|---|---:|"]
            lines += [f"| {k} | {x:.3f} |" if x < 100 else f"| {k} | {x:.0f} |"
                      for k, x in derived]
        lines.append("")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("out")
    s.add_argument("--command", required=True)
    s.add_argument("--trace", default=None, help="the run's kernel_trace.csv")
    t = sub.add_parser("traffic")
    t.add_argument("fetch_csv")
    t.add_argument("write_csv")
    t.add_argument("out")
    t.add_argument("--kernel", required=True)
    t.add_argument("--match", default=None,
                   help="substring that selects the dispatches (default: --kernel), e.g. one "
                        "template instantiation")
    t.add_argument("--copy-mib", type=int, required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--command-fetch", required=True)
    t.add_argument("--command-write", required=True)
    k = sub.add_parser("counters")
    k.add_argument("csv", nargs="+")
    k.add_argument("--out", required=True)
    k.add_argument("--select", action="append", required=True,
                   help="NAME=SUBSTRING of the dispatch names to summarise (repeatable)")
    k.add_argument("--command", action="append", required=True,
                   help="the command of each pass (repeatable)")
    a = ap.parse_args()
    if a.cmd == "counters":
        counters(a.csv, a.out, [tuple(x.split("=", 1)) for x in a.select], a.command)
    elif a.cmd == "stats":
        stats(a.csv, a.out, a.command, a.trace)
    else:
        traffic(a.fetch_csv, a.write_csv, a.out, a.kernel, a.copy_mib, a.workload,
                a.command_fetch, a.command_write, a.match)


if __name__ == "__main__":
    main()
