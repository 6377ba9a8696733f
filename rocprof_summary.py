"""Summarise rocprofv3 CSV output of ``bench.py`` runs into the short text files under profiles/.

Two modes, both reading only what rocprofv3 wrote:

* ``trace DIR``: the ``*kernel_stats.csv`` of a ``--kernel-trace --stats`` run becomes a table
  of calls and average / min / max duration per kernel, plus the decode kernel's algorithmic
  bandwidth (bytes per call taken from the bench JSON line the same run printed).
* ``sq DIR [DIR ...]``: the ``*counter_collection.csv`` of shader-sequencer counter passes
  (``SQ_*`` and ``GRBM_GUI_ACTIVE``) become per-dispatch medians for the dominant kernel and
  the ratios read from them: instructions per wave and per KiB (or per GFLOP), the matrix-core
  and vector-ALU issue shares, the LDS bank-conflict share, and how the waves' time splits into
  issuing, waiting to issue and waiting on memory or barriers.
* ``traffic FETCH_DIR WRITE_DIR``: the ``*counter_collection.csv`` of a ``--pmc FETCH_SIZE``
  run and of a ``--pmc WRITE_SIZE`` run (both with ``bench.py --calibrate``) become HBM bytes
  per dispatch. Each counter is scaled by what it reads for the calibration copy (a plain
  256 MiB device-to-device copy: 256 MiB read and 256 MiB written), and the dominant kernel's
  figure goes to a JSON file that ``bench.py`` reports as ``roofline.traffic`` while the
  kernel sources still hash the same.

Usage (from the repository root):

    python rocprof_summary.py trace <dir> --bench-log <log> --command "<cmd>" --out <md>
    python rocprof_summary.py traffic <fetch_dir> <write_dir> --bench-log <log> \\
        --command "<fetch cmd>" --command "<write cmd>" --out <md> --json <json>
    python rocprof_summary.py sq <dir_a> <dir_b> --bench-log <log> --kernel <name prefix> \\
        --command "<cmd a>" --command "<cmd b>" --out <md>
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
CALIB_BYTES = 2 ** 28  # the calibration copy: 256 MiB read, 256 MiB written


def find_one(d: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not hits:
        sys.exit(f"no *{suffix} under {d}")
    return hits[0]


def bench_line(path: str) -> dict:
    lines = [ln for ln in open(path) if ln.startswith("{")]
    if not lines:
        sys.exit(f"no JSON line in {path}")
    return json.loads(lines[-1])


def short(name: str, n: int = 60) -> str:
    name = name.replace("pa::(anonymous namespace)::", "").replace("(pa::DecodeParams)", "")
    name = name.replace("(pa::PrefillParams)", "")
    if name.startswith("void "):
        name = name[5:]
    return name if len(name) <= n else name[: n - 3] + "..."


def is_dominant(name: str, prefix: str) -> bool:
    return short(name, 1000).startswith(prefix)


def trace(args) -> None:
    stats = find_one(args.dirs[0], "kernel_stats.csv")
    rows = list(csv.DictReader(open(stats)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    b = bench_line(args.bench_log)
    roof = b["roofline"]
    wl = b["config"]["workload"].split(":")[0]
    out = [f"# Kernel trace: {wl}", "",
           "Command (run from the repository root on one MI355X):", ""]
    out += [f"    {c}" for c in args.command]
    out += ["", "| kernel | calls | avg us | min us | max us |", "|---|---:|---:|---:|---:|"]
    dom = None
    for r in rows:
        name = r["Name"]
        avg = float(r["AverageNs"]) / 1e3
        out.append(f"| `{short(name)}` | {r['Calls']} | {avg:.1f} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} |")
        if dom is None and is_dominant(name, args.kernel):
            dom = (name, int(r["Calls"]), avg)
    out.append("")
    # kernels that run once per call beside the dominant one (the shared-prefix pass)
    extra = []
    for pre in args.also:
        for r in rows:
            if is_dominant(r["Name"], pre):
                extra.append((r["Name"], float(r["AverageNs"]) / 1e3))
                break
    if dom is not None:
        call_us = dom[2] + sum(t for _, t in extra)
        parts = " + ".join([f"{dom[2]:.1f} us (`{short(dom[0], 200)}`, {dom[1]} calls)"] +
                           [f"{t:.1f} us (`{short(n, 200)}`)" for n, t in extra])
        if roof.get("unit") == "TFLOP/s":
            flops = b["flops_per_call"]
            tf = flops / (call_us * 1e-6) / 1e12
            out.append(f"{flops} algorithmic flops per call (4 D per attended query-key pair and "
                       f"query head) / {parts} average = {tf:.0f} TFLOP/s "
                       f"({100 * tf / roof['peak']:.1f} % of the {roof['peak']:.0f} TFLOP/s "
                       f"dense fp16 matrix-core peak).")
        else:
            nbytes = roof["algorithmic_bytes_per_call"]
            gbs = nbytes / (call_us * 1e-6) / 1e9
            out.append(f"{nbytes} algorithmic bytes per call (KV + q + out + table entries, plus "
                       f"the appended rows when the append is fused) / {parts} average = "
                       f"{gbs:.0f} GB/s ({100 * gbs / 8000:.1f} % of 8 TB/s).")
        out.append(f"The same run's bench line: {roof['avg_call_us']:.1f} us per call "
                   f"(HIP events over the timed back-to-back calls), {b['ms_per_step'] * 1e3:.1f} "
                   f"us per step, value {b['value']:.0f} {b['unit']}.")
    open(args.out, "w").write("\n".join(out) + "\n")
    print("\n".join(out))


def counters(d: str):
    """{(kernel name, grid): [counter value per dispatch]} in KiB."""
    path = find_one(d, "counter_collection.csv")
    per = {}
    for r in csv.DictReader(open(path)):
        key = (r["Kernel_Name"], int(r["Grid_Size"]))
        per.setdefault(key, {}).setdefault(r["Dispatch_Id"], 0.0)
        per[key][r["Dispatch_Id"]] += float(r["Counter_Value"])
    return {k: list(v.values()) for k, v in per.items()}


def calib_kib(per) -> float:
    copies = [(g, v) for (n, g), v in per.items() if "copyBuffer" in n]
    if not copies:
        sys.exit("no calibration copy in the counter run (bench.py --calibrate)")
    g, v = max(copies, key=lambda x: x[0])
    return statistics.median(v)


def traffic(args) -> None:
    fetch, write = counters(args.dirs[0]), counters(args.dirs[1])
    f_cal, w_cal = calib_kib(fetch), calib_kib(write)
    f_scale = CALIB_BYTES / 1024 / f_cal
    w_scale = CALIB_BYTES / 1024 / w_cal
    b = bench_line(args.bench_log)
    wl = b["config"]["workload"].split(":")[0]
    out = [f"# HBM traffic counters: {wl}", "",
           "Two passes (one counter each), from the repository root on one MI355X:", ""]
    out += [f"    {c}" for c in args.command]
    out += ["", "Calibration: `--calibrate` runs a plain device-to-device copy of 256 MiB (262144 "
            "KiB read and", f"262144 KiB written) three times. FETCH_SIZE reads {f_cal:.0f} KiB "
            f"for it and WRITE_SIZE {w_cal:.0f} KiB,", f"so the scale factors are {f_scale:.3f} "
            f"(fetch) and {w_scale:.3f} (write).", "",
            "| kernel | grid | dispatches | FETCH_SIZE KiB (median) | WRITE_SIZE KiB (median) | "
            "scaled bytes / dispatch |", "|---|---:|---:|---:|---:|---:|"]
    dom = None
    for key in sorted(set(fetch) | set(write), key=lambda k: (short(k[0]), k[1])):
        fv = statistics.median(fetch.get(key, [0.0]))
        wv = statistics.median(write.get(key, [0.0]))
        n = max(len(fetch.get(key, [])), len(write.get(key, [])))
        scaled = (fv * f_scale + wv * w_scale) * 1024
        out.append(f"| `{short(key[0])}` | {key[1]} | {n} | {fv:.0f} | {wv:.0f} | {scaled:.4g} |")
        if is_dominant(key[0], args.kernel) and (dom is None or n > dom[4]):
            dom = (key, fv, wv, scaled, n)
    out.append("")
    if dom is None:
        sys.exit(f"kernel {args.kernel!r} not found")
    alg = b["roofline"].get("algorithmic_bytes_per_call")
    if alg:
        out.append(f"`{short(dom[0][0], 200)}`: {dom[3]:.6g} HBM bytes per call against {alg} "
                   f"algorithmic bytes (ratio {dom[3] / alg:.4f}).")
    else:  # a flop-bound kernel: its bench line prices flops, not bytes
        out.append(f"`{short(dom[0][0], 200)}`: {dom[3]:.6g} HBM bytes per call.")
    open(args.out, "w").write("\n".join(out) + "\n")
    print("\n".join(out))
    if args.json:
        sys.path.insert(0, ROOT)
        import bench

        rec = {"workload": args.workload, "kernel": short(dom[0][0], 200),
               "kernel_source_sha256": bench.kernel_source_hash(),
               "hbm_bytes_per_call": dom[3], "fetch_kib": dom[1], "write_kib": dom[2],
               "fetch_scale": f_scale, "write_scale": w_scale,
               "source": os.path.relpath(args.out, ROOT)}
        json.dump(rec, open(args.json, "w"), indent=1)
        open(args.json, "a").write("\n")


# MI355X: 256 compute units of 4 SIMDs in 8 XCDs. GRBM_GUI_ACTIVE counts GPU-busy cycles once
# per XCD; a wave64 vector-ALU instruction occupies its SIMD for 4 cycles (16 lanes per cycle).
N_SIMDS, N_XCDS, N_CUS, VALU_CYCLES = 1024, 8, 256, 4


def sq_counters(d: str, prefix: str):
    """{counter: median over the dominant kernel's dispatches}, and the median duration (ns)."""
    path = find_one(d, "counter_collection.csv")
    per, dur = {}, {}
    for r in csv.DictReader(open(path)):
        if not is_dominant(r["Kernel_Name"], prefix):
            continue
        disp = r["Dispatch_Id"]
        per.setdefault(r["Counter_Name"], {}).setdefault(disp, 0.0)
        per[r["Counter_Name"]][disp] += float(r["Counter_Value"])
        dur[disp] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    if not per:
        sys.exit(f"kernel {prefix!r} not found in {path}")
    return ({k: statistics.median(v.values()) for k, v in per.items()},
            statistics.median(dur.values()), len(dur))


def sq(args) -> None:
    vals, durs, ndisp = {}, [], 0
    for d in args.dirs:
        v, t, n = sq_counters(d, args.kernel)
        vals.update(v)
        durs.append(t)
        ndisp = max(ndisp, n)
    b = bench_line(args.bench_log)
    wl = b["config"]["workload"].split(":")[0]
    out = [f"# Shader counters: {wl}", "",
           f"Kernel `{args.kernel}`; one rocprofv3 pass per command (from the repository root "
           f"on one MI355X):", ""]
    out += [f"    {c}" for c in args.command]
    out += ["", f"Per-dispatch medians over {ndisp} dispatches; median duration "
            f"{statistics.median(durs) / 1e3:.1f} us under the counters.", "",
            "| counter | value |", "|---|---:|"]
    for k in sorted(vals):
        out.append(f"| `{k}` | {vals[k]:.0f} |")
    out += ["", "Ratios (cycles = GRBM_GUI_ACTIVE / 8, the busy cycles of one XCD during the "
            "dispatch):", "", "| ratio | value | definition |", "|---|---:|---|"]
    g = vals.get
    dur_ns = statistics.median(durs)
    cyc = g("GRBM_GUI_ACTIVE", 0) / N_XCDS
    if cyc:
        out.append(f"| busy cycles per ns | {cyc / dur_ns:.2f} | GRBM_GUI_ACTIVE / 8 XCDs / duration "
                   f"(the clock while busy; above it for dispatches of a few tens of us, whose "
                   f"busy count includes their start-up and drain) |")
    waves = g("SQ_WAVES")
    roof = b.get("roofline", {})
    per_kib = roof.get("algorithmic_bytes_per_call")
    flops = b.get("flops_per_call")
    # SQ_INSTS_VALU counts the matrix-core instructions too (the prefill kernel's tile loop holds
    # 122 vector-ALU and 68 MFMA instructions in its assembly, and the counter reads ~205 per
    # tile), so the vector-ALU rows below take SQ_INSTS_VALU - SQ_INSTS_MFMA.
    valu_only = None
    if g("SQ_INSTS_VALU") is not None:
        valu_only = g("SQ_INSTS_VALU") - g("SQ_INSTS_MFMA", 0)
    rows = [("VALU excl. MFMA", valu_only, "(SQ_INSTS_VALU - SQ_INSTS_MFMA)")]
    rows += [(name[9:], g(name), name)
             for name in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU")]
    for label, val, defn in rows:
        if val is None:
            continue
        if waves:
            out.append(f"| {label} per wave | {val / waves:.0f} | {defn} / SQ_WAVES |")
        if flops:
            out.append(f"| {label} per GFLOP | {val / (flops / 1e9):.0f} | "
                       f"{defn} / algorithmic GFLOP per call |")
        elif per_kib:
            out.append(f"| {label} per KiB | {val / (per_kib / 1024):.1f} | "
                       f"{defn} / algorithmic KiB per call |")
    if cyc and g("SQ_VALU_MFMA_BUSY_CYCLES") is not None:
        out.append(f"| matrix-core busy | {g('SQ_VALU_MFMA_BUSY_CYCLES') / (N_SIMDS * cyc):.3f} | "
                   f"SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x cycles) |")
    if cyc and valu_only is not None:
        out.append(f"| vector-ALU issue share | "
                   f"{VALU_CYCLES * valu_only / (N_SIMDS * cyc):.3f} | "
                   f"4 cycles x (SQ_INSTS_VALU - SQ_INSTS_MFMA) / (1024 SIMDs x cycles) |")
    if cyc and g("SQ_LDS_IDX_ACTIVE"):
        out.append(f"| LDS active | {g('SQ_LDS_IDX_ACTIVE') / (N_CUS * cyc):.3f} | "
                   f"SQ_LDS_IDX_ACTIVE / (256 CUs x cycles) |")
        out.append(f"| LDS bank-conflict share | "
                   f"{g('SQ_LDS_BANK_CONFLICT', 0) / g('SQ_LDS_IDX_ACTIVE'):.3f} | "
                   f"SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE |")
    if g("SQ_WAVE_CYCLES"):
        for name, what in (("SQ_ACTIVE_INST_ANY", "issuing"),
                           ("SQ_WAIT_INST_ANY", "waiting to issue (dependencies, busy units)"),
                           ("SQ_WAIT_ANY", "waiting on memory counters or barriers")):
            if g(name) is not None:
                out.append(f"| wave time {what} | {g(name) / g('SQ_WAVE_CYCLES'):.3f} | "
                           f"{name} / SQ_WAVE_CYCLES |")
    open(args.out, "w").write("\n".join(out) + "\n")
    print("\n".join(out))


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("mode", choices=["trace", "traffic", "sq"])
    ap.add_argument("dirs", nargs="+", help="rocprofv3 output directories")
    ap.add_argument("--bench-log", required=True, help="stdout of the profiled bench.py run")
    ap.add_argument("--command", action="append", default=[], help="command that made the data")
    ap.add_argument("--kernel", default="decode_partition_kernel",
                    help="name prefix of the dominant kernel")
    ap.add_argument("--also", action="append", default=[],
                    help="name prefix of another kernel launched once per call (trace mode)")
    ap.add_argument("--workload", default="8b", help="bench.py --workload of the run")
    ap.add_argument("--out", required=True)
    ap.add_argument("--json", default=None)
    args = ap.parse_args()
    {"trace": trace, "traffic": traffic, "sq": sq}[args.mode](args)


if __name__ == "__main__":
    main()
