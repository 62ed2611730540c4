"""Turn rocprofv3 output into the measurement records kept under profiles/.

Two kinds of record:

* HBM traffic per launch of each stage kernel, from two counter passes
  (``--pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE``, each its own run) of
  ``bench.py``, scaled by what the same counters read for plain device copies
  of a known size (``bench.py --copy-calibration-mib``). One JSON file per
  kernel (``traffic_<kernel>_<workload>_<direction>.json``) carries the bytes
  and a hash of the kernel sources, so ``bench.py`` only reports them while
  the kernel is unchanged, plus a Markdown summary.
* A kernel-trace summary (``--kernel-trace --stats``) as Markdown, with the
  per-kernel averages of the timed calls and the source hashes as JSON.
* Matrix-core and vector-ALU utilisation per kernel (``--pmc MfmaUtil
  VALUBusy MfmaFlopsBF16``), as JSON and Markdown.

Usage (each counter pass is a separate rocprofv3 run; see the written
summaries for the exact commands)::

    python -m triangle_multiplicative_update_amd.profiling traffic \\
        --fetch DIR --write DIR --cal-fetch DIR --cal-write DIR --cal-mib 512 \\
        --workload n768_c128_pad700 --direction outgoing --out profiles
    python -m triangle_multiplicative_update_amd.profiling trace \\
        --stats DIR --workload n768_c128_pad700 --direction outgoing --out profiles
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
KERNEL_FILES = {1: "k1_ln_proj.hip", 2: "k2_contract.hip", 3: "k3_epilogue.hip"}
KERNEL_NAMES = {1: "k1_ln_proj", 2: "k2_contract", 3: "k3_epilogue"}
SHARED_FILES = ("trimul_device.hpp", "trimul_kernels.hpp")
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def kernel_sha(stage: int) -> str:
    """Hash of the sources a stage kernel is built from."""
    h = hashlib.sha256()
    for f in (KERNEL_FILES[stage], *SHARED_FILES):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stage_of(kernel_name: str):
    """Stage (1, 2, 3) of a kernel name as rocprofv3 prints it, e.g.
    ``void trimul::k2_contract<256, ...>(trimul::K2Args)``,
    ``trimul::k2_contract_p(trimul::K2Args)`` or
    ``trimul::(anonymous namespace)::k3_epilogue_ws(trimul::K3Args)``."""
    for s, n in KERNEL_NAMES.items():
        if re.search(r"\b" + n + r"(_ws|_p|_wide|_h256)?(<|\()", kernel_name):
            return s
    return None


def _csv_rows(directory: str, suffix: str):
    files = glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no *{suffix} under {directory}")
    for f in files:
        with open(f, newline="") as fh:
            yield from csv.DictReader(fh)


def counter_per_dispatch(directory: str, counter: str):
    """{kernel name: [counter value of each dispatch]} from a --pmc run."""
    out: dict[str, list[float]] = {}
    for row in _csv_rows(directory, "counter_collection.csv"):
        if row.get("Counter_Name") != counter:
            continue
        out.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return out


def _median_for(values: dict, pred):
    vs = [v for k, lst in values.items() if pred(k) for v in lst]
    if not vs:
        raise KeyError("no matching dispatch")
    return statistics.median(vs)


def traffic(args) -> None:
    from . import perf_model
    import synthetic_inputs as si

    wl = si.WORKLOADS[args.workload]
    fetch = counter_per_dispatch(args.fetch, "FETCH_SIZE")
    write = counter_per_dispatch(args.write, "WRITE_SIZE")
    cal_bytes = args.cal_mib * 2 ** 20
    # a copy reads and writes cal_bytes once each; the counters are in KiB
    cal_f = _median_for(counter_per_dispatch(args.cal_fetch, "FETCH_SIZE"), lambda k: COPY_KERNEL in k)
    cal_w = _median_for(counter_per_dispatch(args.cal_write, "WRITE_SIZE"), lambda k: COPY_KERNEL in k)
    f_scale = cal_bytes / (cal_f * 1024.0)
    w_scale = cal_bytes / (cal_w * 1024.0)
    sb = perf_model.stage_bytes(wl.B, wl.N, wl.c_z, wl.c, mask=wl.mask != "none")
    bench_cmd = f"python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --workload {args.workload} --direction {args.direction}"
    cmds = [
        f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -o run -- {bench_cmd}",
        f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir> -o run -- {bench_cmd}",
        f"rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) --output-format csv -d <dir> -o run -- "
        f"python3 bench.py --steps 3 --copy-calibration-mib {args.cal_mib}",
    ]
    rows = []
    for s in (1, 2, 3):
        name = KERNEL_NAMES[s]
        fk = _median_for(fetch, lambda k: stage_of(k) == s)
        wk = _median_for(write, lambda k: stage_of(k) == s)
        rec = {
            "kernel": name,
            "workload": args.workload,
            "direction": args.direction,
            "kernel_sha": kernel_sha(s),
            "hbm_bytes_per_launch": fk * 1024 * f_scale + wk * 1024 * w_scale,
            "fetch_bytes": fk * 1024 * f_scale,
            "write_bytes": wk * 1024 * w_scale,
            "algorithmic_bytes": sb[s - 1],
            "fetch_kib_raw": fk,
            "write_kib_raw": wk,
            "fetch_scale": f_scale,
            "write_scale": w_scale,
            "commands": cmds,
        }
        with open(os.path.join(args.out, f"traffic_{name}_{args.workload}_{args.direction}.json"), "w") as fh:
            json.dump(rec, fh, indent=1)
        rows.append(rec)
    md = [f"# HBM traffic per launch: {args.workload}, {args.direction}", "",
          "Commands (each its own rocprofv3 run, from /tmp, repository at $R):", "", "```"]
    md += [c.replace("python3 bench.py", "python3 $R/bench.py") for c in cmds]
    md += ["```", "",
           f"Calibration: a {args.cal_mib} MiB device copy (`{COPY_KERNEL}`, {args.cal_mib} MiB read + "
           f"{args.cal_mib} MiB written) reads FETCH_SIZE = {cal_f:.0f} KiB and WRITE_SIZE = {cal_w:.0f} KiB, "
           f"so FETCH_SIZE is scaled by {f_scale:.4f} and WRITE_SIZE by {w_scale:.4f} to bytes.", "",
           "| kernel | FETCH_SIZE (KiB, raw) | WRITE_SIZE (KiB, raw) | HBM read (MB) | HBM write (MB) | "
           "total (MB) | algorithmic (MB) | ratio |",
           "|---|---|---|---|---|---|---|---|"]
    for r in rows:
        md.append(f"| {r['kernel']} | {r['fetch_kib_raw']:.0f} | {r['write_kib_raw']:.0f} | "
                  f"{r['fetch_bytes'] / 1e6:.1f} | {r['write_bytes'] / 1e6:.1f} | "
                  f"{r['hbm_bytes_per_launch'] / 1e6:.1f} | {r['algorithmic_bytes'] / 1e6:.1f} | "
                  f"{r['hbm_bytes_per_launch'] / r['algorithmic_bytes']:.3f} |")
    md += ["", f"The per-kernel records `traffic_<kernel>_{args.workload}_{args.direction}.json` carry these "
           "numbers with a hash of the kernel sources they were taken on; `bench.py` reports them as "
           "`roofline.traffic` only while the hash matches.", ""]
    with open(os.path.join(args.out, f"hbm_traffic_{args.workload}_{args.direction}.md"), "w") as fh:
        fh.write("\n".join(md))


PHASES = ("settle", "warmup", "timed", "graph warmup", "graph")


def phase_means(trace_dir: str, warmup: int, steps: int, settle: int = 0):
    """Mean duration (us) of each stage kernel in each phase of a bench.py run.

    bench.py runs ``settle`` untimed eager steps, ``warmup`` eager steps,
    ``steps`` timed eager steps (HIP events between the stages), then
    ``warmup`` and ``steps`` launches of the captured graph; every step
    dispatches each stage kernel once, so the dispatches of a stage, in start
    order, split into those five phases (a phase of no steps is left out)."""
    durs: dict[int, list] = {1: [], 2: [], 3: []}
    for r in _csv_rows(trace_dir, "kernel_trace.csv"):
        s = stage_of(r["Kernel_Name"])
        if s is not None:
            durs[s].append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    counts = (settle, warmup, steps, warmup, steps)
    bounds, at = {}, 0
    for ph, n in zip(PHASES, counts):
        if n:
            bounds[ph] = (at, at + n)
        at += n
    out = {}
    for s, lst in durs.items():
        if len(lst) != at:
            raise ValueError(f"stage {s}: {len(lst)} dispatches, expected {at}")
        d = [v for _, v in sorted(lst)]
        out[s] = {ph: statistics.mean(d[a:b]) / 1e3 for ph, (a, b) in bounds.items()}
    return out


def trace(args) -> None:
    rows = list(_csv_rows(args.stats, "kernel_stats.csv"))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    md = [f"# Kernel trace: {args.workload}, {args.direction}", "",
          "Command (run from /tmp on the MI355X box, repository at $R):", "", "```",
          f"rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o run -- python3 $R/bench.py "
          f"{args.bench_args}", "```", "", "`run_kernel_stats.csv`:", "",
          "| kernel | calls | average (us) | min (us) | max (us) | share |", "|---|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        md.append(f"| `{r['Name']}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                  f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                  f"{100 * float(r['TotalDurationNs']) / total:.1f} % |")
    rec = None
    if args.bench_json:
        with open(args.bench_json) as fh:
            line = [l for l in fh if l.startswith("{")][-1]
        rec = json.loads(line)
    summary = {"workload": args.workload, "direction": args.direction,
               "command": f"rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o run -- "
                          f"python3 bench.py {args.bench_args}", "kernels": {}}
    for r in rows:
        s = stage_of(r["Name"])
        if s is not None:
            summary["kernels"][KERNEL_NAMES[s]] = {"kernel_sha": kernel_sha(s), "calls": int(r["Calls"]),
                                                   "average_us": float(r["AverageNs"]) / 1e3}
    if args.phases == "auto" and rec is not None:
        args.phases = f"{rec.get('settle_calls', 0)},{rec['warmup']},{rec['steps']}"
    if args.phases:
        parts = [int(v) for v in args.phases.split(",")]
        settle, warmup, steps = parts if len(parts) == 3 else [0] + parts
        pm = phase_means(args.stats, warmup, steps, settle)
        names = [ph for ph in PHASES if ph in pm[1]]
        md += ["", f"Mean duration per phase of the run (`run_kernel_trace.csv`, each stage's dispatches in start "
               f"order: {settle} settle steps, {warmup} warmup steps, {steps} timed eager steps, {warmup} + {steps} "
               f"graph launches), in us:",
               "", "| kernel | " + " | ".join(names) + " | HIP events, timed steps |",
               "|---|" + "---|" * len(names) + "---|"]
        for s in (1, 2, 3):
            ev = (rec or {}).get("per_stage_us", {}).get(KERNEL_NAMES[s])
            md.append(f"| {KERNEL_NAMES[s]} | " + " | ".join(f"{pm[s][ph]:.1f}" for ph in names) +
                      f" | {'' if ev is None else f'{ev:.1f}'} |")
            summary["kernels"][KERNEL_NAMES[s]]["timed_us"] = pm[s]["timed"]
            summary["kernels"][KERNEL_NAMES[s]]["phases_us"] = pm[s]
            if ev is not None:
                summary["kernels"][KERNEL_NAMES[s]]["hip_event_us"] = ev
    if rec is not None:
        md += ["", "The same process's own HIP-event timing of the timed steps (`per_stage_us` of its JSON line):",
               "", "```", json.dumps(rec.get("per_stage_us")), "```"]
    md.append("")
    with open(os.path.join(args.out, f"kernel_trace_{args.workload}_{args.direction}.md"), "w") as fh:
        fh.write("\n".join(md))
    with open(os.path.join(args.out, f"kernel_trace_{args.workload}_{args.direction}.json"), "w") as fh:
        json.dump(summary, fh, indent=1)


UTIL_COUNTERS = ("MfmaUtil", "VALUBusy", "MfmaFlopsBF16")


def util(args) -> None:
    """Matrix-core and vector-ALU utilisation per stage kernel from one
    ``--pmc MfmaUtil VALUBusy MfmaFlopsBF16`` run (rocprofv3's derived
    counters: MfmaUtil = 100 * sum SQ_VALU_MFMA_BUSY_CYCLES / (max
    GRBM_GUI_ACTIVE * SIMD_NUM), VALUBusy = 100 * sum SQ_ACTIVE_INST_VALU /
    CU_NUM / max GRBM_GUI_ACTIVE, MfmaFlopsBF16 = 512 * SQ_INSTS_VALU_MFMA_MOPS_BF16),
    median over the dispatches of each kernel."""
    from . import perf_model
    import synthetic_inputs as si

    wl = si.WORKLOADS[args.workload]
    vals = {c: counter_per_dispatch(args.pmc, c) for c in UTIL_COUNTERS}
    sf = perf_model.stage_flops(wl.B, wl.N, wl.c_z, wl.c)
    cmd = (f"rocprofv3 --pmc {' '.join(UTIL_COUNTERS)} --output-format csv -d <dir> -o run -- "
           f"python3 bench.py {args.bench_args}")
    rec = {"workload": args.workload, "direction": args.direction, "command": cmd, "kernels": {}}
    md = [f"# Matrix-core and vector-ALU utilisation: {args.workload}, {args.direction}", "",
          "Command (from /tmp on the MI355X box, repository at $R):", "", "```",
          cmd.replace("python3 bench.py", "python3 $R/bench.py"), "```", "",
          "rocprofv3's derived counters, median over each kernel's dispatches: MfmaUtil = 100 * sum "
          "SQ_VALU_MFMA_BUSY_CYCLES / (max GRBM_GUI_ACTIVE * SIMD_NUM); VALUBusy = 100 * sum "
          "SQ_ACTIVE_INST_VALU / CU_NUM / max GRBM_GUI_ACTIVE; MfmaFlopsBF16 = 512 * "
          "SQ_INSTS_VALU_MFMA_MOPS_BF16 (issued matrix-core flops, against the algorithmic flops).", "",
          "| kernel | MfmaUtil (%) | VALUBusy (%) | MFMA flops issued (G) | algorithmic flops (G) |",
          "|---|---|---|---|---|"]
    for s in (1, 2, 3):
        name = KERNEL_NAMES[s]
        k = {c: _median_for(vals[c], lambda kn: stage_of(kn) == s) for c in UTIL_COUNTERS}
        rec["kernels"][name] = {"kernel_sha": kernel_sha(s), "mfma_util_pct": k["MfmaUtil"],
                                "valu_busy_pct": k["VALUBusy"], "mfma_flops_bf16": k["MfmaFlopsBF16"],
                                "algorithmic_flops": sf[s - 1]}
        md.append(f"| {name} | {k['MfmaUtil']:.1f} | {k['VALUBusy']:.1f} | {k['MfmaFlopsBF16'] / 1e9:.1f} | "
                  f"{sf[s - 1] / 1e9:.1f} |")
    md.append("")
    base = os.path.join(args.out, f"util_{args.workload}_{args.direction}")
    with open(base + ".json", "w") as fh:
        json.dump(rec, fh, indent=1)
    with open(base + ".md", "w") as fh:
        fh.write("\n".join(md))


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("traffic")
    for a in ("--fetch", "--write", "--cal-fetch", "--cal-write", "--workload", "--direction", "--out"):
        t.add_argument(a, required=True)
    t.add_argument("--cal-mib", type=int, required=True)
    k = sub.add_parser("trace")
    for a in ("--stats", "--workload", "--direction", "--out"):
        k.add_argument(a, required=True)
    k.add_argument("--bench-args", default="")
    k.add_argument("--bench-json", default=None, help="file holding the profiled run's JSON line")
    k.add_argument("--phases", default=None, help="[SETTLE,]WARMUP,STEPS of the profiled bench.py run, or 'auto' to read "
                   "them from --bench-json")
    u = sub.add_parser("util")
    for a in ("--pmc", "--workload", "--direction", "--out"):
        u.add_argument(a, required=True)
    u.add_argument("--bench-args", default="")
    args = ap.parse_args()
    os.makedirs(args.out, exist_ok=True)
    {"traffic": traffic, "trace": trace, "util": util}[args.cmd](args)


if __name__ == "__main__":
    main()
