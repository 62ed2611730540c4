#!/usr/bin/env python3
"""Throughput of the triangle multiplicative update on one MI355X.

One step = one forward call (stage 1 LayerNorm_in + gated projections, stage 2
contraction, stage 3 LayerNorm_out + gated output projection) over the
N = 768, c_z = c = 128, B = 1 workload with inputs already resident in HBM.
After untimed settle and warm-up calls, the K timed steps enqueue the three
stages through the C ABI with HIP events between them, so the per-stage device
times come from the same timed region. The same call captured once as a HIP
graph is then launched W + K times and reported beside it (graph_ms_per_step).

Prints ONE JSON line (rank 0). Extra legs: the roofline of the dominant stage
and the CPU oracle's time on this host (a baseline, not a target).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time


def _host_threads():
    """(cores this process may run on, threads the CPU baseline's BLAS uses):
    the affinity set, capped by an OMP_NUM_THREADS the environment sets."""
    aff = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS", "")
    return aff, (min(aff, int(env)) if env.isdigit() and int(env) > 0 else aff)


# BLAS reads its thread count when numpy is first imported: set it first
AFFINITY_CORES, CPU_THREADS = _host_threads()
for _v in ("OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS"):
    os.environ.setdefault(_v, str(CPU_THREADS))

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from triangle_multiplicative_update_amd.profiling import KERNEL_NAMES, kernel_sha  # noqa: E402

PROFILE_DIR = os.path.join(ROOT, "profiles")
MFMA_BALANCE = 2516.6e12 / 8000e9       # flop per byte where the two roofs meet


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="before the warm-up, untimed calls until this much GPU time has passed and "
                         "the time per call has stopped falling (at most 10x this)")
    ap.add_argument("--workload", default=None, help="workload name (default: the N=768 one)")
    ap.add_argument("--direction", default="outgoing", choices=["outgoing", "incoming"])
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--cpu-sample-rows", type=int, default=0,
                    help="time the oracle on this many output rows only (0 = the whole call)")
    ap.add_argument("--cpu-min-seconds", type=float, default=10.0,
                    help="repeat the oracle sample until this much time has passed (at most 8 runs)")
    ap.add_argument("--profile-dir", default=None,
                    help="where the HBM traffic records are read (default: profiles/)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run --steps plain device copies of this many MiB (for scaling "
                         "the HBM byte counters) and exit")
    return ap.parse_args()


def measured_traffic(stage: int, workload: str, direction: str, profile_dir: str = PROFILE_DIR):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(profile_dir, f"traffic_{KERNEL_NAMES[stage]}_{workload}_{direction}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_sha") != kernel_sha(stage):
        return None
    return rec.get("hbm_bytes_per_launch")


def measured_trace(stage: int, workload: str, direction: str, profile_dir: str = PROFILE_DIR):
    """Average device time (us) of a stage kernel over the timed calls of the
    committed rocprofv3 kernel trace of this workload, if that trace was taken
    on the current kernel source; else None."""
    path = os.path.join(profile_dir, f"kernel_trace_{workload}_{direction}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    k = rec.get("kernels", {}).get(KERNEL_NAMES[stage], {})
    if k.get("kernel_sha") != kernel_sha(stage):
        return None
    return k.get("timed_us")


def settle(call, min_ms: float):
    """Untimed calls, in groups of 10, until at least min_ms of GPU time has
    passed and a group's time per call is within 2 % of the previous group's
    (at most 10 * min_ms): the clock and power state the timed calls see.
    Returns (calls, GPU ms, ms per call of the last group)."""
    import torch
    total, calls, prev, per = 0.0, 0, None, None
    while True:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            call()
        e1.record()
        e1.synchronize()
        ms = e0.elapsed_time(e1)
        total += ms
        calls += 10
        per = ms / 10
        if total >= 10 * min_ms or (total >= min_ms and prev is not None and abs(per - prev) <= 0.02 * prev):
            return calls, total, per
        prev = per


def cpu_baseline(inp, wl, direction, flops_per_call, sample_rows: int, min_seconds: float = 10.0):
    import numpy as np
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
                      or [1])
    except Exception:
        threads = CPU_THREADS
    import oracle
    # the sample is run whole, again and again, until min_seconds have passed
    runs = 0
    t0 = time.perf_counter()
    while True:
        if sample_rows and sample_rows < wl.N:
            oracle.forward_block(inp, direction, list(range(sample_rows)), list(range(wl.N)))
        else:
            oracle.forward(inp, direction)
        runs += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or runs >= 8:
            break
    if sample_rows and sample_rows < wl.N:
        frac = runs * sample_rows / wl.N
        sample = f"oracle.forward_block over {sample_rows} of {wl.N} output rows (all columns), {runs} runs"
    else:
        frac = float(runs)
        sample = f"oracle.forward, the whole {wl.name} {direction} call, {runs} runs"
    del np
    return {
        "value": flops_per_call * frac / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "affinity_cores": AFFINITY_CORES,
        "kind": "oracle",
        "sample": sample,
        "seconds": dt,
        "pair_cells_per_s": wl.B * wl.N * wl.N * frac / dt,
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the library runs on one GPU per process; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import synthetic_inputs as si
    from triangle_multiplicative_update_amd import perf_model

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}), flush=True)
        sys.exit(1)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": args.steps}), flush=True)
        return
    name = args.workload or si.BENCH_WORKLOAD
    wl = si.WORKLOADS[name]
    direction = args.direction
    inp = si.generate(wl)

    def up(a):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    d = {k: up(v) for k, v in inp.items()}
    from triangle_multiplicative_update_amd.api import workspace_bytes
    out = torch.empty_like(d["x"])
    ws = torch.empty(workspace_bytes(wl.B, wl.N, wl.c, direction), dtype=torch.uint8, device=dev)
    from triangle_multiplicative_update_amd.api import Prepared
    prep = Prepared(d["x"], direction, d["mask"], {k: d[k] for k in si.PARAM_NAMES}, out, ws)

    with torch.no_grad():
        settle_calls, settle_ms, settle_per_call = settle(prep.forward, args.settle_ms)
        for _ in range(args.warmup):
            prep.forward()
        torch.cuda.synchronize()

        K = args.steps
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(K):
            ev[k][0].record()
            prep.stage(1)
            ev[k][1].record()
            prep.stage(2)
            ev[k][2].record()
            prep.stage(3)
            ev[k][3].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0

        # the same call as one captured graph launch per step (host overhead of
        # three eager launches removed), timed the same way
        graph = prep.graph()
        for _ in range(args.warmup):
            graph.launch()
        torch.cuda.synchronize()
        tg = time.perf_counter()
        for _ in range(K):
            graph.launch()
        torch.cuda.synchronize()
        graph_wall = time.perf_counter() - tg
        graph.close()

    per_stage_ms = [float(np.mean([ev[k][s].elapsed_time(ev[k][s + 1]) for k in range(K)]))
                    for s in range(3)]
    span_ms = ev[0][0].elapsed_time(ev[K - 1][3]) / K      # device span per step
    # the timed steps: K eager calls, host clock, synchronized on both sides;
    # the HIP events between their stages (on the stream the kernels run on)
    # give the per-stage times of the same region
    ms_per_step = wall * 1e3 / K
    F = perf_model.flops(wl.B, wl.N, wl.c_z, wl.c)
    T = perf_model.traffic_bytes(wl.B, wl.N, wl.c_z, wl.c, mask=inp["mask"] is not None)
    t = ms_per_step * 1e-3
    tflops = F / t / 1e12

    sf = perf_model.stage_flops(wl.B, wl.N, wl.c_z, wl.c)
    sb = perf_model.stage_bytes(wl.B, wl.N, wl.c_z, wl.c, mask=inp["mask"] is not None)
    dom = int(np.argmax(per_stage_ms))
    ts = per_stage_ms[dom] * 1e-3
    intensity = sf[dom] / sb[dom]
    if intensity > MFMA_BALANCE:
        roof = {"bound": "mfma", "achieved": sf[dom] / ts / 1e12, "peak": perf_model.PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": sb[dom] / ts / 1e9, "peak": perf_model.PEAK_HBM_GBS,
                "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(dom + 1, name, direction, args.profile_dir or PROFILE_DIR)
    roof["kernel"] = KERNEL_NAMES[dom + 1]
    roof["kernel_us"] = per_stage_ms[dom] * 1e3
    # the same kernel's average in the committed rocprofv3 trace (kernel time
    # alone, without the launch gap the HIP events also hold), and the
    # fraction it gives
    tr = measured_trace(dom + 1, name, direction, args.profile_dir or PROFILE_DIR)
    roof["trace_kernel_us"] = tr
    if tr:
        work = sb[dom] / 1e9 if roof["bound"] == "hbm" else sf[dom] / 1e12
        roof["trace_frac"] = work / (tr * 1e-6) / roof["peak"]
    roof["algorithmic_bytes"] = sb[dom]
    roof["algorithmic_flops"] = sf[dom]

    line = {
        "metric": "TFLOP/s and pair-cells/s (B*N^2/s) at N=768, c=128, bf16; % of MFMA peak",
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": name, "B": wl.B, "N": wl.N, "c_z": wl.c_z, "c": wl.c,
                   "direction": direction, "mask": wl.mask if wl.mask != "padded" else f"padded L={wl.mask_len}",
                   "biases": wl.biases},
        "pair_cells_per_s": wl.B * wl.N * wl.N / t,
        "pct_mfma_peak": 100.0 * tflops / perf_model.PEAK_BF16_TFLOPS,
        "hbm_gbs_model": T / t / 1e9,
        "per_stage_us": {KERNEL_NAMES[s + 1]: per_stage_ms[s] * 1e3 for s in range(3)},
        "device_ms_per_step": span_ms,
        "graph_ms_per_step": graph_wall * 1e3 / K,
        "settle_calls": settle_calls,
        "settle_gpu_ms": settle_ms,
        "settle_ms_per_call": settle_per_call,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(inp, wl, direction, F, args.cpu_sample_rows, args.cpu_min_seconds)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
