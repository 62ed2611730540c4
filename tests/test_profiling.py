"""Host logic of the measurement records (no GPU, no profiler).

``stage_of`` must place every kernel the library defines in the stage of the
source file that defines it, under the names rocprofv3 prints; ``traffic``
must scale the counters by the copy calibration and write one record per
stage carrying the source hash.
"""

import csv
import json
import os
import re
import types

import pytest

from triangle_multiplicative_update_amd import perf_model, profiling


def _kernels_by_file():
    """{stage: [kernel names]} from the __global__ definitions in each source."""
    out = {}
    for stage, f in profiling.KERNEL_FILES.items():
        with open(os.path.join(profiling.CSRC, f)) as fh:
            src = fh.read()
        out[stage] = sorted(set(re.findall(r"__global__.*?\bvoid\s+(\w+)\s*[<(]", src)))
    return out


def test_every_defined_kernel_maps_to_its_stage():
    found = _kernels_by_file()
    assert all(found.values()), found
    for stage, names in found.items():
        for n in names:
            # the two forms rocprofv3 prints: a template instance and a plain function
            assert profiling.stage_of(f"void trimul::{n}<128>(trimul::K1Args)") == stage, n
            assert profiling.stage_of(f"trimul::(anonymous namespace)::{n}(trimul::K3Args)") == stage, n


def test_other_kernels_map_to_no_stage():
    for n in ("__amd_rocclr_copyBuffer", "void at::native::elementwise_kernel<128, 4>(int)",
              "trimul::k2_contract_px(trimul::K2Args)", "trimul::xk1_ln_proj(trimul::K1Args)"):
        assert profiling.stage_of(n) is None, n


def _write_counters(directory, counter, rows):
    os.makedirs(directory)
    with open(os.path.join(directory, "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for k, v in rows:
            w.writerow({"Kernel_Name": k, "Counter_Name": counter, "Counter_Value": v})


def test_traffic_scales_by_copy_calibration(tmp_path):
    names = {1: "void trimul::(anonymous namespace)::k1_ln_proj<128>(trimul::K1Args)",
             2: "trimul::k2_contract_p(trimul::K2Args)",
             3: "trimul::(anonymous namespace)::k3_epilogue_ws(trimul::K3Args)"}
    cal_mib = 4
    # the copy reads half of what it moves by FETCH_SIZE's count, all by WRITE_SIZE's
    _write_counters(tmp_path / "cf", "FETCH_SIZE", [(profiling.COPY_KERNEL, cal_mib * 512)] * 3)
    _write_counters(tmp_path / "cw", "WRITE_SIZE", [(profiling.COPY_KERNEL, cal_mib * 1024)] * 3)
    # three dispatches per stage; the median is the middle one
    _write_counters(tmp_path / "f", "FETCH_SIZE",
                    [(names[s], 100 * s + d) for s in (1, 2, 3) for d in (-7, 0, 9)])
    _write_counters(tmp_path / "w", "WRITE_SIZE",
                    [(names[s], 10 * s + d) for s in (1, 2, 3) for d in (5, 0, -3)])
    out = tmp_path / "out"
    os.makedirs(out)
    profiling.traffic(types.SimpleNamespace(
        fetch=str(tmp_path / "f"), write=str(tmp_path / "w"), cal_fetch=str(tmp_path / "cf"),
        cal_write=str(tmp_path / "cw"), cal_mib=cal_mib, workload="n768_c128_pad700",
        direction="outgoing", out=str(out)))
    sb = perf_model.stage_bytes(1, 768, 128, 128, mask=True)
    for s in (1, 2, 3):
        name = profiling.KERNEL_NAMES[s]
        with open(out / f"traffic_{name}_n768_c128_pad700_outgoing.json") as fh:
            rec = json.load(fh)
        assert rec["fetch_bytes"] == 100 * s * 1024 * 2.0
        assert rec["write_bytes"] == 10 * s * 1024 * 1.0
        assert rec["hbm_bytes_per_launch"] == rec["fetch_bytes"] + rec["write_bytes"]
        assert rec["algorithmic_bytes"] == sb[s - 1]
        assert rec["kernel_sha"] == profiling.kernel_sha(s)
    assert (out / "hbm_traffic_n768_c128_pad700_outgoing.md").exists()


def test_phase_means_split_dispatches_in_start_order(tmp_path):
    warmup, steps = 2, 3
    names = {1: "void trimul::(anonymous namespace)::k1_ln_proj<128>(trimul::K1Args)",
             2: "trimul::k2_contract_p(trimul::K2Args)",
             3: "trimul::(anonymous namespace)::k3_epilogue_ws(trimul::K3Args)"}
    # phase p of stage s lasts (1000 * s + 100 * p) ns per dispatch; rows are written out of order
    rows, t = [], 0
    for p, n in enumerate((warmup, steps, warmup, steps)):
        for _ in range(n):
            for s in (1, 2, 3):
                rows.append({"Kernel_Name": names[s], "Start_Timestamp": t,
                             "End_Timestamp": t + 1000 * s + 100 * p})
                t += 10000
    rows.append({"Kernel_Name": profiling.COPY_KERNEL, "Start_Timestamp": 5, "End_Timestamp": 9})
    os.makedirs(tmp_path / "tr")
    with open(tmp_path / "tr" / "run_kernel_trace.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        w.writerows(reversed(rows))
    pm = profiling.phase_means(str(tmp_path / "tr"), warmup, steps)
    for s in (1, 2, 3):
        for p, ph in enumerate(("warmup", "timed", "graph warmup", "graph")):
            assert pm[s][ph] == (1000 * s + 100 * p) / 1e3


def test_phase_means_with_settle_steps(tmp_path):
    settle, warmup, steps = 4, 2, 3
    names = {1: "void trimul::(anonymous namespace)::k1_ln_proj<128>(trimul::K1Args)",
             2: "trimul::k2_contract_p(trimul::K2Args)",
             3: "trimul::(anonymous namespace)::k3_epilogue_ws(trimul::K3Args)"}
    rows, t = [], 0
    for p, n in enumerate((settle, warmup, steps, warmup, steps)):
        for _ in range(n):
            for s in (1, 2, 3):
                rows.append({"Kernel_Name": names[s], "Start_Timestamp": t,
                             "End_Timestamp": t + 1000 * s + 100 * p})
                t += 10000
    os.makedirs(tmp_path / "tr")
    with open(tmp_path / "tr" / "run_kernel_trace.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        w.writerows(rows)
    pm = profiling.phase_means(str(tmp_path / "tr"), warmup, steps, settle)
    for s in (1, 2, 3):
        for p, ph in enumerate(profiling.PHASES):
            assert pm[s][ph] == (1000 * s + 100 * p) / 1e3
    with pytest.raises(ValueError, match="dispatches"):
        profiling.phase_means(str(tmp_path / "tr"), warmup, steps)      # settle steps not counted


def test_util_records_per_stage(tmp_path):
    names = {1: "void trimul::(anonymous namespace)::k1_ln_proj<128>(trimul::K1Args)",
             2: "trimul::k2_contract_p(trimul::K2Args)",
             3: "trimul::(anonymous namespace)::k3_epilogue_ws(trimul::K3Args)"}
    os.makedirs(tmp_path / "pmc")
    with open(tmp_path / "pmc" / "run_counter_collection.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for rep in range(3):
            for s in (1, 2, 3):
                w.writerow({"Kernel_Name": names[s], "Counter_Name": "MfmaUtil", "Counter_Value": 10 * s + rep})
                w.writerow({"Kernel_Name": names[s], "Counter_Name": "VALUBusy", "Counter_Value": 5 * s})
                w.writerow({"Kernel_Name": names[s], "Counter_Name": "MfmaFlopsBF16", "Counter_Value": 1e9 * s})
        w.writerow({"Kernel_Name": profiling.COPY_KERNEL, "Counter_Name": "MfmaUtil", "Counter_Value": 99})
    args = types.SimpleNamespace(pmc=str(tmp_path / "pmc"), workload="n768_c128_pad700",
                                 direction="outgoing", out=str(tmp_path), bench_args="--steps 3")
    profiling.util(args)
    rec = json.load(open(tmp_path / "util_n768_c128_pad700_outgoing.json"))
    for s in (1, 2, 3):
        k = rec["kernels"][profiling.KERNEL_NAMES[s]]
        assert k["mfma_util_pct"] == 10 * s + 1           # median of the three dispatches
        assert k["valu_busy_pct"] == 5 * s and k["mfma_flops_bf16"] == 1e9 * s
        assert k["kernel_sha"] == profiling.kernel_sha(s)
    assert "MfmaUtil" in rec["command"]
