"""Helpers shared by the GPU parity tests: device upload, the call through the
C ABI, reading the workspace planes, and the acceptance statistics.

Acceptance bar for the output (the tolerance this library holds itself to, in
line with the page "Triangle Multiplicative Update (SM100 / SM103 / SM107)",
section "Mathematics and numerics", measured numerics):
  * relative RMS  ||gpu - ref||_2 / ||ref||_2  <= 2e-3
  * |gpu - ref| <= 4e-3 + |ref|/64 on all but 10 per million cells
  * |gpu - ref| <= 2e-2 + |ref|/64 on every cell
where ref is the oracle's unrounded fp64 output with the kernel rounding points.
On a sampled subset of n cells the allowance of the second rule is
ceil(10e-6 * n) cells (the same rate, rounded up to whole cells).
"""

from __future__ import annotations

import functools
import math
import sys

import numpy as np
import torch

import synthetic_inputs as si

REL_RMS_MAX = 2e-3
TIGHT_ABS, HARD_ABS, REL_SLOPE = 4e-3, 2e-2, 1.0 / 64
TAIL_PER_MILLION = 10


def say(msg: str) -> None:
    """Name the case before a GPU step (flushed, so a fault still shows it)."""
    print(msg, file=sys.stderr, flush=True)


@functools.lru_cache(maxsize=4)
def workload_inputs(name: str):
    return si.generate(si.WORKLOADS[name])


def bits_to_bf16(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)


def to_device(inp, device):
    return {k: (None if v is None else bits_to_bf16(v, device)) for k, v in inp.items()}


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def call(dev_inp, direction, *, out=None, workspace=None, eps=1e-5, stage=None, mask="as-is"):
    from triangle_multiplicative_update_amd import triangle_multiplicative_update
    d = dev_inp
    m = d["mask"] if mask == "as-is" else mask
    return triangle_multiplicative_update(
        d["x"], direction, m, d["norm_in_weight"], d["norm_in_bias"], d["p_in_weight"],
        d["p_in_bias"], d["g_in_weight"], d["g_in_bias"], d["norm_out_weight"],
        d["norm_out_bias"], d["p_out_weight"], d["p_out_bias"], d["g_out_weight"],
        d["g_out_bias"], eps=eps, out=out, workspace=workspace, _stage=stage)


def planes(workspace: torch.Tensor, B: int, N: int, c: int):
    """Views of the a, b, y planes [c, B*N, n_pad] in a call's workspace."""
    n_pad = (N + 63) // 64 * 64
    elems = c * B * N * n_pad
    pb = (elems * 2 + 255) // 256 * 256
    out = []
    for k in range(3):
        raw = workspace[k * pb: k * pb + elems * 2]
        out.append(raw.view(torch.bfloat16).view(c, B * N, n_pad))
    return out


def plane_layout(v: np.ndarray, direction: str, which: str) -> np.ndarray:
    """Oracle [B, N, N, c] values -> the plane layout [c, B*N, N] of the workspace."""
    B, N, _, c = v.shape
    if which == "y" or direction == "outgoing":
        t = np.transpose(v, (3, 0, 1, 2))           # (ch, b, i, k)
    else:
        t = np.transpose(v, (3, 0, 2, 1))           # (ch, b, i, k) = v[b, k, i, ch]
    return np.ascontiguousarray(t).reshape(c, B * N, N)


def bf16_ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in bf16 ulps between two arrays of bf16 values (as float)."""
    def ordered(v):
        u = np.asarray(v, np.float32).view(np.uint32) >> 16
        u = u.astype(np.int64)
        return np.where(u & 0x8000, -(u & 0x7FFF), u)
    return np.abs(ordered(a) - ordered(b))


def stats(gpu: np.ndarray, ref: np.ndarray) -> dict:
    gpu = np.asarray(gpu, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    diff = np.abs(gpu - ref)
    n = ref.size
    return {
        "cells": int(n),
        "rel_rms": float(np.linalg.norm(gpu - ref) / max(np.linalg.norm(ref), 1e-300)),
        "tight_fail": int(np.count_nonzero(diff > TIGHT_ABS + np.abs(ref) * REL_SLOPE)),
        "hard_fail": int(np.count_nonzero(~(diff <= HARD_ABS + np.abs(ref) * REL_SLOPE))),
        "max_abs": float(diff.max()) if n else 0.0,
        "nonfinite": int(np.count_nonzero(~np.isfinite(gpu))),
    }


def assert_within_tolerance_slabs(gpu_slabs, ref_slabs, label: str) -> dict:
    """The same bar as assert_within_tolerance over every cell of an output
    given as matching slabs (iterables of arrays), without holding the whole
    difference in memory; the tail allowance is that of the whole output."""
    cells = tight = hard = nonfinite = 0
    sq_diff = sq_ref = 0.0
    max_abs = 0.0
    for g, r in zip(gpu_slabs, ref_slabs):
        s = stats(g, r)
        g = np.asarray(g, np.float64)
        r = np.asarray(r, np.float64)
        cells += s["cells"]
        tight += s["tight_fail"]
        hard += s["hard_fail"]
        nonfinite += s["nonfinite"]
        sq_diff += float(np.sum((g - r) ** 2))
        sq_ref += float(np.sum(r ** 2))
        max_abs = max(max_abs, s["max_abs"])
    rel = float(np.sqrt(sq_diff) / max(np.sqrt(sq_ref), 1e-300))
    allowed = math.floor(TAIL_PER_MILLION * 1e-6 * cells)
    summary = {"cells": cells, "rel_rms": rel, "tight_fail": tight, "hard_fail": hard,
               "max_abs": max_abs, "nonfinite": nonfinite}
    say(f"[parity] {label}: {summary} (tail allowance {allowed})")
    assert nonfinite == 0, f"{label}: non-finite outputs {summary}"
    assert rel <= REL_RMS_MAX, f"{label}: relative RMS {rel:.3e} > {REL_RMS_MAX}"
    assert hard == 0, f"{label}: {hard} cells beyond 2e-2 + |ref|/64"
    assert tight <= allowed, f"{label}: {tight} cells beyond 4e-3 + |ref|/64 (allowed {allowed})"
    return summary


def assert_within_tolerance(gpu, ref, label: str, sampled: bool = False) -> dict:
    s = stats(gpu, ref)
    allowed = math.ceil(TAIL_PER_MILLION * 1e-6 * s["cells"]) if sampled else \
        math.floor(TAIL_PER_MILLION * 1e-6 * s["cells"])
    say(f"[parity] {label}: {s} (tail allowance {allowed})")
    assert s["nonfinite"] == 0, f"{label}: non-finite outputs {s}"
    assert s["rel_rms"] <= REL_RMS_MAX, f"{label}: relative RMS {s['rel_rms']:.3e} > {REL_RMS_MAX}"
    assert s["hard_fail"] == 0, f"{label}: {s['hard_fail']} cells beyond 2e-2 + |ref|/64"
    assert s["tight_fail"] <= allowed, \
        f"{label}: {s['tight_fail']} cells beyond 4e-3 + |ref|/64 (allowed {allowed})"
    return s
