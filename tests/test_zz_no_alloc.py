"""GPU test of the allocation-free entry point ``trimul_forward_noalloc``.

It runs the kernels of ``trimul_forward`` with the a, b and y planes in the
library's fixed per-GPU device array instead of a caller workspace, so its
output must carry exactly the bits of ``trimul_forward`` on the same inputs.
Checked through the C ABI on two calls in a row, the second on a smaller
problem than the first (the array keeps the first call's planes), in both
directions, and on the typed decline above the array's size. Every output is
also held to the oracle's tolerance.
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from parity_utils import assert_within_tolerance, bf16_to_f64, say, to_device
from triangle_multiplicative_update_amd import _native, workspace_bytes
from triangle_multiplicative_update_amd._native import lib

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 64 << 20
ORDER = ("x", "mask") + si.PARAM_NAMES


def _ptrs(d):
    return [None if d[k] is None else d[k].data_ptr() for k in ORDER]


def _forward_with_workspace(d, B, N, c, code, out, stream):
    ws = torch.empty(workspace_bytes(B, N, c, "incoming" if code else "outgoing"),
                     dtype=torch.uint8, device=out.device)
    st = lib.trimul_forward(*_ptrs(d), B, N, c, c, code, 1e-5, out.data_ptr(), ws.data_ptr(),
                            ws.numel(), stream)
    assert st == 0, _native.last_error()
    return ws


def _noalloc(d, B, N, c, code, out, stream):
    return lib.trimul_forward_noalloc(*_ptrs(d), B, N, c, c, code, 1e-5, out.data_ptr(), stream)


CASES = [
    # (first call, second call): the second is smaller than the first
    (si.custom(1, 256, 128, mask="bernoulli", seed=31), si.custom(1, 77, 128, mask="padded",
                                                                   mask_len=60, seed=32)),
    (si.custom(1, 192, 256, mask="ones", biases=False, seed=33), si.custom(2, 45, 256, mask="bernoulli",
                                                                           seed=34)),
]


_warm = []


def _warm_up(gpu):
    """One call per process before any memory is compared: the first call on a
    device loads the library's device code there, and with it the array."""
    if _warm:
        return
    wl = si.custom(1, 8, 128, mask="none", seed=30)
    d = to_device(si.generate(wl), gpu)
    out = torch.empty_like(d["x"])
    say("[gpu] noalloc warm-up N=8")
    assert _noalloc(d, 1, 8, 128, 0, out, torch.cuda.current_stream(gpu).cuda_stream) == 0, \
        _native.last_error()
    torch.cuda.synchronize()
    _warm.append(True)


@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_noalloc_matches_forward(gpu, case, direction):
    code = 0 if direction == "outgoing" else 1
    stream = torch.cuda.current_stream(gpu).cuda_stream
    _warm_up(gpu)
    for wl in CASES[case]:
        assert workspace_bytes(wl.B, wl.N, wl.c, direction) <= SCRATCH_BYTES
        inp = si.generate(wl)
        d = to_device(inp, gpu)
        say(f"[gpu] noalloc {wl.name} {direction}")
        ref_out = torch.empty_like(d["x"])
        ws = _forward_with_workspace(d, wl.B, wl.N, wl.c, code, ref_out, stream)
        out = torch.full_like(d["x"], float("nan"))
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info(gpu)[0]
        st = _noalloc(d, wl.B, wl.N, wl.c, code, out, stream)
        assert st == 0, _native.last_error()
        torch.cuda.synchronize()
        assert torch.cuda.mem_get_info(gpu)[0] == free0, "device memory changed during the call"
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), \
            f"{wl.name} {direction}: output differs from trimul_forward's"
        assert_within_tolerance(bf16_to_f64(out), oracle.forward(inp, direction).out,
                                f"noalloc {wl.name} {direction}")
        del ws


def test_noalloc_declines_above_its_scratch(gpu):
    wl = si.custom(1, 288, 128, mask="none", seed=35)
    assert workspace_bytes(1, 288, 128, "outgoing") > SCRATCH_BYTES
    d = to_device(si.generate(wl), gpu)
    out = torch.zeros_like(d["x"])
    say("[gpu] noalloc decline N=288")
    st = _noalloc(d, 1, 288, 128, 0, out, torch.cuda.current_stream(gpu).cuda_stream)
    assert st == _native.TRIMUL_E_UNSUPPORTED
    assert "trimul_forward_noalloc" in _native.last_error()
    torch.cuda.synchronize()
    assert torch.count_nonzero(out.view(torch.int16)) == 0   # nothing was launched
    # the argument rules of trimul_forward apply unchanged
    st = _noalloc(d, 1, 288, 128, 2, out, None)
    assert st == _native.TRIMUL_E_INVALID and "direction" in _native.last_error()
