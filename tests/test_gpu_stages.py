"""GPU checks of the intermediate planes, canaries, determinism and identities.

The workspace layout (a, b, y planes, channel-major, documented in
include/trimul.h) is part of the contract, so the tests read the planes after a
call and compare them with the oracle's bf16 intermediates.
"""

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from parity_utils import (assert_within_tolerance, bf16_to_f64, call, planes,
                          plane_layout, say, to_device)
from triangle_multiplicative_update_amd import workspace_bytes

pytestmark = pytest.mark.gpu


def _ws(B, N, c, direction, device, fill=None):
    n = workspace_bytes(B, N, c, direction)
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    if fill is not None:
        ws.view(torch.bfloat16).fill_(fill)
    return ws


@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
@pytest.mark.parametrize("B,N,c", [(1, 136, 128), (2, 77, 128), (1, 72, 256)])
def test_planes_match_oracle(gpu, direction, B, N, c):
    wl = si.custom(B, N, c, mask="bernoulli", mask_p=0.8, seed=7 + N)
    inp = si.generate(wl)
    say(f"[gpu] planes {wl.name} {direction}")
    d = to_device(inp, gpu)
    ws = _ws(B, N, c, direction, gpu, fill=float("nan"))
    with torch.no_grad():
        out = call(d, direction, workspace=ws)
    torch.cuda.synchronize()
    ref = oracle.forward(inp, direction)
    pa, pb, py = planes(ws, B, N, c)
    report = {}
    for name, plane, want in (("a", pa, ref.a), ("b", pb, ref.b), ("y", py, ref.y)):
        got = bf16_to_f64(plane[:, :, :N])
        exp = plane_layout(want, direction, name).astype(np.float64)
        scale = float(np.sqrt(np.mean(exp ** 2)))
        diff = np.abs(got - exp)
        frac = np.count_nonzero(diff) / diff.size
        # fp32 (GPU) vs fp64 (oracle) before the single rounding: a difference is
        # one bf16 ulp of the value (2^-7 relative at most), or the effect of a
        # one-ulp flip of a z_in element of the same pair (|w| * ulp(z), a few
        # 1e-3 of the plane's scale), rare either way. y also inherits the flips
        # of a and b through the contraction.
        rel, floor, max_frac = (2.0 ** -7, 1e-2, 1e-2) if name != "y" else (2.0 ** -6, 1e-2, 0.2)
        worst = float(np.max(diff - (rel * np.abs(exp) + floor * scale)))
        report[name] = (frac, worst, max_frac)
        say(f"[planes] {name}: mismatch fraction {frac:.2e}, worst excess {worst:.3e} (scale {scale:.3e})")
        if name != "y":
            n_pad = plane.shape[-1]
            if n_pad > N:   # padded plane columns are written as +0.0
                tail = plane[:, :, N:].float().cpu().numpy()
                assert np.all(tail == 0) and not np.any(np.signbit(tail)), name
    for name, (frac, worst, max_frac) in report.items():
        assert worst <= 0, (name, report)
        assert frac <= max_frac, (name, report)
    # the output itself
    assert_within_tolerance(bf16_to_f64(out), ref.out, f"{wl.name} {direction}")


@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
def test_masked_rows_are_positive_zero(gpu, direction):
    B, N, c, L = 1, 100, 128, 70
    wl = si.custom(B, N, c, mask="padded", mask_len=L, seed=3)
    inp = si.generate(wl)
    say(f"[gpu] masked zeros {wl.name} {direction}")
    d = to_device(inp, gpu)
    ws = _ws(B, N, c, direction, gpu, fill=float("nan"))
    with torch.no_grad():
        call(d, direction, workspace=ws)
    torch.cuda.synchronize()
    pa, pb, py = planes(ws, B, N, c)
    for name, plane in (("a", pa), ("b", pb), ("y", py)):
        v = plane[:, :, :N].float().cpu().numpy()        # [c, N, N] (row, column)
        pad = np.zeros((N, N), bool)
        pad[L:, :] = True
        pad[:, L:] = True
        z = v[:, pad]
        assert np.all(z == 0) and not np.any(np.signbit(z)), name
        assert np.count_nonzero(v[:, ~pad]) > 0.9 * v[:, ~pad].size, name


def test_nan_canary_and_determinism(gpu):
    wl = si.custom(2, 130, 128, mask="bernoulli", seed=11)
    inp = si.generate(wl)
    say(f"[gpu] canary {wl.name}")
    d = to_device(inp, gpu)
    B, N, c = 2, 130, 128
    outs = []
    for rep in range(3):
        ws = _ws(B, N, c, "outgoing", gpu, fill=float("nan"))
        out = torch.full((B, N, N, c), float("nan"), dtype=torch.bfloat16, device=gpu)
        with torch.no_grad():
            call(d, "outgoing", out=out, workspace=ws)
        torch.cuda.synchronize()
        assert torch.isfinite(out).all()
        outs.append(out.view(torch.int16).cpu())
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
def test_stage1_repeats_bitwise(gpu, direction):
    # Stage 1 rotates LDS buffers across tiles (LayerNorm output, mask terms,
    # output staging) and overlaps the tiles; a buffer reused before every wave
    # is done with it shows up as planes that differ between repeated calls.
    # Full-size workload (N = 768, padded mask), 20 calls.
    inp = si.generate(si.WORKLOADS["n768_c128_pad700"])
    say(f"[gpu] stage-1 repeats {direction}")
    d = to_device(inp, gpu)
    ws = _ws(1, 768, 128, direction, gpu)
    a, b = planes(ws, 1, 768, 128)[:2]
    first = None
    for rep in range(20):
        with torch.no_grad():
            call(d, direction, workspace=ws, stage=1)
        if first is None:
            first = (a.view(torch.int16).clone(), b.view(torch.int16).clone())
        else:
            assert torch.equal(a.view(torch.int16), first[0]), f"plane a, call {rep} differs"
            assert torch.equal(b.view(torch.int16), first[1]), f"plane b, call {rep} differs"
    torch.cuda.synchronize()


def test_direction_identity_on_gpu(gpu):
    """y of the incoming direction on x equals y of the outgoing direction on x
    with its pair axes swapped (and the mask likewise)."""
    B, N, c = 1, 96, 128
    wl = si.custom(B, N, c, mask="bernoulli", seed=21)
    inp = si.generate(wl)
    inp_t = dict(inp)
    inp_t["x"] = np.ascontiguousarray(np.swapaxes(inp["x"], 1, 2))
    inp_t["mask"] = np.ascontiguousarray(np.swapaxes(inp["mask"], 1, 2))
    say("[gpu] direction identity")
    ws1 = _ws(B, N, c, "incoming", gpu)
    ws2 = _ws(B, N, c, "outgoing", gpu)
    with torch.no_grad():
        call(to_device(inp, gpu), "incoming", workspace=ws1)
        call(to_device(inp_t, gpu), "outgoing", workspace=ws2)
    torch.cuda.synchronize()
    y1 = planes(ws1, B, N, c)[2][:, :, :N].view(torch.int16).cpu()
    y2 = planes(ws2, B, N, c)[2][:, :, :N].view(torch.int16).cpu()
    assert torch.equal(y1, y2)


def test_mask_none_equals_ones_and_biases_none_equal_zero(gpu):
    B, N, c = 1, 70, 128
    wl = si.custom(B, N, c, mask="ones", seed=5)
    inp = si.generate(wl)
    say("[gpu] mask None / zero biases equivalence")
    d = to_device(inp, gpu)
    with torch.no_grad():
        o1 = call(d, "outgoing")
        o2 = call(d, "outgoing", mask=None)
        dz = dict(d)
        for k in ("p_in_bias", "g_in_bias", "p_out_bias", "g_out_bias"):
            dz[k] = torch.zeros_like(d[k])
        dn = dict(d)
        for k in ("p_in_bias", "g_in_bias", "p_out_bias", "g_out_bias"):
            dn[k] = None
        o3 = call(dz, "outgoing")
        o4 = call(dn, "outgoing")
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    # equal up to the sign of zero
    assert torch.equal(o3.float(), o4.float())


def test_stages_chain_equals_forward(gpu):
    B, N, c = 1, 88, 128
    wl = si.custom(B, N, c, mask="bernoulli", seed=8)
    inp = si.generate(wl)
    say("[gpu] stage chain == forward")
    d = to_device(inp, gpu)
    with torch.no_grad():
        o1 = call(d, "incoming")
        ws = _ws(B, N, c, "incoming", gpu)
        o2 = torch.empty_like(o1)
        for s in (1, 2, 3):
            call(d, "incoming", out=o2, workspace=ws, stage=s)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_batchless_and_mask_dtypes(gpu):
    N, c = 40, 128
    wl = si.custom(1, N, c, mask="bernoulli", seed=9)
    inp = si.generate(wl)
    say("[gpu] batchless and mask dtypes")
    d = to_device(inp, gpu)
    with torch.no_grad():
        o_ref = call(d, "outgoing")
        db = dict(d)
        db["x"] = d["x"][0]
        o_bl = call(db, "outgoing", mask=d["mask"][0].bool())
        o_f32 = call(d, "outgoing", mask=d["mask"].float())
    torch.cuda.synchronize()
    assert o_bl.shape == (N, N, c)
    assert torch.equal(o_bl.view(torch.int16), o_ref[0].view(torch.int16))
    assert torch.equal(o_f32.view(torch.int16), o_ref.view(torch.int16))


def test_declines_on_device(gpu):
    from triangle_multiplicative_update_amd import triangle_multiplicative_update
    N, c = 16, 128
    wl = si.custom(1, N, c, mask="ones", seed=1)
    d = to_device(si.generate(wl), gpu)
    with torch.no_grad():
        with pytest.raises(ValueError):
            call(d, "sideways")
        with pytest.raises(ValueError):   # out aliases x
            call(d, "outgoing", out=d["x"])
        with pytest.raises(NotImplementedError):
            triangle_multiplicative_update(d["x"], "outgoing", None, *[d[k] for k in (
                "norm_in_weight", "norm_in_bias", "p_in_weight", "p_in_bias", "g_in_weight",
                "g_in_bias", "norm_out_weight", "norm_out_bias", "p_out_weight", "p_out_bias",
                "g_out_weight", "g_out_bias")], precision="tf32")
    xg = d["x"].clone().requires_grad_(True)
    dg = dict(d)
    dg["x"] = xg
    with pytest.raises(NotImplementedError):
        call(dg, "outgoing")
