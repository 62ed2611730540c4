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


def _z_flip_bound(inp, z, half):
    """Per-channel bound on how far a or b (rows [half*c, half*c + c) of the
    in-projections) moves when one element q of a pair's z_in takes the
    neighbouring bf16 value (the GPU's fp32 LayerNorm and the oracle's fp64
    one can round a z element to different sides of a midpoint).

    a = sigmoid(G) P m with P = z p^T + p_b, G = z g^T + g_b and 0 <= m <= 1; a
    change dz in z_q moves P by p[ch, q] dz and G by g[ch, q] dz, and sigmoid
    has slope at most 1/4, so |da| <= (|p[ch, q]| + |P| |g[ch, q]| / 4) |dz|,
    with |dz| at most the largest ulp of any z element."""
    f = oracle.bf16_bits_to_f64
    c = inp["p_in_weight"].shape[0] // 2
    rows = slice(half * c, half * c + c)
    p_w, g_w = f(inp["p_in_weight"])[rows], f(inp["g_in_weight"])[rows]
    p_b = np.zeros(c) if inp["p_in_bias"] is None else f(inp["p_in_bias"])[rows]
    zz = np.asarray(z, np.float64).reshape(-1, z.shape[-1])
    P_max = np.abs(zz @ p_w.T + p_b).max(axis=0)                          # [c]
    az = np.abs(zz[zz != 0])
    ulp_max = float(np.exp2(np.floor(np.log2(az.max())) - 7)) if az.size else 0.0
    return (np.abs(p_w).max(axis=1) + P_max * np.abs(g_w).max(axis=1) / 4) * ulp_max


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
    ref = oracle.forward(inp, direction, keep_z=True)
    pa, pb, py = planes(ws, B, N, c)
    got = {}
    for half, (name, plane, want) in enumerate((("a", pa, ref.a), ("b", pb, ref.b))):
        g = bf16_to_f64(plane[:, :, :N])
        got[name] = g
        exp = plane_layout(want, direction, name).astype(np.float64)
        diff = np.abs(g - exp)
        frac = np.count_nonzero(diff) / diff.size
        # Before its one rounding the GPU's a is fp32, the oracle's fp64: where
        # they round apart the results are one bf16 ulp apart (<= 2^-7 |a|).
        # Where a z element rounded apart, _z_flip_bound applies, twice (two
        # flipped elements in one pair: about 3e-5 of the pairs at the
        # measured flip rates; three: about 1e-7).
        bound = 2.0 ** -7 * np.abs(exp) + 2 * _z_flip_bound(inp, ref.z, half)[:, None, None]
        worst = float(np.max(diff - bound))
        say(f"[planes] {name}: mismatch fraction {frac:.2e}, worst excess {worst:.3e}")
        assert worst <= 0, name
        assert frac <= 1e-2, name
        n_pad = plane.shape[-1]
        if n_pad > N:   # padded plane columns are written as +0.0
            tail = plane[:, :, N:].float().cpu().numpy()
            assert np.all(tail == 0) and not np.any(np.signbit(tail)), name
    # y against the contraction of the GPU's own a and b planes: the products of
    # bf16 values are exact in fp32, so in any summation order the fp32 sum is
    # within gamma_N sum_k |a_k b_k| of the exact one (gamma_N = N u / (1 - N u),
    # u = 2^-24), and the one bf16 rounding adds at most 2^-8 of the value.
    A = got["a"].reshape(c, B, N, N)
    Bp = got["b"].reshape(c, B, N, N)
    Y = A @ np.swapaxes(Bp, -1, -2)
    S = np.abs(A) @ np.swapaxes(np.abs(Bp), -1, -2)
    gam = N * 2.0 ** -24 / (1 - N * 2.0 ** -24)
    y_got = bf16_to_f64(py[:, :, :N]).reshape(c, B, N, N)
    bound = gam * S + 2.0 ** -8 * (np.abs(Y) + gam * S)
    worst = float(np.max(np.abs(y_got - Y) - bound))
    say(f"[planes] y: worst excess over the contraction of the GPU planes {worst:.3e}")
    assert worst <= 0
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
