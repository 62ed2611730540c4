"""GPU edge cases of the served envelope and invariants of the kernels.

Page "Triangle Multiplicative Update (SM100 / SM103 / SM107)": sections
"Mathematics and numerics" (LayerNorm with eps, rounding points, a zero mask
giving +0.0), "Served today, and the typed declines" (a bias given on one side
only, the precision values, the parameter rows) and "Prepared class API" /
"Tests" (execute allocating nothing and never synchronising, the stream the
call is ordered on).
"""

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from parity_utils import (assert_within_tolerance, bf16_to_f64, call, planes, say, to_device)
from triangle_multiplicative_update_amd import (TriangleMultiplicativeUpdateFwd, prepare_weights,
                                               triangle_multiplicative_update, workspace_bytes)

pytestmark = pytest.mark.gpu

BF16_ONE = np.uint16(0x3F80)


def _ws(B, N, c, direction, device, fill=None):
    ws = torch.empty(workspace_bytes(B, N, c, direction), dtype=torch.uint8, device=device)
    if fill is not None:
        ws.view(torch.bfloat16).fill_(fill)
    return ws


def _check(inp, direction, label, device, eps=1e-5, ws=None):
    say(f"[gpu] {label} {direction}")
    d = to_device(inp, device)
    with torch.no_grad():
        out = call(d, direction, eps=eps, workspace=ws)
    torch.cuda.synchronize()
    ref = oracle.forward(inp, direction, eps=eps).out
    return assert_within_tolerance(bf16_to_f64(out), ref, f"{label} {direction}")


@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
@pytest.mark.parametrize("c", [128, 256])
@pytest.mark.parametrize("eps", [0.0, 1e-3])
def test_eps_values(gpu, direction, c, eps):
    """eps = 0 and eps = 1e-3 at a ragged N: the padded plane columns stay +0.0
    (a zero-variance row with eps = 0 is 0 * inf there) and the output matches
    the oracle computed with the same eps."""
    B, N = 1, 72
    wl = si.custom(B, N, c, mask="bernoulli", seed=500 + c)
    inp = si.generate(wl)
    ws = _ws(B, N, c, direction, gpu, fill=float("nan"))
    _check(inp, direction, f"{wl.name} eps={eps}", gpu, eps=eps, ws=ws)
    pa, pb, py = planes(ws, B, N, c)
    for name, plane in (("a", pa), ("b", pb)):
        tail = plane[:, :, N:].float().cpu().numpy()
        assert tail.size and np.all(tail == 0) and not np.any(np.signbit(tail)), name
    assert torch.isfinite(py[:, :, :N]).all()


@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
@pytest.mark.parametrize("c", [128, 256])
def test_zero_and_constant_pair_rows(gpu, direction, c):
    """Pair rows of x that are all zero or constant (variance 0: LayerNorm gives
    its bias exactly), as padded inputs in real models have."""
    B, N = 1, 80
    wl = si.custom(B, N, c, mask="padded", mask_len=60, seed=510 + c)
    inp = dict(si.generate(wl))
    x = inp["x"].copy()
    x[0, 60:, :, :] = 0                       # padded rows: all zero
    x[0, :, 70:, :] = 0                       # and columns
    x[0, 5, :, :] = np.uint16(0x4050)         # a constant row (3.25)
    x[0, :, 9, :] = np.uint16(0xBF00)         # a constant column (-0.5)
    x[0, 17, 23, :] = np.uint16(0x8000)       # one pair of -0.0
    inp["x"] = x
    _check(inp, direction, f"{wl.name} zero/constant rows", gpu)


@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
@pytest.mark.parametrize("side", ["in_value", "in_gate", "out_value", "out_gate"])
def test_one_sided_biases(gpu, direction, side):
    """One projection bias given, its partner None (= zero)."""
    wl = si.custom(1, 70, 128, mask="bernoulli", seed=520)
    inp = dict(si.generate(wl))
    drop = {"in_value": "g_in_bias", "in_gate": "p_in_bias", "out_value": "g_out_bias",
            "out_gate": "p_out_bias"}[side]
    inp[drop] = None
    _check(inp, direction, f"{wl.name} without {drop}", gpu)


@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
def test_precision_bfloat16_casts_once(gpu, direction):
    """fp32 x and parameters under precision='bfloat16' give exactly the bits of
    the call on tensors cast beforehand, and match the oracle on the cast bits."""
    wl = si.custom(1, 66, 128, mask="bernoulli", seed=530)
    inp = si.generate(wl)
    d = to_device(inp, gpu)
    rng = np.random.default_rng(531)
    # fp32 values that are not bf16-exact: the cast rounds them
    d32 = {k: (None if v is None else
               (v.float() * (1 + torch.from_numpy(rng.uniform(-3e-3, 3e-3, tuple(v.shape))).float().to(gpu))))
           for k, v in d.items()}
    d32["mask"] = d["mask"]
    cast = {k: (None if v is None else v.to(torch.bfloat16)) for k, v in d32.items()}
    say(f"[gpu] precision=bfloat16 {direction}")
    names = si.PARAM_NAMES
    with torch.no_grad():
        o32 = triangle_multiplicative_update(d32["x"], direction, d32["mask"],
                                             *[d32[k] for k in names], precision="bfloat16")
        oc = triangle_multiplicative_update(cast["x"], direction, cast["mask"],
                                            *[cast[k] for k in names])
        with pytest.raises(NotImplementedError, match="bfloat16"):
            triangle_multiplicative_update(d32["x"], direction, d32["mask"], *[d32[k] for k in names])
    torch.cuda.synchronize()
    assert o32.dtype == torch.bfloat16
    assert torch.equal(o32.view(torch.int16), oc.view(torch.int16))
    bits = {k: (None if v is None else v.view(torch.int16).cpu().numpy().view(np.uint16))
            for k, v in cast.items()}
    assert_within_tolerance(bf16_to_f64(o32), oracle.forward(bits, direction).out,
                            f"precision=bfloat16 {direction}")


@pytest.mark.parametrize("c", [128, 256])
def test_stage3_layernorm_in_has_stage1_bits(gpu, c):
    """Stage 3 recomputes LayerNorm_in: its z must carry stage 1's bits.

    With g_in = 0 and p_in = [I; I] (no in-biases, no mask) stage 1 writes
    a = b = sigmoid(0) z = z / 2 exactly, so plane a holds stage 1's z. With
    p_out = 0 and p_out_bias = 1 the output is bf16(sigmoid(g)) with g = 8 z +
    g_out_bias read from stage 3's own z. x is a per-channel base plus small
    noise and g_out_bias = -8 * (the channel's typical z), so g stays near 0,
    where one bf16 ulp of a z element moves sigmoid(g) by about eight bf16 ulps
    of the output; the hardware sigmoid's fp32 error moves it by at most one,
    and only next to a rounding midpoint.
    """
    B, N = 1, 96                # at c = 256 one full 64-pair tile and one ragged one
    rng = np.random.default_rng(540 + c)
    base = rng.standard_normal(c).astype(np.float32)
    noise = rng.standard_normal((B, N, N, c)).astype(np.float32) * np.float32(0.01)
    x = si.f32_to_bf16_bits(base + noise)
    wl = si.custom(B, N, c, mask="none", seed=541)
    inp = dict(si.generate(wl))
    inp["x"] = x
    eye = np.where(np.eye(c, dtype=bool), BF16_ONE, np.uint16(0)).astype(np.uint16)
    inp["p_in_weight"] = np.concatenate([eye, eye])
    inp["g_in_weight"] = np.zeros((2 * c, c), np.uint16)
    inp["p_in_bias"] = inp["g_in_bias"] = None
    inp["p_out_weight"] = np.zeros((c, c), np.uint16)
    inp["p_out_bias"] = np.full(c, BF16_ONE, np.uint16)
    inp["g_out_weight"] = np.where(np.eye(c, dtype=bool), np.uint16(0x4100), np.uint16(0)).astype(np.uint16)  # 8 I
    z_ref = oracle.forward(inp, "outgoing", keep_z=True).z[0]                       # [N, N, c]
    gb = -8.0 * np.median(z_ref.reshape(-1, c), axis=0)
    inp["g_out_bias"] = si.f32_to_bf16_bits(gb.astype(np.float32))
    d = to_device(inp, gpu)
    ws = _ws(B, N, c, "outgoing", gpu)
    say(f"[gpu] stage-3 z bits == stage-1 z bits, c = {c}")
    with torch.no_grad():
        out = call(d, "outgoing", workspace=ws)
    torch.cuda.synchronize()
    a = planes(ws, B, N, c)[0][:, :, :N].float().cpu().numpy().astype(np.float64)   # [c, i, k]
    z1 = 2.0 * np.transpose(a, (1, 2, 0))                                               # [i, j, c]
    assert np.array_equal(z1, z_ref) or np.mean(z1 != z_ref) < 1e-3   # stage 1 is LayerNorm_in
    gbias = oracle.bf16_bits_to_f64(inp["g_out_bias"])
    g = 8.0 * z1 + gbias
    assert np.mean(np.abs(g) < 1.0) > 0.5          # most gates sit on the steep part
    s = 1.0 / (1.0 + np.exp(-g))
    want = oracle.bf16_round(s)
    got = bf16_to_f64(out)[0]
    ulp = np.exp2(np.floor(np.log2(np.abs(want))) - 7)
    off = np.abs(got - want) / ulp
    assert off.max() <= 1.0, f"stage-3 z differs from stage 1's: {np.count_nonzero(off > 1)} cells"
    # a one-ulp difference only next to a rounding midpoint of the exact value
    near = np.abs(np.abs(s - want) / ulp - 0.5) < 1e-3
    assert np.all(near[off == 1.0]), int(np.count_nonzero(off[~near] == 1.0))


def test_execute_allocates_nothing_and_captures(gpu):
    """execute() allocates no device memory, and inside torch's graph capture it
    records the three launches; replays (with eager work and synchronisations
    between them, and a rewritten x) match eager calls bitwise."""
    wl = si.WORKLOADS["n64_c128_ones"]
    inp = si.generate(wl)
    d = to_device(inp, gpu)
    w = prepare_weights(*[d[n] for n in si.PARAM_NAMES])
    plan = TriangleMultiplicativeUpdateFwd(d["x"], "outgoing", 128, True, w.has_in_bias,
                                           w.has_out_bias).compile()
    ws = torch.empty(plan.get_workspace_size(), dtype=torch.uint8, device=gpu)
    out = torch.empty_like(d["x"])
    x = d["x"].clone()
    say("[gpu] execute: no allocation, graph capture")
    plan.execute(x, d["mask"], w, out, ws)        # first call: library state is set up
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info(gpu)[0]
    alloc0 = torch.cuda.memory_allocated(gpu)
    for _ in range(3):
        plan.execute(x, d["mask"], w, out, ws)
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info(gpu)[0] == free0
    assert torch.cuda.memory_allocated(gpu) == alloc0
    eager = out.clone()

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(gpu)
    side.wait_stream(torch.cuda.current_stream(gpu))
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            plan.execute(x, d["mask"], w, out, ws)
    torch.cuda.current_stream(gpu).wait_stream(side)
    torch.cuda.synchronize()
    x2 = to_device(si.generate(si.custom(1, 64, 128, mask="ones", seed=550)), gpu)["x"]
    for rep in range(4):
        src = d["x"] if rep % 2 == 0 else x2
        x.copy_(src)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        replay = out.clone()
        plan.execute(x, d["mask"], w, out, ws)
        torch.cuda.synchronize()
        assert torch.equal(replay.view(torch.int16), out.view(torch.int16)), f"replay {rep}"
        if rep % 2 == 0:
            assert torch.equal(replay.view(torch.int16), eager.view(torch.int16))
    del g


def test_side_stream_call(gpu):
    """stream= orders the call's casts, allocations and launches on that stream;
    memory allocated right after the call on the current stream does not
    disturb it."""
    wl = si.custom(1, 200, 128, mask="bernoulli", seed=560)
    inp = si.generate(wl)
    d = to_device(inp, gpu)
    say("[gpu] side-stream call")
    with torch.no_grad():
        ref = call(d, "outgoing")
        torch.cuda.synchronize()
        s = torch.cuda.Stream(gpu)
        fmask = d["mask"].float()                 # cast inside the call, on s
        out = triangle_multiplicative_update(d["x"], "outgoing", fmask,
                                             *[d[k] for k in si.PARAM_NAMES], stream=s)
        junk = [torch.full((1 << 22,), 7.0, device=gpu) for _ in range(8)]   # current stream
        torch.cuda.current_stream(gpu).wait_stream(s)
        out2 = triangle_multiplicative_update(d["x"], "outgoing", d["mask"],
                                              *[d[k] for k in si.PARAM_NAMES],
                                              stream=s.cuda_stream)   # a raw handle
        torch.cuda.current_stream(gpu).wait_stream(s)
    torch.cuda.synchronize()
    del junk
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(out2.view(torch.int16), ref.view(torch.int16))
