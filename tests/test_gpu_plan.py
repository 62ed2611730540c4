"""GPU tests of the prepared class API and the captured graphs.

Page "Triangle Multiplicative Update (SM100 / SM103 / SM107)", section
"Prepared class API": weights prepared once, a plan per geometry whose
``execute`` allocates nothing, and a graph per buffer set. The plan and the
graph must produce exactly the drop-in function's bits, and a graph must read
its inputs' contents at each launch (checked over several launches with eager
work and synchronisations between them).
"""

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from parity_utils import assert_within_tolerance, bf16_to_f64, call, say, to_device
from triangle_multiplicative_update_amd import (TriangleMultiplicativeUpdateFwd, prepare_weights,
                                               workspace_bytes)

pytestmark = pytest.mark.gpu


def _plan_and_buffers(d, wl, direction, device):
    w = prepare_weights(*[d[n] for n in si.PARAM_NAMES])
    plan = TriangleMultiplicativeUpdateFwd(d["x"], direction, wl.c, d["mask"] is not None,
                                           w.has_in_bias, w.has_out_bias).compile()
    ws = torch.empty(plan.get_workspace_size(), dtype=torch.uint8, device=device)
    out = torch.empty_like(d["x"])
    return plan, w, ws, out


@pytest.mark.parametrize("name,direction", [("n64_c128_ones", "outgoing"), ("n256_c128_bern", "incoming")])
def test_execute_matches_function(gpu, name, direction):
    wl = si.WORKLOADS[name]
    inp = si.generate(wl)
    d = to_device(inp, gpu)
    say(f"[gpu] plan execute {name} {direction}")
    with torch.no_grad():
        ref = call(d, direction)
    plan, w, ws, out = _plan_and_buffers(d, wl, direction, gpu)
    plan.execute(d["x"], d["mask"], w, out, ws)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


def test_plan_flag_mismatch_raises(gpu):
    wl = si.WORKLOADS["n64_c128_ones"]
    d = to_device(si.generate(wl), gpu)
    plan, w, ws, out = _plan_and_buffers(d, wl, "outgoing", gpu)
    with pytest.raises(ValueError, match="has_mask"):
        plan.execute(d["x"], None, w, out, ws)
    w_nobias = prepare_weights(*[None if n.endswith("_bias") and n.startswith(("p_", "g_")) else d[n]
                                 for n in si.PARAM_NAMES])
    with pytest.raises(ValueError, match="has_in_bias"):
        plan.execute(d["x"], d["mask"], w_nobias, out, ws)


@pytest.mark.parametrize("name,direction", [("n64_c128_ones", "outgoing"), ("n256_c128_bern", "incoming"),
                                            ("b2_n512_c256_nobias", "outgoing")])
def test_graph_replays_follow_inputs(gpu, name, direction):
    wl = si.WORKLOADS[name]
    inp = si.generate(wl)
    d = to_device(inp, gpu)
    say(f"[gpu] graph {name} {direction}")
    plan, w, ws, out = _plan_and_buffers(d, wl, direction, gpu)
    eager_out = torch.empty_like(out)
    eager_ws = torch.empty_like(ws)
    g = plan.make_graph(d["x"], d["mask"], w, out, ws)
    x0 = d["x"].clone()
    try:
        for rep in range(3):
            # new input contents in place, then the graph and an eager call on them
            if rep == 1:
                d["x"].copy_(torch.flip(x0, dims=[1]))
            elif rep == 2:
                d["x"].copy_(-x0)
            g.launch()
            torch.cuda.synchronize()
            plan.execute(d["x"], d["mask"], w, eager_out, eager_ws)
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), eager_out.view(torch.int16)), f"replay {rep}"
            out.zero_()
            torch.cuda.synchronize()
        # a launch on a side stream, ordered after the producer of x
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g.launch(stream=s)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager_out.view(torch.int16)), "side stream"
    finally:
        g.close()
    # the last replay against the oracle, on the negated x
    if wl.N <= 256:
        inp2 = dict(inp)
        inp2["x"] = (np.asarray(inp["x"]).view(np.uint16) ^ np.uint16(0x8000)).view(inp["x"].dtype)
        ref = oracle.forward(inp2, direction)
        assert_within_tolerance(bf16_to_f64(out.cpu()), ref.out, f"graph {name} {direction}")
