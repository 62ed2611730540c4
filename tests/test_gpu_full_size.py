"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (one forward call through the C ABI), on every output cell.

The oracle runs the whole call at each size (N = 768, B = 2 N = 512 c = 256 and
N = 1536, each in both directions): every one of the output cells is
held to the bar (relative RMS, the 10-per-million tail rule on the whole
output, and the hard bound on every cell), compared in row slabs to bound the
host memory. On padded pairs (i >= L or j >= L) the output also has a closed
form: y = 0 there, so u = norm_out_bias and the output is
sigmoid(z g_out^T + g_out_b) * (norm_out_bias p_out^T + p_out_b).
"""

import gc

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from oracle import trimul_oracle as T
from parity_utils import (assert_within_tolerance, assert_within_tolerance_slabs, call, say,
                          to_device, workload_inputs)

pytestmark = pytest.mark.gpu

FULL = [
    ("n768_c128_pad700", "outgoing"),
    ("n768_c128_pad700", "incoming"),
    ("b2_n512_c256_nobias", "outgoing"),
    ("b2_n512_c256_nobias", "incoming"),
    ("n1536_c128_pad1400", "outgoing"),
    ("n1536_c128_pad1400", "incoming"),     # the direction its workload does not list
]

SLAB = 128   # output rows per compared slab


@pytest.mark.parametrize("name,direction", FULL)
def test_full_size_every_cell(gpu, name, direction):
    wl = si.WORKLOADS[name]
    inp = workload_inputs(name)
    say(f"[gpu] full size {name} {direction}")
    d = to_device(inp, gpu)
    with torch.no_grad():
        out = call(d, direction)
    torch.cuda.synchronize()
    out_h = out.float().cpu().numpy()     # bf16 values, exact in float32
    del out, d
    torch.cuda.empty_cache()

    say(f"[cpu] oracle {name} {direction}")
    ref = oracle.forward(inp, direction).out
    N = wl.N
    gpu_slabs = (out_h[b, r0:r0 + SLAB] for b in range(wl.B) for r0 in range(0, N, SLAB))
    ref_slabs = (ref[b, r0:r0 + SLAB] for b in range(wl.B) for r0 in range(0, N, SLAB))
    s = assert_within_tolerance_slabs(gpu_slabs, ref_slabs, f"{name} {direction} every cell")
    assert s["cells"] == wl.B * N * N * wl.c_z
    del ref
    gc.collect()

    if wl.mask == "padded":
        L = wl.mask_len
        pad = np.zeros((N, N), bool)
        pad[L:, :] = True
        pad[:, L:] = True
        prm = T.params_from_bits(inp)
        e = T.eps_as_f32(1e-5)
        x_pad = T.bf16_bits_to_f64(inp["x"][0][pad])                 # [P, c_z]
        z = T.ln_in(x_pad, prm, e, "kernel")
        u = np.broadcast_to(prm.ln_out_b, (z.shape[0], prm.ln_out_b.size))
        closed = T.output(z, u, prm)
        assert_within_tolerance(out_h[0][pad].astype(np.float64), closed,
                                f"{name} {direction} padded pairs (closed form)")


def test_maximum_extent_sampled(gpu):
    """The largest problem the 32-bit extent rule serves at c = 256 and B = 1:
    N = 2040, 2 * c * B * N * n_pad = 2 139 095 040 < 2^31 (N = 2048 is declined).
    The oracle runs on sampled output blocks (every row block of 64 pairs and the
    ragged last one, against columns across the 256-wide contraction tiles and
    the last column), every cell of those blocks held to the bar; the whole
    output is checked finite."""
    from triangle_multiplicative_update_amd import check_support
    N, c = 2040, 256
    check_support(1, N, c, c, "outgoing")
    with pytest.raises(NotImplementedError):
        check_support(1, 2048, c, c, "outgoing")
    wl = si.custom(1, N, c, mask="bernoulli", seed=2040)
    inp = si.generate(wl)
    say(f"[gpu] maximum extent N={N} c={c} outgoing")
    d = to_device(inp, gpu)
    with torch.no_grad():
        out = call(d, "outgoing")
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    rows = [0, 63, 64, 255, 256, 1023, 1024, 1983, 1984, 2039]
    cols = [0, 1, 255, 256, 511, 512, 1279, 1280, 2038, 2039]
    got = out[0][rows][:, cols].float().cpu().numpy().astype(np.float64)
    del out, d
    torch.cuda.empty_cache()
    _, ref = oracle.forward_block(inp, "outgoing", rows, cols)
    assert_within_tolerance(got, ref, f"N={N} c={c} sampled blocks", sampled=True)
