"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (one forward call through the C ABI).

At these sizes the oracle is evaluated on sampled output blocks (rows x columns
chosen across tile edges, the padded-mask boundary and at random), and the whole
output is checked against properties that hold at any size:
  * every cell finite;
  * on padded pairs (i >= L or j >= L) y = 0, so u = norm_out_bias and the
    output has the closed form sigmoid(z g_out^T + g_out_b) *
    (norm_out_bias p_out^T + p_out_b), checked on every padded pair.
"""

import zlib

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from oracle import trimul_oracle as T
from parity_utils import assert_within_tolerance, bf16_to_f64, call, say, to_device, workload_inputs

pytestmark = pytest.mark.gpu

FULL = [
    ("n768_c128_pad700", "outgoing"),
    ("n768_c128_pad700", "incoming"),
    ("b2_n512_c256_nobias", "outgoing"),
    ("b2_n512_c256_nobias", "incoming"),
    ("n1536_c128_pad1400", "outgoing"),
]


def _sample_indices(N, L, rng, k=6):
    edges = {0, 1, 63, 64, 127, 128, N // 2, N - 2, N - 1}
    if L:
        edges |= {L - 1, L, min(N - 1, L + 1)}
    rnd = set(rng.choice(N, size=k, replace=False).tolist())
    return sorted(i for i in edges | rnd if 0 <= i < N)


@pytest.mark.parametrize("name,direction", FULL)
def test_full_size_sampled(gpu, name, direction):
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
    assert np.isfinite(out_h).all()

    rng = np.random.default_rng(zlib.crc32(f"{name}/{direction}".encode()))
    rows = _sample_indices(wl.N, wl.mask_len if wl.mask == "padded" else 0, rng)
    cols = _sample_indices(wl.N, wl.mask_len if wl.mask == "padded" else 0, rng)
    gpu_s, ref_s = [], []
    for b in range(wl.B):
        _, ref = oracle.forward_block(inp, direction, rows, cols, batch=b)
        gpu_s.append(out_h[b][np.ix_(rows, cols)].astype(np.float64))
        ref_s.append(ref)
    assert_within_tolerance(np.stack(gpu_s), np.stack(ref_s), f"{name} {direction} sampled",
                            sampled=True)

    if wl.mask == "padded":
        L, N = wl.mask_len, wl.N
        pad = np.zeros((N, N), bool)
        pad[L:, :] = True
        pad[:, L:] = True
        prm = T.params_from_bits(inp)
        e = T.eps_as_f32(1e-5)
        x_pad = T.bf16_bits_to_f64(inp["x"][0][pad])                 # [P, c_z]
        z = T.ln_in(x_pad, prm, e, "kernel")
        u = np.broadcast_to(prm.ln_out_b, (z.shape[0], prm.ln_out_b.size))
        ref = T.output(z, u, prm)
        assert_within_tolerance(out_h[0][pad].astype(np.float64), ref,
                                f"{name} {direction} padded pairs (closed form)")
