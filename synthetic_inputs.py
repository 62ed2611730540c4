"""Seeded synthetic inputs for the triangle multiplicative update.

This module feeds both sides of every comparison: the tests and the benchmark
draw inputs here and hand the same bits to the CPU oracle and to the GPU library
(neither of which imports it). It only draws random numbers and stores them as
bf16 bit patterns; it holds none of the operation's arithmetic.

Distributions follow the workload descriptions for the operation (pair
representation x ~ N(0, s^2); projection weights ~ N(0, 1/fan_in); biases
~ N(0, 0.02^2); LayerNorm weights ~ 1 + N(0, 0.1^2)). Parameter shapes follow the
page "Triangle Multiplicative Update (SM100 / SM103 / SM107)", section
"Mathematics and numerics": p_in/g_in are [2c, c_z] with rows [a; b], p_out is
[c_z, c], g_out is [c_z, c_z], LayerNorm vectors are [c_z] (in) and [c] (out).

Every draw is float32 from ``numpy.random.default_rng(seed)``, scaled in float32,
then rounded to bf16 with round-to-nearest-even. The draw order is fixed: x, mask,
norm_in_w, norm_in_b, p_in_w, p_in_b, g_in_w, g_in_b, norm_out_w, norm_out_b,
p_out_w, p_out_b, g_out_w, g_out_b. Projection biases are always drawn (so the
stream does not depend on whether they are used) and dropped when ``biases`` is
False.
"""

from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

PARAM_NAMES = (
    "norm_in_weight", "norm_in_bias", "p_in_weight", "p_in_bias",
    "g_in_weight", "g_in_bias", "norm_out_weight", "norm_out_bias",
    "p_out_weight", "p_out_bias", "g_out_weight", "g_out_bias",
)
OPTIONAL_BIASES = ("p_in_bias", "g_in_bias", "p_out_bias", "g_out_bias")


def f32_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern (uint16), round to nearest even. Finite inputs."""
    # For finite float32 the sum stays below 2**32, so uint32 arithmetic is exact.
    u = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32)
    r = (u >> 16) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    return r.astype(np.uint16)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic problem: shape, input distributions and mask structure."""

    name: str
    B: int
    N: int
    c_z: int
    c: int
    directions: tuple
    x_std: float = 1.0
    mask: str = "ones"        # "ones" | "bernoulli" | "padded" | "none"
    mask_p: float = 0.9       # p(valid) for "bernoulli"
    mask_len: int = 0         # valid length L for "padded"
    biases: bool = True
    seed: int = 0

    @property
    def pairs(self) -> int:
        return self.B * self.N * self.N


# The five workloads the method is exercised on (names carry their sizes).
WORKLOADS: Dict[str, Workload] = {
    "n64_c128_ones": Workload("n64_c128_ones", 1, 64, 128, 128, ("outgoing",)),
    "n256_c128_bern": Workload("n256_c128_bern", 1, 256, 128, 128, ("incoming",),
                               mask="bernoulli", mask_p=0.9),
    "n768_c128_pad700": Workload("n768_c128_pad700", 1, 768, 128, 128,
                                 ("outgoing", "incoming"), mask="padded", mask_len=700),
    "b2_n512_c256_nobias": Workload("b2_n512_c256_nobias", 2, 512, 256, 256,
                                    ("outgoing", "incoming"), biases=False),
    "n1536_c128_pad1400": Workload("n1536_c128_pad1400", 1, 1536, 128, 128, ("outgoing",),
                                   x_std=2.0, mask="padded", mask_len=1400),
}

# The throughput workload: N=768, c_z=c=128, B=1.
BENCH_WORKLOAD = "n768_c128_pad700"


def _normal_bits(rng: np.random.Generator, shape, std: float, mean: float = 0.0) -> np.ndarray:
    d = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        d *= np.float32(std)
    if mean != 0.0:
        d += np.float32(mean)
    return f32_to_bf16_bits(d)


def make_mask(wl: Workload, rng: np.random.Generator) -> Optional[np.ndarray]:
    B, N = wl.B, wl.N
    one = np.uint16(0x3F80)  # bf16 1.0
    if wl.mask == "none":
        return None
    if wl.mask == "ones":
        return np.full((B, N, N), one, dtype=np.uint16)
    if wl.mask == "bernoulli":
        keep = rng.random(size=(B, N, N), dtype=np.float32) < np.float32(wl.mask_p)
        return np.where(keep, one, np.uint16(0)).astype(np.uint16)
    if wl.mask == "padded":
        L = wl.mask_len
        idx = np.arange(N)
        keep = (idx[:, None] < L) & (idx[None, :] < L)
        return np.broadcast_to(np.where(keep, one, np.uint16(0)).astype(np.uint16), (B, N, N)).copy()
    raise ValueError(f"unknown mask kind {wl.mask!r}")


def generate(wl: Workload) -> Dict[str, Optional[np.ndarray]]:
    """Draw every input of one workload as bf16 bit patterns (numpy uint16).

    Returns a dict with "x" [B,N,N,c_z], "mask" [B,N,N] or None, and the twelve
    parameters by name (projection biases None when ``wl.biases`` is False).
    """
    rng = np.random.default_rng(wl.seed)
    B, N, cz, c = wl.B, wl.N, wl.c_z, wl.c
    out: Dict[str, Optional[np.ndarray]] = {}
    out["x"] = _normal_bits(rng, (B, N, N, cz), wl.x_std)
    out["mask"] = make_mask(wl, rng)
    out["norm_in_weight"] = _normal_bits(rng, (cz,), 0.1, 1.0)
    out["norm_in_bias"] = _normal_bits(rng, (cz,), 0.02)
    out["p_in_weight"] = _normal_bits(rng, (2 * c, cz), 1.0 / np.sqrt(cz))
    out["p_in_bias"] = _normal_bits(rng, (2 * c,), 0.02)
    out["g_in_weight"] = _normal_bits(rng, (2 * c, cz), 1.0 / np.sqrt(cz))
    out["g_in_bias"] = _normal_bits(rng, (2 * c,), 0.02)
    out["norm_out_weight"] = _normal_bits(rng, (c,), 0.1, 1.0)
    out["norm_out_bias"] = _normal_bits(rng, (c,), 0.02)
    out["p_out_weight"] = _normal_bits(rng, (cz, c), 1.0 / np.sqrt(c))
    out["p_out_bias"] = _normal_bits(rng, (cz,), 0.02)
    out["g_out_weight"] = _normal_bits(rng, (cz, cz), 1.0 / np.sqrt(cz))
    out["g_out_bias"] = _normal_bits(rng, (cz,), 0.02)
    if not wl.biases:
        for k in OPTIONAL_BIASES:
            out[k] = None
    return out


def custom(B: int, N: int, c: int, *, c_z: Optional[int] = None, x_std: float = 1.0,
           mask: str = "bernoulli", mask_p: float = 0.9, mask_len: int = 0,
           biases: bool = True, seed: int = 0, directions=("outgoing", "incoming")) -> Workload:
    """A workload of arbitrary size (parity cases, ragged tails, edge cases)."""
    cz = c if c_z is None else c_z
    name = f"b{B}_n{N}_c{c}_{mask}_s{seed}"
    return Workload(name, B, N, cz, c, tuple(directions), x_std=x_std, mask=mask,
                    mask_p=mask_p, mask_len=mask_len, biases=biases, seed=seed)
