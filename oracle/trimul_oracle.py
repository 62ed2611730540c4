"""Plain CPU fp64 oracle of the triangle multiplicative update.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import or call this module. It shares no code
with the HIP path and imports nothing from it; its only dependency is numpy.

What it computes: the formula on the page "Triangle Multiplicative Update (SM100 /
SM103 / SM107)", section "Mathematics and numerics", for every pair (i, j) of a
batch entry with pair mask m:

  z_in = LayerNorm_{c_z}(x; norm_in_weight, norm_in_bias, eps)
  a    = sigmoid(z_in g_in[:c]^T + g_in_b[:c]) * (z_in p_in[:c]^T + p_in_b[:c]) * m
  b    = sigmoid(z_in g_in[c:]^T + g_in_b[c:]) * (z_in p_in[c:]^T + p_in_b[c:]) * m
  y    = einsum("bikc,bjkc->bijc", a, b)   outgoing
         einsum("bkic,bkjc->bijc", a, b)   incoming
  u    = LayerNorm_c(y; norm_out_weight, norm_out_bias, eps)
  out  = sigmoid(z_in g_out^T + g_out_b) * (u p_out^T + p_out_b)

with every bias optional (None = zero) and the output unmasked.

Rounding points (same section, "rounding points" paragraph), inserted when
``rounding="kernel"``: the LayerNormed operands z_in and u are rounded once to
bf16; a and b are rounded once to bf16 after the mask multiply (a zero mask gives
exactly +0.0); y is rounded once to bf16. The final output is left unrounded in
fp64: it is the comparison target for a bf16 result. ``rounding="none"`` is the
pure formula in fp64 with no rounding at all.

Readings taken where the page is silent (each is listed in the design notes):
  * LayerNorm uses the biased variance (divide by n), eps inside the square root,
    the affine after normalisation, and two passes (mean, then mean of squared
    deviations).
  * eps is taken at float32 precision (the value a float32 kernel sees).
  * The g_out gate reads the same bf16-rounded z_in as the input projections.
  * sigmoid is exact: 1 / (1 + exp(-t)).
  * a and b are the fp64 product sigmoid(G) * P * m rounded once; "+ 0.0" turns a
    -0.0 product into +0.0 and changes no other value.
  * The contraction sums k < N only (padding contributes nothing).

All bf16 values are held in float32 arrays (bf16 is exactly representable in
float32) to halve the memory of large cases; every sum runs in fp64.
"""

from __future__ import annotations

import dataclasses
from typing import Dict, Optional, Sequence

import numpy as np

_BF16_MIN_EXP_QUANTUM = -133       # spacing of bf16 subnormals: 2**-133
_BF16_MAX = float.fromhex("0x1.fep127")
_BF16_OVERFLOW_EDGE = _BF16_MAX + 2.0 ** (127 - 8)   # midpoint above the largest bf16


# --------------------------------------------------------------------------- #
# bf16 helpers                                                                #
# --------------------------------------------------------------------------- #

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def bf16_round(v: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even, in one step.

    bf16 keeps 8 significant bits (1 implicit + 7 stored) and float32's exponent
    range. For |v| in [2**e, 2**(e+1)) the bf16 spacing is 2**(e-7), never finer
    than the subnormal spacing 2**-133. Values at or beyond the midpoint above
    the largest finite bf16 become +-inf; NaN stays NaN; the sign of zero is kept.
    Returns float64 holding the rounded values.
    """
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty_like(v)
    flat_v, flat_o = v.reshape(-1), out.reshape(-1)
    step = 1 << 18                       # chunks keep the temporaries in cache
    for s0 in range(0, flat_v.size, step):
        flat_o[s0:s0 + step] = _bf16_round_chunk(flat_v[s0:s0 + step])
    return out


def _bf16_round_chunk(v: np.ndarray) -> np.ndarray:
    # Normal bf16 range: float64 has 52 fraction bits, bf16 keeps 7, so round the
    # float64 bit pattern at bit 45 (ties to even); a carry ripples into the
    # exponent, which is the correct result at a binade boundary.
    u = v.view(np.uint64)
    r = (u >> np.uint64(45)) & np.uint64(1)
    r += np.uint64((1 << 44) - 1)
    r += u
    r &= np.uint64(0xFFFFE00000000000)
    out = r.view(np.float64)
    a = np.abs(v)
    if not (a.max(initial=0.0) < _BF16_OVERFLOW_EDGE):   # also true when a NaN is present
        special = ~np.isfinite(v)
        out[special] = v[special]                        # NaN and +-inf unchanged
        big = np.isfinite(v) & (a >= _BF16_OVERFLOW_EDGE)
        out[big] = np.copysign(np.inf, v[big])           # beyond the largest bf16
    tiny = (a < 2.0 ** -126) & (v != 0.0)
    if np.any(tiny):
        # Below the smallest normal bf16 (2**-126) the spacing is fixed at 2**-133.
        vt = v[tiny]
        scaled = np.ldexp(vt, -_BF16_MIN_EXP_QUANTUM)                 # exact
        out[tiny] = np.ldexp(np.rint(scaled), _BF16_MIN_EXP_QUANTUM)  # rint: half to even
    return out


def _to_store(v: np.ndarray, rounding: str) -> np.ndarray:
    """Apply a rounding point: bf16 in "kernel" mode, identity in "none" mode."""
    if rounding == "kernel":
        return bf16_round(v).astype(np.float32)
    return v


# --------------------------------------------------------------------------- #
# the steps of the formula                                                    #
# --------------------------------------------------------------------------- #

def layer_norm(v: np.ndarray, w: np.ndarray, b: np.ndarray, eps: float) -> np.ndarray:
    """LayerNorm over the last axis in fp64: two passes, biased variance.

    mean = sum(v)/n; var = sum((v - mean)^2)/n; (v - mean)/sqrt(var + eps) * w + b.
    """
    v = np.asarray(v, dtype=np.float64)
    n = v.shape[-1]
    mean = v.sum(axis=-1, keepdims=True) / n
    d = v - mean
    var = (d * d).sum(axis=-1, keepdims=True) / n
    return d / np.sqrt(var + eps) * w + b


def sigmoid(t: np.ndarray) -> np.ndarray:
    """Exact logistic function 1 / (1 + exp(-t)) in fp64."""
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-np.asarray(t, dtype=np.float64)))


@dataclasses.dataclass
class Params:
    """The twelve parameters as fp64 arrays (biases default to zero)."""

    ln_in_w: np.ndarray
    ln_in_b: np.ndarray
    p_in: np.ndarray       # [2c, c_z]
    p_in_b: np.ndarray     # [2c]
    g_in: np.ndarray       # [2c, c_z]
    g_in_b: np.ndarray     # [2c]
    ln_out_w: np.ndarray
    ln_out_b: np.ndarray
    p_out: np.ndarray      # [c_z, c]
    p_out_b: np.ndarray    # [c_z]
    g_out: np.ndarray      # [c_z, c_z]
    g_out_b: np.ndarray    # [c_z]

    @property
    def c(self) -> int:
        return self.p_in.shape[0] // 2


def params_from_bits(inp: Dict[str, Optional[np.ndarray]]) -> Params:
    """Build fp64 parameters from bf16 bit patterns; a missing bias is zero."""
    def req(name):
        if inp.get(name) is None:
            raise ValueError(f"{name} is required")
        return bf16_bits_to_f64(inp[name])

    def opt(name, n):
        return np.zeros(n) if inp.get(name) is None else bf16_bits_to_f64(inp[name])

    p_in = req("p_in_weight")
    c2, cz = p_in.shape
    return Params(
        ln_in_w=req("norm_in_weight"), ln_in_b=req("norm_in_bias"),
        p_in=p_in, p_in_b=opt("p_in_bias", c2),
        g_in=req("g_in_weight"), g_in_b=opt("g_in_bias", c2),
        ln_out_w=req("norm_out_weight"), ln_out_b=req("norm_out_bias"),
        p_out=req("p_out_weight"), p_out_b=opt("p_out_bias", cz),
        g_out=req("g_out_weight"), g_out_b=opt("g_out_bias", cz),
    )


def eps_as_f32(eps: float) -> float:
    return float(np.float32(eps))


def ln_in(x_pairs: np.ndarray, prm: Params, eps: float, rounding: str) -> np.ndarray:
    """z_in for a block of pairs [..., c_z] (one rounding point in kernel mode)."""
    return _to_store(layer_norm(x_pairs, prm.ln_in_w, prm.ln_in_b, eps), rounding)


def gated_projection(z: np.ndarray, m: np.ndarray, prm: Params, rounding: str):
    """a and b for a block of pairs: z [..., c_z], m [...] -> ([..., c], [..., c]).

    a = sigmoid(z g_in[:c]^T + g_in_b[:c]) * (z p_in[:c]^T + p_in_b[:c]) * m, b
    likewise with rows [c:]; each rounded once (kernel mode), +0.0 for m = 0.
    """
    c = prm.c
    z = np.asarray(z, dtype=np.float64)
    P = z @ prm.p_in.T + prm.p_in_b
    G = z @ prm.g_in.T + prm.g_in_b
    mm = np.asarray(m, dtype=np.float64)[..., None]
    a = sigmoid(G[..., :c]) * P[..., :c] * mm + 0.0
    b = sigmoid(G[..., c:]) * P[..., c:] * mm + 0.0
    return _to_store(a, rounding), _to_store(b, rounding)


def ln_out(y: np.ndarray, prm: Params, eps: float, rounding: str) -> np.ndarray:
    """u = LayerNorm_c(y) (one rounding point in kernel mode)."""
    return _to_store(layer_norm(y, prm.ln_out_w, prm.ln_out_b, eps), rounding)


def output(z: np.ndarray, u: np.ndarray, prm: Params) -> np.ndarray:
    """out = sigmoid(z g_out^T + g_out_b) * (u p_out^T + p_out_b), fp64, unrounded."""
    z = np.asarray(z, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    return sigmoid(z @ prm.g_out.T + prm.g_out_b) * (u @ prm.p_out.T + prm.p_out_b)


def contract_outgoing(a_rows: np.ndarray, b_rows: np.ndarray) -> np.ndarray:
    """y[i, j, ch] = sum_k a[i, k, ch] * b[j, k, ch]  (one batch entry), fp64.

    a_rows [I, K, c], b_rows [J, K, c] -> [I, J, c].
    """
    A = np.ascontiguousarray(np.moveaxis(np.asarray(a_rows, np.float64), -1, 0))  # [c, I, K]
    Bm = np.ascontiguousarray(np.moveaxis(np.asarray(b_rows, np.float64), -1, 0))  # [c, J, K]
    Y = np.matmul(A, np.swapaxes(Bm, 1, 2))                                           # [c, I, J]
    return np.moveaxis(Y, 0, -1)


def contract_incoming(a_cols: np.ndarray, b_cols: np.ndarray) -> np.ndarray:
    """y[i, j, ch] = sum_k a[k, i, ch] * b[k, j, ch]  (one batch entry), fp64.

    a_cols [K, I, c], b_cols [K, J, c] -> [I, J, c].
    """
    A = np.ascontiguousarray(np.moveaxis(np.asarray(a_cols, np.float64), -1, 0))  # [c, K, I]
    Bm = np.ascontiguousarray(np.moveaxis(np.asarray(b_cols, np.float64), -1, 0))  # [c, K, J]
    Y = np.matmul(np.swapaxes(A, 1, 2), Bm)                                           # [c, I, J]
    return np.moveaxis(Y, 0, -1)


# --------------------------------------------------------------------------- #
# whole-problem drivers                                                       #
# --------------------------------------------------------------------------- #

@dataclasses.dataclass
class Intermediates:
    """Per-stage values of one call (bf16-exact in kernel mode, stored as float32)."""

    z: Optional[np.ndarray]   # [B, N, N, c_z] (None when not kept)
    a: np.ndarray             # [B, N, N, c]
    b: np.ndarray             # [B, N, N, c]
    y: np.ndarray             # [B, N, N, c]
    out: np.ndarray           # [B, N, N, c_z] fp64 (unrounded)


def _mask_f64(inp, B, N) -> np.ndarray:
    m = inp.get("mask")
    if m is None:
        return np.ones((B, N, N))
    m = bf16_bits_to_f64(m)
    if m.ndim == 2:
        m = m[None]
    return m


def _x_f64_rows(x_bits: np.ndarray, b: int, rows) -> np.ndarray:
    return bf16_bits_to_f64(x_bits[b, rows])


def forward(inp: Dict[str, Optional[np.ndarray]], direction: str, *, eps: float = 1e-5,
            rounding: str = "kernel", keep_z: bool = False, row_block: int = 64,
            ch_block: int = 16) -> Intermediates:
    """Whole forward pass on bf16 inputs (bit patterns).

    ``inp`` holds "x" [B,N,N,c_z] (or [N,N,c_z]), optional "mask" [B,N,N] (or
    [N,N]) and the twelve named parameters, all as bf16 bit patterns. The
    pairwise steps run over ``row_block`` rows of pairs at a time and the
    contraction over ``ch_block`` channels at a time, only to bound memory: every
    value is computed independently of the blocking.
    """
    if row_block < 1 or ch_block < 1:
        raise ValueError("row_block and ch_block must be >= 1")
    if direction not in ("outgoing", "incoming"):
        raise ValueError(f"direction must be 'outgoing' or 'incoming', got {direction!r}")
    if rounding not in ("kernel", "none"):
        raise ValueError(f"rounding must be 'kernel' or 'none', got {rounding!r}")
    x_bits = inp["x"]
    if x_bits.ndim == 3:
        x_bits = x_bits[None]
    B, N, _, cz = x_bits.shape
    prm = params_from_bits(inp)
    c = prm.c
    e = eps_as_f32(eps)
    m = _mask_f64(inp, B, N)
    store_t = np.float32 if rounding == "kernel" else np.float64

    A = np.empty((B, N, N, c), store_t)
    Bp = np.empty((B, N, N, c), store_t)
    Z = np.empty((B, N, N, cz), store_t) if keep_z else None
    for bi in range(B):
        for r0 in range(0, N, row_block):
            rows = slice(r0, min(N, r0 + row_block))
            z = ln_in(_x_f64_rows(x_bits, bi, rows), prm, e, rounding)
            a, b = gated_projection(z, m[bi, rows], prm, rounding)
            A[bi, rows], Bp[bi, rows] = a, b
            if keep_z:
                Z[bi, rows] = z

    Y = np.empty((B, N, N, c), store_t)
    for bi in range(B):
        for c0 in range(0, c, ch_block):
            cs = slice(c0, min(c, c0 + ch_block))
            if direction == "outgoing":
                y = contract_outgoing(A[bi, :, :, cs], Bp[bi, :, :, cs])
            else:
                y = contract_incoming(A[bi, :, :, cs], Bp[bi, :, :, cs])
            Y[bi, :, :, cs] = _to_store(y, rounding)

    OUT = np.empty((B, N, N, cz), np.float64)
    for bi in range(B):
        for r0 in range(0, N, row_block):
            rows = slice(r0, min(N, r0 + row_block))
            z = Z[bi, rows] if keep_z else ln_in(_x_f64_rows(x_bits, bi, rows), prm, e, rounding)
            u = ln_out(Y[bi, rows], prm, e, rounding)
            OUT[bi, rows] = output(z, u, prm)
    return Intermediates(z=Z, a=A, b=Bp, y=Y, out=OUT)


def forward_block(inp: Dict[str, Optional[np.ndarray]], direction: str, rows: Sequence[int],
                  cols: Sequence[int], *, batch: int = 0, eps: float = 1e-5,
                  rounding: str = "kernel"):
    """Outputs of one batch entry on the block rows x cols only.

    Computes exactly what ``forward`` computes for the pairs (i, j) with i in
    ``rows`` and j in ``cols``, projecting only the pairs those outputs need:
    outgoing needs a[i, k] for i in rows and b[j, k] for j in cols (all k);
    incoming needs a[k, i] and b[k, j]. Returns (y, out) with shapes
    [len(rows), len(cols), c] and [len(rows), len(cols), c_z].
    """
    x_bits = inp["x"]
    if x_bits.ndim == 3:
        x_bits = x_bits[None]
    B, N, _, cz = x_bits.shape
    prm = params_from_bits(inp)
    e = eps_as_f32(eps)
    m = _mask_f64(inp, B, N)[batch]
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    xb = x_bits[batch]

    if direction == "outgoing":
        za = ln_in(bf16_bits_to_f64(xb[rows]), prm, e, rounding)              # [I, N, cz]
        a, _ = gated_projection(za, m[rows], prm, rounding)
        zb = ln_in(bf16_bits_to_f64(xb[cols]), prm, e, rounding)              # [J, N, cz]
        _, b = gated_projection(zb, m[cols], prm, rounding)
        y = contract_outgoing(a, b)
    elif direction == "incoming":
        za = ln_in(bf16_bits_to_f64(xb[:, rows]), prm, e, rounding)           # [N, I, cz]
        a, _ = gated_projection(za, m[:, rows], prm, rounding)
        zb = ln_in(bf16_bits_to_f64(xb[:, cols]), prm, e, rounding)           # [N, J, cz]
        _, b = gated_projection(zb, m[:, cols], prm, rounding)
        y = contract_incoming(a, b)
    else:
        raise ValueError(f"direction must be 'outgoing' or 'incoming', got {direction!r}")
    y = _to_store(y, rounding)
    z = ln_in(bf16_bits_to_f64(xb[np.ix_(rows, cols)]), prm, e, rounding)   # [I, J, cz]
    u = ln_out(y, prm, e, rounding)
    return y, output(z, u, prm)
