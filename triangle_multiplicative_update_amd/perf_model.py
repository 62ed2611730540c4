"""Algorithmic FLOP and HBM-byte models of one forward call.

Page "Triangle Multiplicative Update (SM100 / SM103 / SM107)", section
"Traffic model and measured performance": compulsory traffic is 18 N^2 C bytes
per batch entry (stage 1 reads x 2 B and writes a, b 4 B per pair-channel; stage
2 reads 4 B and writes y 2 B; stage 3 reads y and x 4 B and writes out 2 B) plus
2 B per pair of mask. The FLOP count is not printed as a formula; counting the
dense matrix products gives 2 B N^2 (4 c c_z + c N + c_z^2 + c c_z), which
reproduces the page's TFLOPS column from its times.
"""

from __future__ import annotations

# MI355X published peaks (dense).
PEAK_BF16_TFLOPS = 2516.6       # 256 CUs x 2.4 GHz x 4096 flop/clk
PEAK_HBM_GBS = 8000.0


def flops(B: int, N: int, c_z: int, c: int) -> float:
    """Dense matrix-product FLOPs of one call (mask is data, not sparsity)."""
    return 2.0 * B * N * N * (4 * c * c_z + c * N + c_z * c_z + c * c_z)


def stage_flops(B: int, N: int, c_z: int, c: int):
    p = B * N * N
    return (2.0 * p * 4 * c * c_z, 2.0 * p * c * N, 2.0 * p * (c_z * c_z + c * c_z))


def stage_bytes(B: int, N: int, c_z: int, c: int, mask: bool = True):
    """Compulsory HBM bytes of stages 1, 2, 3 (mask bytes counted in stage 1)."""
    p = B * N * N
    return (p * (2 * c_z + 4 * c + (2 if mask else 0)), p * 6 * c, p * (2 * c + 4 * c_z))


def traffic_bytes(B: int, N: int, c_z: int, c: int, mask: bool = True) -> float:
    return float(sum(stage_bytes(B, N, c_z, c, mask)))
