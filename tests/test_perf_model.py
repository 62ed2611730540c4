"""The FLOP and byte models against the figures the page prints.

Fixtures: tests/golden/page_perf_table_c128_b1.txt and
tests/golden/page_nsight_bytes_n1024.txt (each cites its page section).
"""

import os

import pytest

from triangle_multiplicative_update_amd import perf_model

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line.split()


@pytest.mark.parametrize("row", list(_rows("page_perf_table_c128_b1.txt")), ids=lambda r: f"{r[0]}-{r[1]}")
def test_models_reproduce_page_rates(row):
    N, _direction, us, gbs, tflops = int(row[0]), row[1], float(row[2]), float(row[3]), float(row[4])
    t = us * 1e-6
    f = perf_model.flops(1, N, 128, 128)
    b = perf_model.traffic_bytes(1, N, 128, 128, mask=True)
    # the page rounds TFLOPS and GB/s to whole numbers and the time to 0.1 us
    time_rel = 0.05 / us
    assert abs(f / t / 1e12 - tflops) <= 0.5 + tflops * time_rel
    assert abs(b / t / 1e9 - gbs) <= 0.5 + gbs * time_rel


def test_model_total_bytes_n1024():
    (row,) = list(_rows("page_nsight_bytes_n1024.txt"))
    N, c, B, mb = int(row[0]), int(row[1]), int(row[2]), float(row[3])
    assert abs(perf_model.traffic_bytes(B, N, c, c) / 1e6 - mb) < 1.0


def test_stage_split_matches_total():
    for (B, N, c) in [(1, 768, 128), (2, 512, 256), (1, 1536, 128)]:
        assert sum(perf_model.stage_flops(B, N, c, c)) == perf_model.flops(B, N, c, c)
        assert sum(perf_model.stage_bytes(B, N, c, c)) == perf_model.traffic_bytes(B, N, c, c)
    # 18 N^2 C per batch entry plus 2 B per pair of mask
    assert perf_model.traffic_bytes(1, 768, 128, 128) == 18 * 768 ** 2 * 128 + 2 * 768 ** 2
