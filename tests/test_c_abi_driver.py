"""The C ABI used from C++ alone (no Python binding, no torch): a small driver
program built against include/trimul.h and libtrimul.so.

CPU: the driver compiles and links. GPU: it runs one call on inputs written
here and its output is held to the oracle's tolerance (page "Triangle
Multiplicative Update (SM100 / SM103 / SM107)", section "Mathematics and
numerics").
"""

import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import synthetic_inputs as si
from parity_utils import assert_within_tolerance, say

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_abi", "trimul_c_driver.cpp")
PKG = os.path.join(ROOT, "triangle_multiplicative_update_amd")


def _hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    pytest.skip("hipcc not found")


def build_driver(out_dir) -> str:
    exe = os.path.join(str(out_dir), "trimul_c_driver")
    cmd = [_hipcc(), "-O2", "-std=c++17", "-I", os.path.join(ROOT, "include"), SRC, "-o", exe,
           "-L", PKG, "-ltrimul", f"-Wl,-rpath,{PKG}"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    return exe


def test_driver_builds(tmp_path):
    exe = build_driver(tmp_path)
    assert os.path.exists(exe)


@pytest.mark.gpu
@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
def test_driver_matches_oracle(gpu, tmp_path, direction):
    exe = build_driver(tmp_path)
    wl = si.custom(1, 77, 128, mask="bernoulli", seed=81)
    inp = si.generate(wl)
    for k, v in inp.items():
        if v is not None:
            np.ascontiguousarray(v).tofile(os.path.join(tmp_path, f"{k}.bin"))
    code = 0 if direction == "outgoing" else 1
    say(f"[gpu] C driver {wl.name} {direction}")
    res = subprocess.run([exe, str(tmp_path), "1", "77", "128", str(code), "1", "1"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr + res.stdout
    bits = np.fromfile(os.path.join(tmp_path, "out.bin"), dtype=np.uint16).reshape(1, 77, 77, 128)
    got = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert_within_tolerance(got, oracle.forward(inp, direction).out, f"C driver {direction}")
