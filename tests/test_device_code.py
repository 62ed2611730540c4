"""Checks on the gfx950 assembly the kernels compile to (CPU only: hipcc
cross-compiles, nothing runs on a GPU).

A buffer store of more than 8 bytes reads its data registers over more than
one cycle. The compiler keeps the next instruction from overwriting them only
when the store's scalar offset is not a register; with a register there, a
plane store's first data dword was seen to take the value written by the
following instruction (run-to-run differences in plane b). The kernels
therefore pass whole offsets in the vector operand; these tests pin that.
"""

import os
import re
import shutil
import subprocess

import pytest

from triangle_multiplicative_update_amd import build as tb

KERNELS = ["k1_ln_proj.hip", "k2_contract.hip", "k3_epilogue.hip"]
WIDE_STORE = re.compile(r"^\s*(buffer_store_dwordx[34]|buffer_store_b(96|128))\s+v\[(\d+):(\d+)\],\s*v\d+,\s*s\[\d+:\d+\],\s*(\S+)")


def _asm(src: str, tmp_path) -> list[str]:
    out = tmp_path / (os.path.basename(src) + ".s")
    cmd = [tb.hipcc(), *[f for f in tb.HIP_FLAGS if f != "-fPIC"], "-x", "hip", "--cuda-device-only", "-S",
           src, "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    return out.read_text().splitlines()


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not installed")
@pytest.mark.parametrize("name", KERNELS)
def test_wide_buffer_stores_take_no_scalar_offset_register(name, tmp_path):
    lines = _asm(os.path.join(tb.CSRC, name), tmp_path)
    wide = 0
    for i, line in enumerate(lines):
        m = WIDE_STORE.match(line)
        if not m:
            continue
        wide += 1
        lo, hi, soff = int(m.group(3)), int(m.group(4)), m.group(5)
        assert soff == "0", f"{name}: {line.strip()} has a register scalar offset"
        nxt = lines[i + 1].strip()
        dst = re.match(r"v_\S+\s+v(?:\[)?(\d+)", nxt)
        assert not (dst and lo <= int(dst.group(1)) <= hi), f"{name}: {line.strip()} then {nxt}"
    if name != "k2_contract.hip":
        assert wide > 0, f"{name}: expected buffer stores"


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not installed")
@pytest.mark.parametrize("name", KERNELS)
def test_m0_is_only_the_direct_loads_lds_address(name, tmp_path):
    """The direct loads are inline assembly that sets M0 (the LDS address of
    the copy) itself, which is only sound if no compiler-generated code keeps
    a value in M0: every M0 reference must be that assembly's `s_mov_b32 m0`
    with its direct load right behind it."""
    lines = [l.strip() for l in _asm(os.path.join(tb.CSRC, name), tmp_path)]
    code = [l for l in lines if l and not l.startswith((";", ".", "_"))]
    loads = 0
    for i, line in enumerate(code):
        if "global_load_lds" in line:
            loads += 1
        if not re.search(r"\bm0\b", line):
            continue
        assert re.fullmatch(r"s_mov_b32 m0, s\d+", line), f"{name}: {line}"
        follow = code[i + 1:i + 3]
        assert follow[0] == "s_nop 0" and follow[1].startswith("global_load_lds_dwordx4"), f"{name}: {line} then {follow}"
    assert loads > 0
