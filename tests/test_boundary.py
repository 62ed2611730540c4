"""Host-side tests of the C ABI (no GPU needed): the library loads, exports
every declared symbol, sizes the workspace as documented, and returns the typed
decline for every argument rule without touching a device.

Rules: page "Triangle Multiplicative Update (SM100 / SM103 / SM107)", section
"Served today, and the typed declines", re-targeted to gfx950.
"""

import ctypes
import os
import re

import pytest
import torch

from triangle_multiplicative_update_amd import _native, api, workspace_bytes
from triangle_multiplicative_update_amd._native import lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, INVALID, UNSUPPORTED, DEVICE = 0, 1, 2, 3


def declared_functions():
    src = open(os.path.join(ROOT, "include", "trimul.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(trimul_\w+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 8
    so = ctypes.CDLL(_native.LIB_PATH)
    for n in names:
        assert hasattr(so, n), n
    assert set(names) == set(_native.SIGNATURES), "binding and header disagree"


def test_version_and_error_strings():
    assert _native.version().startswith("trimul-gfx950")
    assert isinstance(_native.last_error(), str)


def n_pad(N):
    return (N + 63) // 64 * 64


@pytest.mark.parametrize("B,N,c", [(1, 64, 128), (1, 77, 128), (2, 512, 256), (1, 1536, 128), (3, 1, 128)])
def test_workspace_layout(B, N, c):
    assert lib.trimul_n_pad(N) == n_pad(N)
    plane = c * B * N * n_pad(N) * 2
    plane = (plane + 255) // 256 * 256
    for d in ("outgoing", "incoming"):
        assert workspace_bytes(B, N, c, d) == 3 * plane
    assert lib.trimul_workspace_bytes(B, N, c, 7) == 0
    assert lib.trimul_workspace_bytes(0, N, c, 0) == 0


# ---- trimul_validate with fake, never-dereferenced addresses ----

BASE = 1 << 40
MB = 1 << 20


def good_args(B=1, N=64, c=128, direction=0, **over):
    cz = c
    pairs = B * N * N
    a = {
        "x": BASE, "mask": BASE + 1 * 512 * MB,
        "norm_in_w": BASE + 2 * 512 * MB, "norm_in_b": BASE + 2 * 512 * MB + 4096,
        "p_in_w": BASE + 3 * 512 * MB, "p_in_b": BASE + 3 * 512 * MB + 2 * MB,
        "g_in_w": BASE + 4 * 512 * MB, "g_in_b": BASE + 4 * 512 * MB + 2 * MB,
        "norm_out_w": BASE + 5 * 512 * MB, "norm_out_b": BASE + 5 * 512 * MB + 4096,
        "p_out_w": BASE + 6 * 512 * MB, "p_out_b": BASE + 6 * 512 * MB + 2 * MB,
        "g_out_w": BASE + 7 * 512 * MB, "g_out_b": BASE + 7 * 512 * MB + 2 * MB,
        "B": B, "N": N, "c_z": cz, "c": c, "direction": direction, "eps": 1e-5,
        "out": BASE + (1 << 36), "workspace": BASE + (1 << 37),
        "workspace_bytes": lib.trimul_workspace_bytes(B, N, c, direction if direction in (0, 1) else 0),
    }
    assert pairs * cz * 2 < 512 * MB
    a.update(over)
    return a


ORDER = ["x", "mask", "norm_in_w", "norm_in_b", "p_in_w", "p_in_b", "g_in_w", "g_in_b",
         "norm_out_w", "norm_out_b", "p_out_w", "p_out_b", "g_out_w", "g_out_b",
         "B", "N", "c_z", "c", "direction", "eps", "out", "workspace", "workspace_bytes"]


def validate(a):
    return lib.trimul_validate(*[a[k] for k in ORDER])


def test_valid_arguments_pass():
    assert validate(good_args()) == OK
    assert validate(good_args(mask=None, p_in_b=None, g_in_b=None, p_out_b=None, g_out_b=None)) == OK
    assert validate(good_args(B=2, N=77, c=256, direction=1)) == OK
    assert _native.last_error() == ""


@pytest.mark.parametrize("over,code,needle", [
    ({"direction": 2}, INVALID, "direction"),
    ({"B": 0}, INVALID, "B and N"),
    ({"N": 0}, INVALID, "B and N"),
    ({"c_z": 100}, INVALID, "multiple of 32"),
    ({"c_z": 256}, UNSUPPORTED, "c_z != c"),
    ({"c": 64, "c_z": 64}, UNSUPPORTED, "128 or 256"),
    ({"c": 384, "c_z": 384}, UNSUPPORTED, "128 or 256"),
    ({"x": None}, INVALID, "x is required"),
    ({"norm_in_w": None}, INVALID, "norm_in_weight is required"),
    ({"norm_out_b": None}, INVALID, "norm_out_bias is required"),
    ({"p_in_w": None}, INVALID, "p_in_weight is required"),
    ({"g_out_w": None}, INVALID, "g_out_weight is required"),
    ({"out": None}, INVALID, "out is required"),
    ({"workspace": None}, INVALID, "workspace is required"),
    ({"workspace_bytes": 100}, INVALID, "workspace too small"),
    ({"eps": float("nan")}, INVALID, "eps"),
    ({"eps": -1.0}, INVALID, "eps"),
    ({"x": BASE + 8}, INVALID, "x must be 16-byte aligned"),
    ({"out": BASE + (1 << 36) + 2}, INVALID, "out must be 16-byte aligned"),
    ({"mask": BASE + 1 * 512 * MB + 1}, INVALID, "mask must be 2-byte aligned"),
    ({"out": BASE + 1024}, INVALID, "out overlaps x"),
    ({"workspace": BASE + 3 * 512 * MB - 4096}, INVALID, "workspace overlaps p_in_weight"),
    ({"out": BASE + 7 * 512 * MB + 2 * MB}, INVALID, "out overlaps g_out_bias"),
    ({"out": BASE + (1 << 37) + 256}, INVALID, "out overlaps workspace"),
])
def test_declines(over, code, needle):
    a = good_args(**over)
    if "c" in over or "c_z" in over:
        a["workspace_bytes"] = 1 << 40
    got = validate(a)
    assert got == code, (got, _native.last_error())
    assert needle in _native.last_error()


def test_extent_limits():
    # 2*c*B*N*n_pad must stay below 2^31: N = 2048, c = 256, B = 1 is exactly 2^31
    assert lib.trimul_check_support(1, 2048, 256, 256, 0, -1) == UNSUPPORTED
    assert "2^31" in _native.last_error()
    assert lib.trimul_check_support(1, 2040, 256, 256, 0, -1) == OK
    assert lib.trimul_check_support(4, 2048, 128, 128, 1, -1) == UNSUPPORTED
    assert lib.trimul_check_support(1, 1536, 128, 128, 0, -1) == OK
    assert lib.trimul_check_support(2, 512, 256, 256, 1, -1) == OK


def test_no_device_is_a_clean_status():
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    assert lib.trimul_check_support(1, 64, 128, 128, 0, 0) == DEVICE
    a = good_args()
    st = lib.trimul_forward(*[a[k] for k in ORDER], None)
    assert st == DEVICE, _native.last_error()


def test_python_declines_without_gpu():
    x = torch.zeros(4, 4, 128, dtype=torch.bfloat16)
    w = torch.zeros(128, dtype=torch.bfloat16)
    m = torch.zeros(256, 128, dtype=torch.bfloat16)
    o = torch.zeros(128, 128, dtype=torch.bfloat16)
    params = [w, w, m, None, m, None, w, w, o, None, o, None]
    with pytest.raises(ValueError, match="direction"):
        api.triangle_multiplicative_update(x, "diagonal", None, *params)
    with pytest.raises(NotImplementedError, match="precision"):
        api.triangle_multiplicative_update(x, "outgoing", None, *params, precision="mxfp8")
    with pytest.raises(ValueError, match="required"):
        api.triangle_multiplicative_update(x, "outgoing", None, *([None] + params[1:]))
    with pytest.raises(ValueError, match="GPU"):
        api.triangle_multiplicative_update(x, "outgoing", None, *params)
    xg = x.clone().float().requires_grad_(True)
    with pytest.raises(NotImplementedError, match="autograd"):
        api.triangle_multiplicative_update(xg, "outgoing", None, *params)
    with torch.no_grad():
        with pytest.raises(ValueError, match="GPU"):
            api.triangle_multiplicative_update(xg, "outgoing", None, *params)


def test_graph_handles_without_device():
    # argument rules are checked before any HIP call; the handle is cleared
    h = ctypes.c_void_p(1234)
    a = good_args(x=None)
    assert lib.trimul_graph_create(*[a[k] for k in ORDER], ctypes.byref(h)) == INVALID
    assert h.value is None
    assert "x is required" in _native.last_error()
    a = good_args()
    assert lib.trimul_graph_create(*[a[k] for k in ORDER], None) == INVALID
    assert "NULL" in _native.last_error()
    assert lib.trimul_graph_launch(None, None) == INVALID
    assert lib.trimul_graph_destroy(None) == OK
    if not torch.cuda.is_available():
        h2 = ctypes.c_void_p(1234)
        assert lib.trimul_graph_create(*[a[k] for k in ORDER], ctypes.byref(h2)) == DEVICE
        assert h2.value is None


def test_plan_declines_without_gpu():
    with pytest.raises(ValueError, match="direction"):
        api.TriangleMultiplicativeUpdateFwd((1, 8, 8, 128), "diagonal", 128, True, True, True)
    with pytest.raises(ValueError, match="square"):
        api.TriangleMultiplicativeUpdateFwd((1, 8, 9, 128), "outgoing", 128, True, True, True)
    plan = api.TriangleMultiplicativeUpdateFwd((2, 77, 77, 256), "incoming", 256, False, False, True,
                                               device="cpu")
    assert plan.get_workspace_size() == workspace_bytes(2, 77, 256, "incoming")
    with pytest.raises(ValueError, match="GPU"):
        plan.check_support()
    w = torch.zeros(128, dtype=torch.bfloat16)
    m = torch.zeros(256, 128, dtype=torch.bfloat16)
    o = torch.zeros(128, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        api.prepare_weights(w, w, m, None, m, None, w, w, o, None, o, None)
    with pytest.raises(ValueError, match="required"):
        api.prepare_weights(w, w, None, None, m, None, w, w, o, None, o, None)
    with pytest.raises(NotImplementedError, match="precision"):
        api.prepare_weights(w, w, m, None, m, None, w, w, o, None, o, None, precision="tf32")


def test_drop_in_signature_pin():
    """The drop-in function's parameters: the page's names, order and defaults
    (section "Drop-in function"), out= and stream= keyword-only."""
    import inspect
    sig = inspect.signature(api.triangle_multiplicative_update)
    names = list(sig.parameters)
    assert names[:17] == ["x", "direction", "mask", "norm_in_weight", "norm_in_bias", "p_in_weight",
                          "p_in_bias", "g_in_weight", "g_in_bias", "norm_out_weight", "norm_out_bias",
                          "p_out_weight", "p_out_bias", "g_out_weight", "g_out_bias", "eps", "precision"]
    p = sig.parameters
    assert p["direction"].default == "outgoing" and p["eps"].default == 1e-5
    assert p["precision"].default is None
    assert all(p[n].default is None for n in names[2:15])
    for n in ("out", "stream"):
        assert p[n].kind is inspect.Parameter.KEYWORD_ONLY and p[n].default is None
    # the prepared class API (section "Prepared class API")
    pw = list(inspect.signature(api.prepare_weights).parameters)
    assert pw == names[3:15] + ["precision"]
    fwd = list(inspect.signature(api.TriangleMultiplicativeUpdateFwd.__init__).parameters)
    assert fwd[1:7] == ["x", "direction", "c_hidden", "has_mask", "has_in_bias", "has_out_bias"]
    ex = list(inspect.signature(api.TriangleMultiplicativeUpdateFwd.execute).parameters)
    assert ex[1:6] == ["x", "mask", "weights", "out", "workspace"]
