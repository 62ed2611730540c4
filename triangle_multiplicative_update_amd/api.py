"""Drop-in Python entry point over the gfx950 C ABI.

The signature and behaviour follow the page "Triangle Multiplicative Update
(SM100 / SM103 / SM107)", section "Drop-in function" (parameter names, order
and defaults; the keyword-only ``out=`` and ``stream=``), and the declines of
section "Served today, and the typed declines". PyTorch supplies device memory
and the stream; every step of the computation runs in the HIP kernels.
"""

from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _native
from ._native import lib

_DIRECTIONS = {"outgoing": _native.TRIMUL_OUTGOING, "incoming": _native.TRIMUL_INCOMING}
_SERVED_PRECISION = (None, "default", "none", "bfloat16", "bf16")
_DECLINED_PRECISION = ("mxfp8", "ieee", "tf32")
_PARAM_ORDER = ("norm_in_weight", "norm_in_bias", "p_in_weight", "p_in_bias", "g_in_weight",
                "g_in_bias", "norm_out_weight", "norm_out_bias", "p_out_weight", "p_out_bias",
                "g_out_weight", "g_out_bias")
_REQUIRED = ("norm_in_weight", "norm_in_bias", "p_in_weight", "g_in_weight", "norm_out_weight",
             "norm_out_bias", "p_out_weight", "g_out_weight")


def raise_for_status(status: int, what: str = "trimul") -> None:
    """Map a C-ABI status to the page's typed errors."""
    if status == _native.TRIMUL_OK:
        return
    msg = f"{what}: {_native.last_error()}"
    if status == _native.TRIMUL_E_INVALID:
        raise ValueError(msg)
    if status == _native.TRIMUL_E_UNSUPPORTED:
        raise NotImplementedError(msg)
    raise RuntimeError(msg)


def workspace_bytes(B: int, N: int, c: int, direction: str = "outgoing") -> int:
    """Bytes of the a, b, y planes for one call (layout in include/trimul.h)."""
    return int(lib.trimul_workspace_bytes(B, N, c, _direction_code(direction)))


def check_support(B: int, N: int, c_z: int, c: int, direction: str = "outgoing",
                  device: Optional[int] = None) -> None:
    """Typed declines with no launch; ``device`` None skips the device check."""
    st = lib.trimul_check_support(B, N, c_z, c, _direction_code(direction),
                                  -1 if device is None else int(device))
    raise_for_status(st, "check_support")


def _direction_code(direction) -> int:
    if direction not in _DIRECTIONS:
        raise ValueError(f"direction must be 'outgoing' or 'incoming', got {direction!r}")
    return _DIRECTIONS[direction]


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _as_stream(stream, device) -> torch.cuda.Stream:
    """A torch stream object for a torch stream or a raw hipStream_t handle."""
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=device)


def _prep_param(name, t, precision, device):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, x is on {device}")
    if t.dtype != torch.bfloat16:
        if precision in ("bfloat16", "bf16"):
            t = t.to(torch.bfloat16)
        else:
            raise NotImplementedError(
                f"{name} is {t.dtype}; parameters must be bf16 (or pass precision='bfloat16')")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def triangle_multiplicative_update(
        x, direction="outgoing", mask=None,
        norm_in_weight=None, norm_in_bias=None, p_in_weight=None, p_in_bias=None,
        g_in_weight=None, g_in_bias=None, norm_out_weight=None, norm_out_bias=None,
        p_out_weight=None, p_out_bias=None, g_out_weight=None, g_out_bias=None,
        eps=1e-5, precision=None, *, out=None, stream=None, workspace=None,
        _stage=None) -> torch.Tensor:
    """Triangle multiplicative update, forward, bf16, on an MI355X (gfx950).

    x: [B, N, N, c_z] or [N, N, c_z] bf16 CUDA/HIP tensor, contiguous.
    mask: None, or [B, N, N] ([N, N] at B = 1) of any real or bool dtype.
    Returns out with x's rank (or ``out`` itself when given). The residual add is
    the caller's. ``workspace``: optional uint8 tensor of at least
    ``workspace_bytes(B, N, c, direction)`` bytes (allocated per call otherwise).
    """
    code = _direction_code(direction)
    if precision in _DECLINED_PRECISION or precision not in _SERVED_PRECISION:
        raise NotImplementedError(f"precision={precision!r} is not served "
                                  f"(served: None, 'default', 'none', 'bfloat16')")
    if not isinstance(x, torch.Tensor):
        raise ValueError("x must be a tensor")
    if x.device.type == "cuda" and stream is not None:
        # Every cast, allocation and launch of the call goes on the caller's
        # stream, after the work already queued on torch's current stream
        # (which may have produced the inputs); memory allocated here then
        # belongs to that stream's pool and is not handed to another stream
        # while the kernels still use it.
        ext = _as_stream(stream, x.device)
        cur = torch.cuda.current_stream(x.device)
        if ext != cur:
            ext.wait_stream(cur)
        with torch.cuda.stream(ext):
            return triangle_multiplicative_update(
                x, direction, mask, norm_in_weight, norm_in_bias, p_in_weight, p_in_bias,
                g_in_weight, g_in_bias, norm_out_weight, norm_out_bias, p_out_weight, p_out_bias,
                g_out_weight, g_out_bias, eps, precision, out=out, stream=None,
                workspace=workspace, _stage=_stage)
    params = dict(zip(_PARAM_ORDER, (norm_in_weight, norm_in_bias, p_in_weight, p_in_bias,
                                      g_in_weight, g_in_bias, norm_out_weight, norm_out_bias,
                                      p_out_weight, p_out_bias, g_out_weight, g_out_bias)))
    if torch.is_grad_enabled():
        grads = [n for n, t in [("x", x), ("mask", mask), *params.items()]
                 if isinstance(t, torch.Tensor) and t.requires_grad]
        if grads:
            raise NotImplementedError(
                f"autograd is not supported (forward only): {grads[0]} requires grad; "
                "call under torch.no_grad() or detach")
    for n in _REQUIRED:
        if params[n] is None:
            raise ValueError(f"{n} is required")
    if x.device.type != "cuda":
        raise ValueError(f"x must be on a GPU device, got {x.device}")
    if x.dtype != torch.bfloat16:
        if precision in ("bfloat16", "bf16"):
            x = x.to(torch.bfloat16)
        else:
            raise NotImplementedError(f"x is {x.dtype}; the pair representation must be bf16 "
                                      "(or pass precision='bfloat16')")
    if not x.is_contiguous():
        raise ValueError("x must be contiguous (no hidden copy is made)")
    batchless = x.dim() == 3
    if x.dim() not in (3, 4):
        raise ValueError(f"x must be [B, N, N, c_z] or [N, N, c_z], got shape {tuple(x.shape)}")
    xb = x.unsqueeze(0) if batchless else x
    B, N, N2, c_z = xb.shape
    if N != N2:
        raise ValueError(f"x must be square in its pair axes, got {tuple(x.shape)}")
    device = x.device
    for n in _PARAM_ORDER:
        params[n] = _prep_param(n, params[n], precision, device)
    c = params["p_in_weight"].shape[0] // 2
    shapes = {"norm_in_weight": (c_z,), "norm_in_bias": (c_z,), "p_in_weight": (2 * c, c_z),
              "p_in_bias": (2 * c,), "g_in_weight": (2 * c, c_z), "g_in_bias": (2 * c,),
              "norm_out_weight": (c,), "norm_out_bias": (c,), "p_out_weight": (c_z, c),
              "p_out_bias": (c_z,), "g_out_weight": (c_z, c_z), "g_out_bias": (c_z,)}
    for n, shp in shapes.items():
        t = params[n]
        if t is not None and tuple(t.shape) != shp:
            raise ValueError(f"{n} must have shape {shp}, got {tuple(t.shape)}")

    if mask is not None:
        if not isinstance(mask, torch.Tensor):
            raise ValueError("mask must be a tensor or None")
        if mask.device != device:
            raise ValueError(f"mask is on {mask.device}, x is on {device}")
        if mask.dim() == 2 and B == 1:
            mask = mask.unsqueeze(0)
        if tuple(mask.shape) != (B, N, N):
            raise ValueError(f"mask must be [B, N, N] = {(B, N, N)}"
                             f"{' or [N, N]' if B == 1 else ''}, got {tuple(mask.shape)}")
        if mask.dtype != torch.bfloat16 or not mask.is_contiguous():
            mask = mask.to(torch.bfloat16).contiguous()   # cast once per call

    if out is None:
        out_t = torch.empty_like(xb)
        ret = out_t[0] if batchless else out_t
    else:
        if not isinstance(out, torch.Tensor) or out.dtype != torch.bfloat16:
            raise ValueError("out must be a bf16 tensor")
        if out.numel() != xb.numel() or out.shape[-3:] != xb.shape[-3:] or out.device != device:
            raise ValueError(f"out must be {tuple(xb.shape)} (or batchless at B = 1) on {device}")
        if not out.is_contiguous():
            raise ValueError("out must be contiguous")
        out_t, ret = out, out

    need = workspace_bytes(B, N, c, direction) if c in (128, 256) and B > 0 else 0
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    ws_bytes = workspace.numel() * workspace.element_size()

    stream_h = torch.cuda.current_stream(device).cuda_stream

    args = [_ptr(xb), _ptr(mask)] + [_ptr(params[n]) for n in _PARAM_ORDER] + \
        [B, N, c_z, c, code, float(eps), _ptr(out_t), workspace.data_ptr(), ws_bytes, stream_h]
    with torch.cuda.device(device):
        if _stage is None:
            st = lib.trimul_forward(*args)
        else:
            st = lib.trimul_forward_stage(int(_stage), *args)
    raise_for_status(st, "triangle_multiplicative_update")
    return ret


class Prepared:
    """A call with its tensors fixed: arguments are checked and marshalled once,
    then ``forward()`` / ``stage(s)`` go straight to the C ABI (no per-call
    Python checks, no allocation). The C side still validates every call.

    Buffers must stay alive and unchanged in shape for the object's lifetime.
    """

    def __init__(self, x, direction, mask, params, out, workspace, eps=1e-5, stream=None):
        code = _direction_code(direction)
        for n in _REQUIRED:
            if params.get(n) is None:
                raise ValueError(f"{n} is required")
        for n, t in [("x", x), ("out", out), ("mask", mask), *params.items()]:
            if t is not None and (t.dtype != torch.bfloat16 or not t.is_contiguous()
                                  or t.device != x.device):
                raise ValueError(f"{n} must be a contiguous bf16 tensor on {x.device}")
        xb = x.unsqueeze(0) if x.dim() == 3 else x
        B, N, _, c_z = xb.shape
        c = params["p_in_weight"].shape[0] // 2
        self.device = x.device
        self.stream = (torch.cuda.current_stream(x.device).cuda_stream if stream is None
                       else (stream.cuda_stream if isinstance(stream, torch.cuda.Stream) else int(stream)))
        self._keep = (x, mask, params, out, workspace)
        self.args = tuple([_ptr(x), _ptr(mask)] + [_ptr(params.get(n)) for n in _PARAM_ORDER] +
                          [B, N, c_z, c, code, float(eps), out.data_ptr(), workspace.data_ptr(),
                           workspace.numel() * workspace.element_size(), self.stream])
        st = lib.trimul_validate(*self.args[:-1])
        raise_for_status(st, "Prepared")

    def forward(self) -> None:
        raise_for_status(lib.trimul_forward(*self.args), "forward")

    def stage(self, s: int) -> None:
        raise_for_status(lib.trimul_forward_stage(s, *self.args), f"stage {s}")

    def graph(self) -> "TrimulGraph":
        """The same call captured once (one graph launch per call)."""
        h = ctypes.c_void_p()
        with torch.cuda.device(self.device):
            raise_for_status(lib.trimul_graph_create(*self.args[:-1], ctypes.byref(h)), "graph")
        return TrimulGraph(h.value, self.device, self._keep)


# ---------------------------------------------------------------------------
# Prepared class API (page "Triangle Multiplicative Update (SM100 / SM103 /
# SM107)", section "Prepared class API"): parameters prepared once, a plan
# declared for one geometry, execute() with no allocation and no sync, and a
# captured graph per buffer set for the host-bound small-N calls.
# ---------------------------------------------------------------------------

class PreparedWeights:
    """The twelve parameters, checked once: bf16, contiguous, one device, the
    declared shapes. A bias given on one side only (in: p_in / g_in, out:
    p_out / g_out) is paired with zeros here, never per call."""

    def __init__(self, tensors: dict, c_z: int, c: int, device):
        self.tensors = tensors
        self.c_z, self.c, self.device = c_z, c, device
        self.has_in_bias = tensors["p_in_bias"] is not None
        self.has_out_bias = tensors["p_out_bias"] is not None

    def ptrs(self):
        return [_ptr(self.tensors[n]) for n in _PARAM_ORDER]


def prepare_weights(norm_in_weight, norm_in_bias, p_in_weight, p_in_bias, g_in_weight, g_in_bias,
                    norm_out_weight, norm_out_bias, p_out_weight, p_out_bias, g_out_weight,
                    g_out_bias, precision=None) -> PreparedWeights:
    if precision in _DECLINED_PRECISION or precision not in _SERVED_PRECISION:
        raise NotImplementedError(f"precision={precision!r} is not served")
    params = dict(zip(_PARAM_ORDER, (norm_in_weight, norm_in_bias, p_in_weight, p_in_bias,
                                      g_in_weight, g_in_bias, norm_out_weight, norm_out_bias,
                                      p_out_weight, p_out_bias, g_out_weight, g_out_bias)))
    for n in _REQUIRED:
        if params[n] is None:
            raise ValueError(f"{n} is required")
    device = params["p_in_weight"].device
    if device.type != "cuda":
        raise ValueError(f"parameters must be on a GPU device, got {device}")
    for n in _PARAM_ORDER:
        params[n] = _prep_param(n, params[n], precision, device)
    two_c, c_z = params["p_in_weight"].shape
    c = two_c // 2
    shapes = {"norm_in_weight": (c_z,), "norm_in_bias": (c_z,), "p_in_weight": (2 * c, c_z),
              "p_in_bias": (2 * c,), "g_in_weight": (2 * c, c_z), "g_in_bias": (2 * c,),
              "norm_out_weight": (c,), "norm_out_bias": (c,), "p_out_weight": (c_z, c),
              "p_out_bias": (c_z,), "g_out_weight": (c_z, c_z), "g_out_bias": (c_z,)}
    for n, shp in shapes.items():
        t = params[n]
        if t is not None and tuple(t.shape) != shp:
            raise ValueError(f"{n} must have shape {shp}, got {tuple(t.shape)}")
    for a, b in (("p_in_bias", "g_in_bias"), ("p_out_bias", "g_out_bias")):
        if (params[a] is None) != (params[b] is None):
            given = a if params[a] is not None else b
            other = b if given == a else a
            params[other] = torch.zeros_like(params[given])
    return PreparedWeights(params, c_z, c, device)


class TrimulGraph:
    """One forward pass captured for a fixed buffer set (a HIP graph owned by
    the C library). ``launch()`` enqueues it; the buffers' contents are read
    at launch time. Keep the buffers alive while the graph lives."""

    def __init__(self, handle: int, device, keep):
        self._h = handle
        self.device = device
        self._keep = keep

    def launch(self, stream=None) -> None:
        if self._h is None:
            raise RuntimeError("graph is closed")
        if stream is None:
            s = torch.cuda.current_stream(self.device).cuda_stream
        elif isinstance(stream, torch.cuda.Stream):
            s = stream.cuda_stream
        else:
            s = int(stream)
        with torch.cuda.device(self.device):
            raise_for_status(lib.trimul_graph_launch(self._h, s), "graph launch")

    replay = launch

    def close(self) -> None:
        if self._h is not None:
            h, self._h = self._h, None
            raise_for_status(lib.trimul_graph_destroy(h), "graph destroy")

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            if self._h is not None:
                lib.trimul_graph_destroy(self._h)
                self._h = None
        except Exception:
            pass


class TriangleMultiplicativeUpdateFwd:
    """A plan for one geometry: ``x`` (a tensor or its shape [B, N, N, c_z] /
    [N, N, c_z]), the direction, c_hidden, and whether calls carry a mask and
    the in/out projection biases. The flags are part of the declaration:
    ``execute`` raises if its arguments do not match them."""

    def __init__(self, x, direction, c_hidden, has_mask, has_in_bias, has_out_bias, eps=1e-5,
                 device=None):
        self.code = _direction_code(direction)
        self.direction = direction
        if isinstance(x, torch.Tensor):
            shape, dev = tuple(x.shape), x.device
        else:
            shape, dev = tuple(x), torch.device(device) if device is not None else None
        if len(shape) not in (3, 4):
            raise ValueError(f"x must be [B, N, N, c_z] or [N, N, c_z], got shape {shape}")
        self.batchless = len(shape) == 3
        B, N, N2, c_z = (1, *shape) if self.batchless else shape
        if N != N2:
            raise ValueError(f"x must be square in its pair axes, got {shape}")
        self.B, self.N, self.c_z, self.c = B, N, c_z, int(c_hidden)
        self.shape = shape
        self.device = dev if dev is not None else torch.device("cuda", torch.cuda.current_device())
        self.has_mask, self.has_in_bias, self.has_out_bias = bool(has_mask), bool(has_in_bias), bool(has_out_bias)
        self.eps = float(eps)

    def check_support(self) -> None:
        idx = self.device.index if self.device.type == "cuda" else None
        if self.device.type != "cuda":
            raise ValueError(f"plans run on a GPU device, got {self.device}")
        check_support(self.B, self.N, self.c_z, self.c, self.direction,
                      idx if idx is not None else torch.cuda.current_device())

    def compile(self):
        """The kernels are built ahead of time for gfx950: this only runs the
        support checks (and loads the library)."""
        self.check_support()
        return self

    def get_workspace_size(self) -> int:
        return workspace_bytes(self.B, self.N, self.c, self.direction)

    def _args(self, x, mask, weights, out, workspace):
        if not isinstance(weights, PreparedWeights):
            raise ValueError("weights must come from prepare_weights()")
        if (mask is not None) != self.has_mask:
            raise ValueError(f"plan declared has_mask={self.has_mask} but mask is "
                             f"{'given' if mask is not None else 'None'}")
        if weights.has_in_bias != self.has_in_bias or weights.has_out_bias != self.has_out_bias:
            raise ValueError(f"plan declared has_in_bias={self.has_in_bias}, "
                             f"has_out_bias={self.has_out_bias}; the weights have "
                             f"{weights.has_in_bias}, {weights.has_out_bias}")
        if weights.c != self.c or weights.c_z != self.c_z:
            raise ValueError(f"weights are for c_z={weights.c_z}, c={weights.c}; the plan for "
                             f"c_z={self.c_z}, c={self.c}")
        for n, t in (("x", x), ("out", out)):
            if not isinstance(t, torch.Tensor) or tuple(t.shape) not in (self.shape, (self.B, self.N, self.N, self.c_z)):
                raise ValueError(f"{n} must have the declared shape {self.shape}")
            if t.dtype != torch.bfloat16 or not t.is_contiguous() or t.device != self.device:
                raise ValueError(f"{n} must be a contiguous bf16 tensor on {self.device}")
        if mask is not None:
            if mask.dtype != torch.bfloat16 or not mask.is_contiguous() or mask.device != self.device:
                raise ValueError(f"mask must be a contiguous bf16 tensor on {self.device}")
            if mask.numel() != self.B * self.N * self.N:
                raise ValueError(f"mask must be [B, N, N] = {(self.B, self.N, self.N)}")
        if workspace.device != self.device:
            raise ValueError(f"workspace must be on {self.device}")
        return ([_ptr(x), _ptr(mask)] + weights.ptrs() +
                [self.B, self.N, self.c_z, self.c, self.code, self.eps, out.data_ptr(),
                 workspace.data_ptr(), workspace.numel() * workspace.element_size()])

    def execute(self, x, mask, weights, out, workspace, current_stream=None) -> None:
        """Validates and enqueues the three stages; no allocation, no sync."""
        args = self._args(x, mask, weights, out, workspace)
        if current_stream is None:
            s = torch.cuda.current_stream(self.device).cuda_stream
        elif isinstance(current_stream, torch.cuda.Stream):
            s = current_stream.cuda_stream
        else:
            s = int(current_stream)
        with torch.cuda.device(self.device):
            raise_for_status(lib.trimul_forward(*args, s), "execute")

    def make_graph(self, x, mask, weights, out, workspace) -> TrimulGraph:
        """Capture one forward pass for these buffers (one launch per call)."""
        args = self._args(x, mask, weights, out, workspace)
        h = ctypes.c_void_p()
        with torch.cuda.device(self.device):
            raise_for_status(lib.trimul_graph_create(*args, ctypes.byref(h)), "make_graph")
        return TrimulGraph(h.value, self.device, (x, mask, weights, out, workspace))

    make_cuda_graph = make_graph
