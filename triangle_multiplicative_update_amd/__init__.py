"""Triangle multiplicative update for the MI355X (gfx950): HIP kernels behind a C ABI.

``triangle_multiplicative_update`` is the drop-in function; ``workspace_bytes``
and ``check_support`` mirror the C ABI in ``include/trimul.h``;
``prepare_weights`` + ``TriangleMultiplicativeUpdateFwd`` are the prepared
class API (``execute`` and captured graphs for fixed buffers).
"""

from .api import (  # noqa: F401
    PreparedWeights, TriangleMultiplicativeUpdateFwd, TrimulGraph, check_support, prepare_weights,
    raise_for_status, triangle_multiplicative_update, workspace_bytes)
from . import perf_model  # noqa: F401

__all__ = ["triangle_multiplicative_update", "workspace_bytes", "check_support", "perf_model",
           "prepare_weights", "PreparedWeights", "TriangleMultiplicativeUpdateFwd", "TrimulGraph"]
