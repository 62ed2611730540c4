"""Triangle multiplicative update for the MI355X (gfx950): HIP kernels behind a C ABI.

``triangle_multiplicative_update`` is the drop-in function; ``workspace_bytes``
and ``check_support`` mirror the C ABI in ``include/trimul.h``.
"""

from .api import check_support, raise_for_status, triangle_multiplicative_update, workspace_bytes  # noqa: F401
from . import perf_model  # noqa: F401

__all__ = ["triangle_multiplicative_update", "workspace_bytes", "check_support", "perf_model"]
