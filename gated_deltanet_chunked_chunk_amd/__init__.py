"""MI355X-native Gated DeltaNet chunked-prefill forward.

The computation lives in libgdn.so (hand-written HIP for gfx950, C ABI in
include/gdn.h); this package is the thin Python binding over it.
"""
from .api import PreparedForward, chunk_cumsum, chunk_gated_delta_rule, make_desc, plan  # noqa: F401

__all__ = ["chunk_gated_delta_rule", "chunk_cumsum", "plan", "make_desc", "PreparedForward"]
