"""MI355X-native Gated DeltaNet chunked-prefill forward.

The computation lives in libgdn.so (hand-written HIP for gfx950, C ABI in
include/gdn.h); this package is the thin Python binding over it.
"""
from .api import (PreparedForward, chunk_cumsum, chunk_gated_delta_rule, chunk_gated_delta_rule_fwd,  # noqa: F401
                  make_desc, plan)

__all__ = ["chunk_gated_delta_rule", "chunk_gated_delta_rule_fwd", "chunk_cumsum", "plan", "make_desc",
           "PreparedForward"]
