"""MI355X-native Gated DeltaNet chunked prefill: forward and backward.

The computation lives in libgdn.so (hand-written HIP for gfx950, C ABI in
include/gdn.h); this package is the thin Python binding over it.
"""
from .api import (PreparedForward, PreparedForwardBackward, bwd_plan, chunk_cumsum, chunk_gated_delta_rule,  # noqa: F401
                  chunk_gated_delta_rule_bwd, chunk_gated_delta_rule_fwd, make_bwd_desc, make_desc, plan)

__all__ = ["chunk_gated_delta_rule", "chunk_gated_delta_rule_fwd", "chunk_gated_delta_rule_bwd", "chunk_cumsum",
           "plan", "bwd_plan", "make_desc", "make_bwd_desc", "PreparedForward", "PreparedForwardBackward"]
