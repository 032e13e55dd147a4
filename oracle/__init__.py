"""Float64 CPU oracle (test infrastructure only; see oracle/verify_attn_f64.py)."""
from .verify_attn_f64 import (ancestor_or_self_mask, attend_request, lse_merge, verify_attn,
                          verify_attn_inputs, verify_attn_rows, visibility_mask)

__all__ = ["ancestor_or_self_mask", "attend_request", "lse_merge", "verify_attn",
           "verify_attn_inputs", "verify_attn_rows", "visibility_mask"]
