"""MI355X (gfx950) tree-verify MLA-absorb attention.

The product path is the HIP library ``libkdtree_verify.so`` (C ABI in
include/kdtree_verify.h) and its ctypes binding in ``binding``.  ``synth`` generates
seeded synthetic inputs.  Nothing here imports the float64 oracle.
"""
from .binding import (KDTREE_MAX_QLEN, VerifyAttn, choose_num_splits, decode_status,
                      kdtree_max_qlen, kdtree_verify_attn, kdtree_verify_attn_workspace_bytes,
                      load_library, verify_attn)

__all__ = ["KDTREE_MAX_QLEN", "VerifyAttn", "choose_num_splits", "decode_status",
           "kdtree_max_qlen", "kdtree_verify_attn", "kdtree_verify_attn_workspace_bytes",
           "load_library", "verify_attn"]
