"""MI355X (gfx950) tree-verify MLA-absorb attention and the draft-tree steps around it
(builder, packing, greedy accept, temperature draw).

The product path is the HIP library ``libkdtree_verify.so`` (C ABI in
include/kdtree_verify.h) and its ctypes binding in ``binding``.  ``synth`` generates
seeded synthetic inputs.  Nothing here imports the float64 oracle.
"""
from .binding import (KDTREE_MAX_QLEN, VerifyAttn, build_ddtree, choose_num_splits,
                      decode_status, kdtree_build_ddtree, kdtree_max_qlen, kdtree_pack_tree,
                      kdtree_sample_tokens, kdtree_tree_accept, kdtree_verify_attn,
                      kdtree_verify_attn_attend, kdtree_verify_attn_prepare,
                      kdtree_verify_attn_workspace_bytes, load_library, pack_tree,
                      sample_tokens, tree_accept, verify_attn)

__all__ = ["KDTREE_MAX_QLEN", "VerifyAttn", "build_ddtree", "choose_num_splits",
           "decode_status", "kdtree_build_ddtree", "kdtree_max_qlen", "kdtree_pack_tree",
           "kdtree_sample_tokens", "kdtree_tree_accept", "kdtree_verify_attn",
           "kdtree_verify_attn_attend", "kdtree_verify_attn_prepare",
           "kdtree_verify_attn_workspace_bytes", "load_library", "pack_tree", "sample_tokens",
           "tree_accept", "verify_attn"]
