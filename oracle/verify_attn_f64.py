"""Float64 CPU oracle for tree-verify MLA-absorb attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  The product path (the HIP
library and its Python binding) never imports, calls or links anything here, and
this module imports nothing from the product path.

What it computes is the plain definition, over an explicit dense mask, one request at
a time, in float64:

* "The Milestone Commit: Cementing Phase 1 ..." -- section "The Context", item 2:
  verify attention is a masked softmax over the request's prefix followed by the
  draft-tree tail, in MLA-absorb form, giving latent output.
* same page, section "Input Knowledge Required" (MLA paragraph) and "Strategic
  Pivots in CUDA Kernel Engineering ..." section "Input Knowledge Required" (MLA
  paragraph): queries and keys live in the compressed latent space.
* "Strategic Pivots ..." -- section "The Message" (agent reasoning): the check is
  random MLA-shaped tensors plus a tree visibility mask from the builder, with the
  expected attention output computed on the host.

Readings taken where the pages are silent (all listed in the design notes):
  K = [kv_lat | k_rope] (576 dims), V = kv_lat (512 dims), shared by all heads;
  Q = [q_lat | q_rope]; score = scale * (Q . K) with ``scale`` applied to the sum of
  the latent and rope dot products; key k of request b is visible to node i iff
  k < P_b, or k - P_b is node i or one of its ancestors (ancestor-or-self mask);
  lse = natural log of sum_k exp(score_k) over visible keys.

Pins (tests/test_oracle_pins.py): per-node brute force with math.fsum on tiny trees;
chain tree == bottom-right causal attention through torch's SDPA; closed forms
(q = 0, scale = 0, root with empty prefix, single-key ranges); invariances; the split
+ LSE-merge identity; a hand-worked golden example under tests/golden/.
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

import numpy as np

_NEG_INF = -np.inf


def ancestor_or_self_mask(parent: Sequence[int]) -> np.ndarray:
    """Dense bool [T, T]: M[i, j] is True iff tree node j lies on the path root -> i
    (inclusive).  Built by walking every node's parent chain; the walk does not
    assume parent[i] < i, only that parent[0] == -1 and the chains reach the root."""
    par = np.asarray(parent, dtype=np.int64)
    t = len(par)
    if t == 0:
        raise ValueError("empty tree")
    if par[0] != -1:
        raise ValueError("node 0 must be the root (parent -1)")
    m = np.zeros((t, t), dtype=bool)
    for i in range(t):
        n = i
        hops = 0
        while n != -1:
            if not 0 <= n < t:
                raise ValueError(f"parent index out of range at node {i}")
            m[i, n] = True
            n = int(par[n])
            hops += 1
            if hops > t:
                raise ValueError("parent array has a cycle")
    return m


def visibility_mask(prefix_len: int, parent: Sequence[int]) -> np.ndarray:
    """Dense bool [T, P+T] over the concatenated KV stream (prefix, then the tail in
    node order): every prefix key is visible; tail key P+j is visible to node i iff
    j is an ancestor-or-self of i."""
    t = len(parent)
    m = np.zeros((t, prefix_len + t), dtype=bool)
    m[:, :prefix_len] = True
    m[:, prefix_len:] = ancestor_or_self_mask(parent)
    return m


def _head_chunk(t: int, n_keys: int, heads: int, budget_bytes: int = 1 << 28) -> int:
    per_head = max(1, t * n_keys * 8 * 3)
    return int(max(1, min(heads, budget_bytes // per_head)))


def attend_request(q_lat: np.ndarray, q_rope: np.ndarray, kv_lat: np.ndarray,
                   k_rope: np.ndarray, mask: np.ndarray, scale: float,
                   return_probs: bool = False):
    """Masked softmax attention of one request, float64.

    q_lat [T, H, DL], q_rope [T, H, DR], kv_lat [N, DL], k_rope [N, DR], mask [T, N].
    Returns out [T, H, DL] and lse [T, H]; rows with no visible key get out = 0 and
    lse = -inf.  With ``return_probs`` also the dense probabilities [T, H, N]."""
    q = np.concatenate([np.asarray(q_lat, np.float64), np.asarray(q_rope, np.float64)], axis=-1)
    k = np.concatenate([np.asarray(kv_lat, np.float64), np.asarray(k_rope, np.float64)], axis=-1)
    v = np.asarray(kv_lat, np.float64)
    t, h, d = q.shape
    n = k.shape[0]
    out = np.zeros((t, h, v.shape[1]), np.float64)
    lse = np.full((t, h), _NEG_INF, np.float64)
    probs = np.zeros((t, h, n), np.float64) if return_probs else None
    if n == 0:
        return (out, lse, probs) if return_probs else (out, lse)
    hc = _head_chunk(t, n, h)
    for h0 in range(0, h, hc):
        h1 = min(h, h0 + hc)
        qc = q[:, h0:h1, :].reshape(t * (h1 - h0), d)
        s = (qc @ k.T).reshape(t, h1 - h0, n) * float(scale)
        s = np.where(mask[:, None, :], s, _NEG_INF)
        m = s.max(axis=-1)
        has = np.isfinite(m)
        m_safe = np.where(has, m, 0.0)
        e = np.exp(s - m_safe[..., None])
        l = e.sum(axis=-1)
        o = (e.reshape(t * (h1 - h0), n) @ v).reshape(t, h1 - h0, v.shape[1])
        l_safe = np.where(has, l, 1.0)
        out[:, h0:h1, :] = np.where(has[..., None], o / l_safe[..., None], 0.0)
        lse[:, h0:h1] = np.where(has, m_safe + np.log(l_safe), _NEG_INF)
        if return_probs:
            probs[:, h0:h1, :] = e / l_safe[..., None]
    return (out, lse, probs) if return_probs else (out, lse)


def _request_slices(prefix_len, q_len):
    prefix_len = np.asarray(prefix_len, np.int64)
    q_len = np.asarray(q_len, np.int64)
    qoff = np.concatenate([[0], np.cumsum(q_len)[:-1]])
    kvoff = np.concatenate([[0], np.cumsum(prefix_len + q_len)[:-1]])
    return prefix_len, q_len, qoff, kvoff


def verify_attn(q_lat, q_rope, kv_lat, k_rope, prefix_len, tree_parent, q_len, scale,
                key_range: Optional[Tuple[Sequence[int], Sequence[int]]] = None):
    """Tree-verify MLA-absorb attention over a packed batch (see module docstring).

    Packed layout: request b owns query rows [qoff_b, qoff_b + T_b) and KV rows
    [kvoff_b, kvoff_b + P_b + T_b) (P_b prefix rows, then the tail in node order);
    offsets are exclusive prefix sums of q_len and prefix_len + q_len.

    ``key_range`` = (lo[b], hi[b]) optionally restricts request b to keys
    [lo_b, hi_b) of its concatenated stream (same mask otherwise); this is the
    partial result that the split-KV + merge scheme combines.

    Returns out_lat [sum_q, H, DL] and out_lse [sum_q, H] (float64)."""
    prefix_len, q_len, qoff, kvoff = _request_slices(prefix_len, q_len)
    sum_q, h, dl = np.shape(q_lat)
    out = np.zeros((sum_q, h, dl), np.float64)
    lse = np.full((sum_q, h), _NEG_INF, np.float64)
    parent_all = np.asarray(tree_parent, np.int64)
    for b in range(len(q_len)):
        p, t, qo, ko = int(prefix_len[b]), int(q_len[b]), int(qoff[b]), int(kvoff[b])
        mask = visibility_mask(p, parent_all[qo:qo + t])
        if key_range is not None:
            lo, hi = int(key_range[0][b]), int(key_range[1][b])
            mask[:, :max(lo, 0)] = False
            mask[:, max(hi, 0):] = False
        o, l = attend_request(q_lat[qo:qo + t], q_rope[qo:qo + t], kv_lat[ko:ko + p + t],
                              k_rope[ko:ko + p + t], mask, scale)
        out[qo:qo + t] = o
        lse[qo:qo + t] = l
    return out, lse


def lse_merge(outs: Sequence[np.ndarray], lses: Sequence[np.ndarray]):
    """Combine partial results over disjoint key sets ("The Milestone Commit ...",
    sections "Why This Message Was Written" and "What to defer": flash partial
    outputs merged for long prefixes).

    Each part s holds its own normalised output O_s [..., D] and lse_s [...] (lse -inf,
    O = 0 when part s saw no key).  With L = max_s lse_s and w_s = exp(lse_s - L):
    out = sum_s w_s O_s / sum_s w_s and lse = L + ln(sum_s w_s)."""
    lse_st = np.stack([np.asarray(x, np.float64) for x in lses])
    out_st = np.stack([np.asarray(x, np.float64) for x in outs])
    big = lse_st.max(axis=0)
    has = np.isfinite(big)
    big_safe = np.where(has, big, 0.0)
    w = np.where(np.isfinite(lse_st), np.exp(lse_st - big_safe[None]), 0.0)
    wsum = w.sum(axis=0)
    wsum_safe = np.where(has, wsum, 1.0)
    out = (w[..., None] * out_st).sum(axis=0) / wsum_safe[..., None]
    out = np.where(has[..., None], out, 0.0)
    lse = np.where(has, big_safe + np.log(wsum_safe), _NEG_INF)
    return out, lse


def verify_attn_inputs(inp, key_range=None):
    """Convenience wrapper over a ``VerifyInputs``-like object (duck-typed)."""
    return verify_attn(inp.q_lat, inp.q_rope, inp.kv_lat, inp.k_rope, inp.prefix_len,
                       inp.tree_parent, inp.q_len, inp.scale, key_range=key_range)


def verify_attn_rows(inp, b: int, nodes: Sequence[int], heads: Sequence[int]):
    """Oracle output for selected (node, head) rows of request ``b`` only, so that
    single rows of a large workload can be checked one by one.
    Returns out [len(nodes), len(heads), DL] and lse [len(nodes), len(heads)]."""
    prefix_len, q_len, qoff, kvoff = _request_slices(inp.prefix_len, inp.q_len)
    p, t, qo, ko = int(prefix_len[b]), int(q_len[b]), int(qoff[b]), int(kvoff[b])
    full_mask = visibility_mask(p, np.asarray(inp.tree_parent[qo:qo + t]))
    nodes = list(nodes)
    heads = list(heads)
    mask = full_mask[nodes]
    ql = np.asarray(inp.q_lat[qo:qo + t])[nodes][:, heads]
    qr = np.asarray(inp.q_rope[qo:qo + t])[nodes][:, heads]
    return attend_request(ql, qr, inp.kv_lat[ko:ko + p + t], inp.k_rope[ko:ko + p + t],
                          mask, inp.scale)
