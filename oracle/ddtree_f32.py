"""CPU oracle for the two steps around tree-verify attention in a greedy DDTree step:
the best-first draft-tree builder and the greedy follow-verified-tree accept.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  The product path (the HIP
library and its Python binding) never imports, calls or links anything here, and
this module imports nothing from the product path.

* Builder -- "The Milestone Commit: Cementing Phase 1 ...", section "The Context",
  item 1 (a best-first tree builder on the device in place of a per-request host
  heap) and "Strategic Pivots in CUDA Kernel Engineering ...", sections "The Message"
  and "Why This Message Was Written" (trees from the drafter's top-k log-probabilities
  and token ids; budgets up to 64, depth up to 15, batch 64; bit-exact parity including
  the heap's tie-breaks and the float32 accumulation order).
* Accept -- "The Milestone Commit ...", section "The Context", item 3 (a greedy
  follow-verified-tree walk over next-token / next-sibling pointers, one thread per
  request).

Readings taken where the pages are silent (all listed in the design notes):
  the drafter gives, for each draft position d = 1..D, K candidates sorted by
  log-probability (descending) with their token ids; a tree node at depth d that takes
  rank r carries token ids[d-1][r] and scores parent_score + logp[d-1][r], added in
  float32 from the root down (the root scores 0); best-first pops the highest score,
  ties to the earliest push; expansion is lazy -- popping (d, r) under parent p pushes
  its next sibling (d, r+1) under p and its first child (d+1, 0) under itself -- which,
  for sorted rows, pops the same nodes as pushing all K children of every popped node;
  node indices are pop order (root = 0); a -inf log-probability marks an absent
  candidate (rows shorter than K).  Accept follows, from the root, the child whose
  token equals the target model's greedy next token at the current node (lowest index
  first if several do), and ends with that next token (the bonus token).
"""
from __future__ import annotations

import heapq
from typing import List, Sequence, Tuple

import numpy as np


def build_ddtree(logp: np.ndarray, token_ids: np.ndarray, root_token: int, budget: int):
    """Best-first draft tree of one request.

    logp [D, K] float32 (rows sorted descending; -inf = no candidate), token_ids [D, K]
    int32.
    Returns a dict of int32 arrays over nodes 0..n (n <= budget drafted nodes): parent,
    token, depth, rank, first_child, next_sibling, plus float32 ``score``."""
    lp = np.asarray(logp, dtype=np.float32)
    ids = np.asarray(token_ids, dtype=np.int32)
    n_depth, top_k = lp.shape
    parent: List[int] = [-1]
    token: List[int] = [int(root_token)]
    depth: List[int] = [0]
    rank: List[int] = [-1]
    score: List[np.float32] = [np.float32(0.0)]
    heap: List[Tuple[float, int, int, int, int]] = []
    counter = 0

    def push(s: np.float32, d: int, r: int, p: int):
        nonlocal counter
        # heap order: higher score first, then earlier push
        heapq.heappush(heap, (-float(s), counter, d, r, p))
        counter += 1

    def candidate(d: int, r: int) -> bool:  # (depth d, rank r) exists; -inf = no candidate
        return d <= n_depth and r < top_k and lp[d - 1, r] > -np.inf

    if budget >= 1 and candidate(1, 0):
        push(np.float32(score[0] + lp[0, 0]), 1, 0, 0)
    while heap and len(parent) - 1 < budget:
        _, _, d, r, p = heapq.heappop(heap)
        node = len(parent)
        parent.append(p)
        token.append(int(ids[d - 1, r]))
        depth.append(d)
        rank.append(r)
        score.append(np.float32(score[p] + lp[d - 1, r]))
        if candidate(d, r + 1):
            push(np.float32(score[p] + lp[d - 1, r + 1]), d, r + 1, p)
        if candidate(d + 1, 0):
            push(np.float32(score[node] + lp[d, 0]), d + 1, 0, node)
    n = len(parent)
    first_child = np.full(n, -1, np.int32)
    next_sibling = np.full(n, -1, np.int32)
    last_child = np.full(n, -1, np.int64)
    for i in range(1, n):  # children in index order
        p = parent[i]
        if first_child[p] < 0:
            first_child[p] = i
        else:
            next_sibling[last_child[p]] = i
        last_child[p] = i
    return {"parent": np.asarray(parent, np.int32), "token": np.asarray(token, np.int32),
            "depth": np.asarray(depth, np.int32), "rank": np.asarray(rank, np.int32),
            "score": np.asarray(score, np.float32), "first_child": first_child,
            "next_sibling": next_sibling}


def build_ddtree_batch(logp: np.ndarray, token_ids: np.ndarray, root_token: Sequence[int],
                       budget: int):
    """build_ddtree for every request; returns padded [batch, budget + 1] int32 arrays
    (entries past q_len[b] are -1) and q_len [batch]."""
    batch = logp.shape[0]
    width = budget + 1
    out = {k: np.full((batch, width), -1, np.int32)
           for k in ("parent", "token", "depth", "first_child", "next_sibling")}
    q_len = np.zeros(batch, np.int32)
    for b in range(batch):
        t = build_ddtree(logp[b], token_ids[b], int(root_token[b]), budget)
        n = len(t["parent"])
        q_len[b] = n
        for k in out:
            out[k][b, :n] = t[k]
    out["q_len"] = q_len
    return out


def tree_accept(token: Sequence[int], first_child: Sequence[int], next_sibling: Sequence[int],
                target_next: Sequence[int]):
    """Greedy follow-verified-tree walk of one request.

    target_next[i] is the target model's greedy next token after node i.  Returns
    (accepted draft node indices, accepted tokens ending with the bonus token)."""
    nodes: List[int] = []
    tokens: List[int] = []
    cur = 0
    while True:
        want = int(target_next[cur])
        c = int(first_child[cur])
        while c >= 0 and int(token[c]) != want:
            c = int(next_sibling[c])
        if c < 0:
            tokens.append(want)  # bonus token: the target's own next token
            return nodes, tokens
        nodes.append(c)
        tokens.append(want)
        cur = c
