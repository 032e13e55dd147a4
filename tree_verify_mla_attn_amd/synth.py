"""Seeded synthetic inputs for tree-verify MLA-absorb attention.

This module only *generates inputs*: draft trees (as parent arrays) and MLA-shaped
query / latent-KV tensors.  It holds none of the attention arithmetic, so both the
HIP path and the float64 oracle can consume what it produces.

Draft trees follow the greedy DDTree step described in "The Milestone Commit:
Cementing Phase 1 ..." (section "The Context", item 1: a best-first tree builder
that replaces a per-request heap on the host) and "Strategic Pivots in CUDA Kernel
Engineering ..." (section "Why This Message Was Written": trees are built from the
drafter's top-k log-probabilities, up to budget 64 / q_len 65, depth up to 15,
batch 64).  The drafter is replaced by random per-depth top-K log-probability
tables: for every depth d = 1..15 there is one list of K log-probabilities, the
log-softmax of K logits drawn from N(0, sigma=2), sorted in descending order.  A
node at depth d that takes rank r scores logp[d][r]; a path scores the sum along
it.  Best-first pops the highest cumulative log-probability first (ties: earlier
insertion first), and a node's index is its pop order, so parent[i] < i.  The root
(node 0) is the last accepted token and is always a query row.

Tensors are drawn N(0, 1) in float32 and, for the bf16 workloads, rounded to
bfloat16 with round-to-nearest-even; the float32 arrays then hold exactly the
bf16 values that the GPU receives.
"""
from __future__ import annotations

import dataclasses
import heapq
from typing import List, Optional, Sequence

import numpy as np

D_LATENT = 512
D_ROPE = 64
MAX_DEPTH = 15
MAX_QLEN = 65
LOGIT_STD = 2.0


# --------------------------------------------------------------------------- bf16
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even); return the raw
    16-bit patterns as uint16.  NaN stays NaN (quiet), infinities stay infinite.
    (uint32 arithmetic cannot wrap: the largest non-NaN pattern is 0xFF800000.)"""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    out = ((u + (np.uint32(0x7FFF) + lsb)) >> np.uint32(16)).astype(np.uint16)
    is_nan = np.isnan(f)
    if is_nan.any():
        out[is_nan] = ((u[is_nan] >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16)
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32 exactly."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 array holding the bfloat16-rounded values of ``x``."""
    return bf16_to_f32(bf16_bits(x))


# -------------------------------------------------------------------------- trees
def logprob_table(rng: np.random.Generator, top_k: int, depth: int = MAX_DEPTH) -> np.ndarray:
    """Per-depth top-K log-probabilities [depth, K], each row sorted descending.

    Row d is the log-softmax of K logits ~ N(0, LOGIT_STD) (the drafter's top-K
    candidates for draft position d+1)."""
    logits = rng.normal(0.0, LOGIT_STD, size=(depth, top_k))
    mx = logits.max(axis=1, keepdims=True)
    lse = mx + np.log(np.exp(logits - mx).sum(axis=1, keepdims=True))
    lp = logits - lse
    return -np.sort(-lp, axis=1)


def best_first_tree(logp: np.ndarray, budget: int):
    """Best-first draft tree over a per-depth log-probability table.

    Returns ``(parent, depth, rank, cum)`` for nodes 0..n (node 0 = root; n <= budget
    drafted nodes).  Lazy expansion: popping (depth d, rank r, parent p) pushes its
    next sibling (d, r+1, p) and its first child (d+1, 0, new node).  Because each
    depth's list is sorted descending, this pops nodes in the same order as pushing
    all K children of every popped node (ties aside)."""
    n_depth, top_k = logp.shape
    parent = [-1]
    depth = [0]
    rank = [-1]
    cum = [0.0]
    heap = []
    counter = 0
    if n_depth >= 1 and top_k >= 1 and budget >= 1:
        heap.append((-(cum[0] + float(logp[0, 0])), counter, 1, 0, 0))
        counter += 1
    while heap and len(parent) - 1 < budget:
        neg, _, d, r, p = heapq.heappop(heap)
        node = len(parent)
        parent.append(p)
        depth.append(d)
        rank.append(r)
        cum.append(-neg)
        if r + 1 < top_k:
            heapq.heappush(heap, (-(cum[p] + float(logp[d - 1, r + 1])), counter, d, r + 1, p))
            counter += 1
        if d + 1 <= n_depth:
            heapq.heappush(heap, (-(cum[node] + float(logp[d, 0])), counter, d + 1, 0, node))
            counter += 1
    return (np.asarray(parent, np.int32), np.asarray(depth, np.int32),
            np.asarray(rank, np.int32), np.asarray(cum, np.float64))


def chain_tree(q_len: int) -> np.ndarray:
    """parent array of a chain: node i's parent is i-1."""
    return np.arange(-1, q_len - 1, dtype=np.int32)


def star_tree(q_len: int) -> np.ndarray:
    """parent array of a star: every node hangs off the root."""
    p = np.zeros(q_len, np.int32)
    p[0] = -1
    return p


def random_tree(rng: np.random.Generator, q_len: int) -> np.ndarray:
    """Uniformly random recursive tree: parent[i] drawn from [0, i)."""
    p = np.empty(q_len, np.int32)
    p[0] = -1
    for i in range(1, q_len):
        p[i] = rng.integers(0, i)
    return p


def tree_depths(parent: np.ndarray) -> np.ndarray:
    """Depth of every node (root = 0) of a parent array with parent[i] < i."""
    d = np.zeros(len(parent), np.int32)
    for i in range(1, len(parent)):
        d[i] = d[parent[i]] + 1
    return d


# ------------------------------------------------------------------------- inputs
@dataclasses.dataclass
class VerifyInputs:
    """One batch of tree-verify attention inputs (host numpy arrays).

    Layout (rows packed, no padding):
      q_lat  [sum_q, H, 512]   q_rope [sum_q, H, 64]
      kv_lat [sum_kv, 512]     k_rope [sum_kv, 64]
    Request b owns query rows [qoff_b, qoff_b + q_len[b]) and KV rows
    [kvoff_b, kvoff_b + prefix_len[b] + q_len[b]): prefix_len[b] prefix rows, then
    the tree tail in node order (tail row j = tree node j; the root at kvoff_b+P_b).
    tree_parent holds local node indices, -1 at each root.
    For dtype 'bf16' the float32 arrays hold bf16-representable values.
    """
    q_lat: np.ndarray
    q_rope: np.ndarray
    kv_lat: np.ndarray
    k_rope: np.ndarray
    prefix_len: np.ndarray
    tree_parent: np.ndarray
    q_len: np.ndarray
    scale: float
    dtype: str
    num_heads: int
    num_splits: int = 1
    name: str = ""
    split_ratio: float = 1.0

    @property
    def batch(self) -> int:
        return int(len(self.q_len))

    @property
    def total_q(self) -> int:
        return int(self.q_len.sum())

    @property
    def total_kv(self) -> int:
        return int((self.prefix_len.astype(np.int64) + self.q_len).sum())

    @property
    def max_q_len(self) -> int:
        return int(self.q_len.max())

    def q_offsets(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.q_len.astype(np.int64))[:-1]])

    def kv_offsets(self) -> np.ndarray:
        kv = self.prefix_len.astype(np.int64) + self.q_len
        return np.concatenate([[0], np.cumsum(kv)[:-1]])

    def parents_of(self, b: int) -> np.ndarray:
        o = int(self.q_offsets()[b])
        return self.tree_parent[o:o + int(self.q_len[b])]

    def algorithmic_flops(self) -> int:
        """2*(576+512) flops per visible (row, key) pair, masked pairs excluded."""
        d_qk = self.q_lat.shape[-1] + self.q_rope.shape[-1]
        d_v = self.kv_lat.shape[-1]
        pairs = 0
        for b in range(self.batch):
            dep = tree_depths(self.parents_of(b)).astype(np.int64)
            pairs += int((int(self.prefix_len[b]) + dep + 1).sum())
        return pairs * self.num_heads * 2 * (d_qk + d_v)

    def algorithmic_bytes(self) -> int:
        """Q once + KV once (input precision) + fp32 latent output + fp32 lse."""
        s_in = 2 if self.dtype == "bf16" else 4
        d_qk = self.q_lat.shape[-1] + self.q_rope.shape[-1]
        rows = self.total_q * self.num_heads
        return (rows * d_qk * s_in + self.total_kv * d_qk * s_in
                + rows * self.kv_lat.shape[-1] * 4 + rows * 4)


def _normal(rng, shape, dtype):
    x = rng.standard_normal(shape, dtype=np.float32)
    return round_to_bf16(x) if dtype == "bf16" else x


def make_inputs(rng: np.random.Generator, *, num_heads: int, prefix_lens: Sequence[int],
                parents: Sequence[np.ndarray], dtype: str, scale: Optional[float] = None,
                d_latent: int = D_LATENT, d_rope: int = D_ROPE, num_splits: int = 1,
                name: str = "") -> VerifyInputs:
    """Draw q_lat, q_rope, kv_lat, k_rope (in that order) ~ N(0,1) for given trees."""
    if dtype not in ("fp32", "bf16"):
        raise ValueError(dtype)
    q_len = np.asarray([len(p) for p in parents], np.int32)
    prefix = np.asarray(prefix_lens, np.int32)
    sum_q = int(q_len.sum())
    sum_kv = int((prefix.astype(np.int64) + q_len).sum())
    q_lat = _normal(rng, (sum_q, num_heads, d_latent), dtype)
    q_rope = _normal(rng, (sum_q, num_heads, d_rope), dtype)
    kv_lat = _normal(rng, (sum_kv, d_latent), dtype)
    k_rope = _normal(rng, (sum_kv, d_rope), dtype)
    if scale is None:
        scale = 1.0 / np.sqrt(192.0)
    return VerifyInputs(q_lat=q_lat, q_rope=q_rope, kv_lat=kv_lat, k_rope=k_rope,
                        prefix_len=prefix, tree_parent=np.concatenate(parents).astype(np.int32),
                        q_len=q_len, scale=float(scale), dtype=dtype, num_heads=num_heads,
                        num_splits=num_splits, name=name)


# ------------------------------------------------------------------------ configs
# The five workloads: batch, heads, prefix, draft budget / top-K, dtype, and the split-KV
# launch configuration (workload 5 prescribes 16 chunks; the others use the count that
# ran fastest on MI355X: small fp32 batches need splits to occupy the chip, and the best
# counts keep the workgroups (row tiles x splits) within one round of the 256 CUs).  Where
# the workgroups overrun whole rounds of the CUs, workload 5 (2112 workgroups) runs
# fastest with geometric chunk sizes (split_ratio < 1, largest first), and workload 3
# (264 row tiles on 256 CUs) with one split, its 33rd row tile per XCD cut into key
# pieces by the library (faster than 2 geometric splits at ratio 0.4).
CONFIGS = {
    1: dict(name="tiny_b1_p256_q9_fp32", batch=1, heads=64, prefix=256, top_k=[8], budget=8,
            dtype="fp32", num_splits=12),
    2: dict(name="b1_p2048_q33_wide_fp32", batch=1, heads=64, prefix=2048, top_k=[8], budget=32,
            dtype="fp32", num_splits=7),
    3: dict(name="b8_p4096_q65_deep_bf16", batch=8, heads=64, prefix=4096, top_k=[2], budget=64,
            dtype="bf16", num_splits=1),
    4: dict(name="b64_ragged1024-8192_q33_mixed_bf16", batch=64, heads=64, prefix=(1024, 8192),
            top_k=[8] * 32 + [2] * 32, budget=32, dtype="bf16", num_splits=1),
    5: dict(name="b4_p32768_q65_split16_bf16", batch=4, heads=64, prefix=32768, top_k=[4],
            budget=64, dtype="bf16", num_splits=16, split_ratio=0.85),
}


def config_trees(cfg: int, rng: Optional[np.random.Generator] = None):
    """Prefix lengths and draft trees of workload ``cfg`` (the first draws of its
    seeded stream).  Returns (rng, prefix_len [B], parents list)."""
    c = CONFIGS[cfg]
    if rng is None:
        rng = np.random.default_rng(1000 + cfg)
    b = c["batch"]
    if isinstance(c["prefix"], tuple):
        lo, hi = c["prefix"]
        prefix = rng.integers(lo, hi + 1, size=b).astype(np.int32)
    else:
        prefix = np.full(b, c["prefix"], np.int32)
    ks = c["top_k"] if len(c["top_k"]) == b else c["top_k"] * b
    parents: List[np.ndarray] = []
    for i in range(b):
        table = logprob_table(rng, ks[i])
        parents.append(best_first_tree(table, c["budget"])[0])
    return rng, prefix, parents


def config_inputs(cfg: int, num_splits: Optional[int] = None,
                  split_ratio: Optional[float] = None) -> VerifyInputs:
    """Seeded inputs of workload ``cfg`` (1..5): rng = default_rng(1000 + cfg).

    Draw order: prefix lengths (ragged workload only), per-request log-prob tables
    and trees, then q_lat, q_rope, kv_lat, k_rope."""
    c = CONFIGS[cfg]
    rng, prefix, parents = config_trees(cfg)
    inp = make_inputs(rng, num_heads=c["heads"], prefix_lens=prefix, parents=parents,
                      dtype=c["dtype"], num_splits=num_splits or c["num_splits"],
                      name=c["name"])
    inp.split_ratio = split_ratio if split_ratio is not None else c.get("split_ratio", 1.0)
    return inp


def device_tensors(inp: VerifyInputs, device="cuda"):
    """Copy a VerifyInputs batch to torch tensors on ``device`` (bf16 bit-exact)."""
    import torch

    def t(x):
        if inp.dtype == "bf16":
            bits = bf16_bits(x).view(np.int16)
            return torch.from_numpy(bits).to(device).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(device)

    def ti(x):
        return torch.from_numpy(np.ascontiguousarray(x, np.int32)).to(device)

    return dict(q_lat=t(inp.q_lat), q_rope=t(inp.q_rope), kv_lat=t(inp.kv_lat),
                k_rope=t(inp.k_rope), prefix_len=ti(inp.prefix_len),
                tree_parent=ti(inp.tree_parent), q_len=ti(inp.q_len))


# ------------------------------------------------------ draft tables and target tokens
VOCAB = 163840


def draft_tables(rng: np.random.Generator, batch: int, top_k, depth: int = MAX_DEPTH,
                 vocab: int = VOCAB):
    """Drafter outputs for the tree builder: per request and draft position, K
    log-probabilities (float32, sorted descending) and K distinct token ids.

    Returns (logp [batch, depth, K] float32, token_ids [batch, depth, K] int32,
    root_token [batch] int32).  ``top_k`` may be one value or one per request (then
    the tables use the largest K and the other requests' extra columns are -inf)."""
    ks = [top_k] * batch if np.isscalar(top_k) else list(top_k)
    kmax = max(ks)
    logp = np.full((batch, depth, kmax), -np.inf, np.float32)
    ids = np.zeros((batch, depth, kmax), np.int32)
    for b in range(batch):
        logp[b, :, :ks[b]] = logprob_table(rng, ks[b], depth).astype(np.float32)
        for d in range(depth):
            ids[b, d] = rng.choice(vocab, size=kmax, replace=False)
    root = rng.integers(0, vocab, size=batch).astype(np.int32)
    return logp, ids, root


def children_lists(parent: np.ndarray) -> List[List[int]]:
    """Children of every node of one tree, in index order."""
    kids: List[List[int]] = [[] for _ in range(len(parent))]
    for i in range(1, len(parent)):
        kids[int(parent[i])].append(i)
    return kids


def target_next_tokens(rng: np.random.Generator, parent: np.ndarray, token: np.ndarray,
                       p_follow: float, width: int, vocab: int = VOCAB) -> np.ndarray:
    """Synthetic target-model greedy next tokens for one tree: at every node, with
    probability p_follow the token of one of its children (chosen uniformly), else a
    random token.  Returns [width] int32 (entries past the tree are -1)."""
    out = np.full(width, -1, np.int32)
    kids = children_lists(parent)
    for i in range(len(parent)):
        if kids[i] and rng.random() < p_follow:
            out[i] = token[kids[i][int(rng.integers(0, len(kids[i])))]]
        else:
            out[i] = int(rng.integers(0, vocab))
    return out
