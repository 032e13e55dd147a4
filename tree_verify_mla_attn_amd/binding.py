"""Thin ctypes binding of ``libkdtree_verify.so`` (C ABI in include/kdtree_verify.h).

Argument marshalling only: every step of the computation runs in the HIP kernels.  The
bridge shape -- raw device pointers from torch tensors, the caller's current stream,
the library found through ``$KDTREE_LIB`` or next to the package -- follows "The
Capstone Commit: Validating a Native CUDA DDTree Inference Engine", section "The
Message Itself" (commit body: ctypes bindings accepting device tensors and the current
stream, loaded via an environment variable or the build directory).

There is no fallback: if the library is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import heapq
import math
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
DEFAULT_LIB = os.path.join(HERE, "libkdtree_verify.so")

KDTREE_MAX_QLEN = 65
KDTREE_MAX_BUDGET = 64
KDTREE_MAX_DEPTH = 64
KDTREE_MAX_TABLE = 4096
KDTREE_MAX_ACCEPT_NODES = 4096
KDTREE_DTYPE_FP32 = 0
KDTREE_DTYPE_BF16 = 1
ERRORS = {0: "OK", -1: "null pointer", -2: "bad shape", -3: "bad max_q_len", -4: "bad dtype",
          -5: "bad num_splits / workspace", -6: "non-finite scale", -7: "HIP launch failure",
          -8: "needs more than the static scratch"}
KDTREE_NOALLOC_SCRATCH_BYTES = 128 * 1024 * 1024
STATUS_BITS = {1: "bad q_len", 2: "bad prefix_len", 4: "bad tree_parent", 8: "offset overflow",
               16: "non-finite output", 32: "bf16 input outside the fp16 range"}
D_LATENT = 512
D_ROPE = 64

# entry points sharing the kdtree_verify_attn argument list
ENTRY_POINTS = ("kdtree_verify_attn", "kdtree_verify_attn_prepare", "kdtree_verify_attn_attend")

_lib = None


def lib_path() -> str:
    return os.environ.get("KDTREE_LIB") or DEFAULT_LIB


def load_library():
    """Load the HIP library (once).  Raises RuntimeError if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library not found at {path}; build it with "
                           "`python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.kdtree_max_qlen.restype = i32
    lib.kdtree_max_qlen.argtypes = []
    lib.kdtree_verify_attn_workspace_bytes.restype = sz
    lib.kdtree_verify_attn_workspace_bytes.argtypes = [i64, i64, i32, i32, i32, i32]
    for name in ENTRY_POINTS:
        fn = getattr(lib, name)
        fn.restype = i32
        fn.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp,
                       i32, i32, i32, i64, i64, i32, i32, ctypes.c_float, vp, sz, vp]
    lib.kdtree_verify_attn_noalloc.restype = i32
    lib.kdtree_verify_attn_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp,
                                               vp, i32, i32, i32, i64, i64, i32, i32,
                                               ctypes.c_float, vp]
    lib.kdtree_build_ddtree.restype = i32
    lib.kdtree_build_ddtree.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp,
                                        vp, vp]
    lib.kdtree_pack_tree.restype = i32
    lib.kdtree_pack_tree.argtypes = [vp, vp, vp, i32, i32, i64, vp, vp, vp, vp]
    lib.kdtree_sample_tokens.restype = i32
    lib.kdtree_sample_tokens.argtypes = [vp, i32, i64, i32, i64, ctypes.c_float, ctypes.c_uint64,
                                         ctypes.c_uint64, vp, vp]
    lib.kdtree_tree_accept.restype = i32
    lib.kdtree_tree_accept.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, vp, vp, vp, vp]
    _lib = lib
    return lib


# ---------------------------------------------------------------- C entry points
def kdtree_max_qlen() -> int:
    return int(load_library().kdtree_max_qlen())


def kdtree_verify_attn_workspace_bytes(total_q: int, total_kv: int, batch: int, num_heads: int,
                                       num_splits: int, dtype: int) -> int:
    return int(load_library().kdtree_verify_attn_workspace_bytes(total_q, total_kv, batch,
                                                                 num_heads, num_splits, dtype))


def _raw(name, q_lat, q_rope, kv_lat, k_rope, prefix_len, tree_parent, q_len, scale, out_lat,
         out_lse, stream, batch, num_heads, max_q_len, total_q, total_kv, dtype, num_splits,
         workspace, workspace_bytes, status, split_ratio=1.0) -> int:
    # split_ratio is last here (keyword, default 1: equal splits); in the C signature it
    # follows num_splits
    return int(getattr(load_library(), name)(
        q_lat, q_rope, kv_lat, k_rope, prefix_len, tree_parent, q_len, ctypes.c_float(scale),
        out_lat, out_lse, stream, batch, num_heads, max_q_len, total_q, total_kv, dtype,
        num_splits, ctypes.c_float(split_ratio), workspace, workspace_bytes, status))


def kdtree_verify_attn(*args, **kw) -> int:
    """Raw call: every pointer argument is an integer device address (0 = NULL)."""
    return _raw("kdtree_verify_attn", *args, **kw)


def kdtree_verify_attn_prepare(*args, **kw) -> int:
    """Raw call of the pre-pass phase (same arguments as kdtree_verify_attn)."""
    return _raw("kdtree_verify_attn_prepare", *args, **kw)


def kdtree_verify_attn_attend(*args, **kw) -> int:
    """Raw call of the attention phase (same arguments as kdtree_verify_attn)."""
    return _raw("kdtree_verify_attn_attend", *args, **kw)


def kdtree_verify_attn_noalloc(q_lat, q_rope, kv_lat, k_rope, prefix_len, tree_parent, q_len,
                               scale, out_lat, out_lse, stream, batch, num_heads, max_q_len,
                               total_q, total_kv, dtype, num_splits, status,
                               split_ratio=1.0) -> int:
    """Raw call of the allocation-free variant (no workspace argument; pointers as integer
    device addresses, split_ratio last as in _raw)."""
    return int(load_library().kdtree_verify_attn_noalloc(
        q_lat, q_rope, kv_lat, k_rope, prefix_len, tree_parent, q_len, ctypes.c_float(scale),
        out_lat, out_lse, stream, batch, num_heads, max_q_len, total_q, total_kv, dtype,
        num_splits, ctypes.c_float(split_ratio), status))


def kdtree_build_ddtree(logp, token_ids, root_token, batch, depth, top_k, budget, q_len,
                        tree_parent, tree_token, tree_depth, first_child, next_sibling,
                        tree_score, stream) -> int:
    """Raw call of the draft-tree builder (pointers as integer device addresses)."""
    return int(load_library().kdtree_build_ddtree(
        logp, token_ids, root_token, batch, depth, top_k, budget, q_len, tree_parent,
        tree_token, tree_depth, first_child, next_sibling, tree_score, stream))


def kdtree_pack_tree(q_len, tree_parent, tree_token, batch, width, total_q, packed_parent,
                     packed_token, q_offsets, stream) -> int:
    """Raw call of the padded -> packed tree conversion (pointers as device addresses)."""
    return int(load_library().kdtree_pack_tree(q_len, tree_parent, tree_token, batch, width,
                                               total_q, packed_parent, packed_token, q_offsets,
                                               stream))


def kdtree_tree_accept(tree_token, first_child, next_sibling, q_len, target_next, batch,
                       max_nodes, max_accept, accept_len, accept_tokens, accept_nodes,
                       stream) -> int:
    """Raw call of the greedy tree accept (pointers as integer device addresses)."""
    return int(load_library().kdtree_tree_accept(
        tree_token, first_child, next_sibling, q_len, target_next, batch, max_nodes,
        max_accept, accept_len, accept_tokens, accept_nodes, stream))


def kdtree_sample_tokens(logits, dtype, rows, vocab, row_stride, temperature, seed, offset,
                         tokens, stream) -> int:
    """Raw call of the temperature draw (pointers as integer device addresses)."""
    return int(load_library().kdtree_sample_tokens(logits, dtype, rows, vocab, row_stride,
                                                   ctypes.c_float(temperature), seed, offset,
                                                   tokens, stream))


# ---------------------------------------------------------------- torch convenience
def _check_dev(t, name, dtype, shape):
    import torch  # noqa: F401
    if not t.is_cuda or t.dtype != dtype or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be a contiguous {dtype} GPU tensor of shape {tuple(shape)}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")


def build_ddtree(logp, token_ids, root_token, budget: int, with_score: bool = True):
    """Draft trees of a batch on the device.

    logp fp32 [B, D, K] (rows sorted descending, -inf = absent), token_ids int32 [B, D, K],
    root_token int32 [B].  Returns a dict of [B, budget + 1] tensors (parent, token, depth,
    first_child, next_sibling, and score if ``with_score``; -1 / -inf past q_len) plus
    q_len [B], all on the inputs' device, written on the current stream."""
    import torch
    if logp.dim() != 3:
        raise ValueError("logp must be [batch, depth, top_k]")
    b, d, k = (int(x) for x in logp.shape)
    _check_dev(logp, "logp", torch.float32, (b, d, k))
    _check_dev(token_ids, "token_ids", torch.int32, (b, d, k))
    _check_dev(root_token, "root_token", torch.int32, (b,))
    dev, w = logp.device, int(budget) + 1
    out = {n: torch.empty((b, w), dtype=torch.int32, device=dev)
           for n in ("parent", "token", "depth", "first_child", "next_sibling")}
    out["q_len"] = torch.empty((b,), dtype=torch.int32, device=dev)
    if with_score:
        out["score"] = torch.empty((b, w), dtype=torch.float32, device=dev)
    rc = kdtree_build_ddtree(
        logp.data_ptr(), token_ids.data_ptr(), root_token.data_ptr(), b, d, k, int(budget),
        out["q_len"].data_ptr(), out["parent"].data_ptr(), out["token"].data_ptr(),
        out["depth"].data_ptr(), out["first_child"].data_ptr(), out["next_sibling"].data_ptr(),
        out["score"].data_ptr() if with_score else 0, torch.cuda.current_stream(dev).cuda_stream)
    if rc != 0:
        raise RuntimeError(f"kdtree_build_ddtree failed: {rc} ({ERRORS.get(rc, '?')})")
    return out


def pack_tree(q_len, tree_parent, tree_token=None, total_q: Optional[int] = None):
    """Padded [B, W] tree rows -> packed rows on the device.  Returns (packed_parent
    [total_q], packed_token [total_q] or None, q_offsets int64 [B + 1]); total_q defaults
    to B * W (the capacity: rows past q_offsets[B] are left unwritten)."""
    import torch
    if tree_parent.dim() != 2:
        raise ValueError("tree_parent must be [batch, width]")
    b, w = (int(x) for x in tree_parent.shape)
    _check_dev(tree_parent, "tree_parent", torch.int32, (b, w))
    _check_dev(q_len, "q_len", torch.int32, (b,))
    if tree_token is not None:
        _check_dev(tree_token, "tree_token", torch.int32, (b, w))
    dev = tree_parent.device
    total_q = b * w if total_q is None else int(total_q)
    packed_parent = torch.empty((total_q,), dtype=torch.int32, device=dev)
    packed_token = None if tree_token is None else torch.empty((total_q,), dtype=torch.int32,
                                                               device=dev)
    q_offsets = torch.empty((b + 1,), dtype=torch.int64, device=dev)
    rc = kdtree_pack_tree(q_len.data_ptr(), tree_parent.data_ptr(),
                          0 if tree_token is None else tree_token.data_ptr(), b, w, total_q,
                          packed_parent.data_ptr(),
                          0 if packed_token is None else packed_token.data_ptr(),
                          q_offsets.data_ptr(), torch.cuda.current_stream(dev).cuda_stream)
    if rc != 0:
        raise RuntimeError(f"kdtree_pack_tree failed: {rc} ({ERRORS.get(rc, '?')})")
    return packed_parent, packed_token, q_offsets


def sample_tokens(logits, temperature: float, seed: int, offset: int = 0, vocab=None,
                  tokens=None):
    """The target's next token per row of logits [rows, >= vocab] (fp32 or bf16 on the GPU,
    unit stride along the vocabulary) at temperature T (0 = argmax).  Returns int32
    [rows] on the current stream."""
    import torch
    if logits.dim() != 2 or logits.stride(1) != 1 or not logits.is_cuda:
        raise ValueError("logits must be a GPU tensor [rows, vocab] with unit inner stride")
    if logits.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("logits must be float32 or bfloat16")
    rows = int(logits.shape[0])
    vocab = int(logits.shape[1]) if vocab is None else int(vocab)
    if tokens is None:
        tokens = torch.empty((rows,), dtype=torch.int32, device=logits.device)
    _check_dev(tokens, "tokens", torch.int32, (rows,))
    dt = KDTREE_DTYPE_BF16 if logits.dtype == torch.bfloat16 else KDTREE_DTYPE_FP32
    rc = kdtree_sample_tokens(logits.data_ptr(), dt, rows, vocab, int(logits.stride(0)),
                              float(temperature), int(seed), int(offset), tokens.data_ptr(),
                              torch.cuda.current_stream(logits.device).cuda_stream)
    if rc != 0:
        raise RuntimeError(f"kdtree_sample_tokens failed: {rc} ({ERRORS.get(rc, '?')})")
    return tokens


def tree_accept(tree_token, first_child, next_sibling, q_len, target_next, max_accept: int):
    """Greedy accept of a batch on the device.  The tree arrays and target_next are int32
    [B, N]; q_len int32 [B].  Returns (accept_len [B], accept_tokens [B, max_accept],
    accept_nodes [B, max_accept]), written on the current stream."""
    import torch
    if tree_token.dim() != 2:
        raise ValueError("tree_token must be [batch, max_nodes]")
    b, n = (int(x) for x in tree_token.shape)
    for t, name in ((tree_token, "tree_token"), (first_child, "first_child"),
                    (next_sibling, "next_sibling"), (target_next, "target_next")):
        _check_dev(t, name, torch.int32, (b, n))
    _check_dev(q_len, "q_len", torch.int32, (b,))
    dev = tree_token.device
    acc_len = torch.empty((b,), dtype=torch.int32, device=dev)
    acc_tok = torch.empty((b, int(max_accept)), dtype=torch.int32, device=dev)
    acc_node = torch.empty((b, int(max_accept)), dtype=torch.int32, device=dev)
    rc = kdtree_tree_accept(tree_token.data_ptr(), first_child.data_ptr(), next_sibling.data_ptr(),
                            q_len.data_ptr(), target_next.data_ptr(), b, n, int(max_accept),
                            acc_len.data_ptr(), acc_tok.data_ptr(), acc_node.data_ptr(),
                            torch.cuda.current_stream(dev).cuda_stream)
    if rc != 0:
        raise RuntimeError(f"kdtree_tree_accept failed: {rc} ({ERRORS.get(rc, '?')})")
    return acc_len, acc_tok, acc_node
def choose_num_splits(batch: int, num_heads: int, max_q_len: int, mean_kv: float,
                      dtype: int = KDTREE_DTYPE_BF16, n_cu: int = 256,
                      overhead_keys: int = 800) -> int:
    """Host-side split-KV choice for callers that know their prefix lengths.

    One workgroup runs per CU, so a launch takes ceil(workgroups / n_cu) rounds, and a
    round lasts about one split's keys (whole 32-key tiles) plus a fixed per-workgroup
    cost of ~overhead_keys keys (the query fragment, pipeline start, output rows; fitted
    on MI355X).  Returns the split count in 1..256 with the smallest
    rounds * (chunk + overhead), the smallest count on ties.  It is a starting point, not
    a measurement: it matches swept optima for short and medium prefixes, but for one
    32768-key prefix per request it picks 7 where 16 ran 3.5% faster (smaller chunks keep
    each split's keys within an XCD's L2)."""
    rows_per_block = 128 if dtype == KDTREE_DTYPE_BF16 else 64
    blocks = batch * math.ceil(max_q_len * num_heads / rows_per_block)
    best, best_cost = 1, None
    for s in range(1, 257):
        chunk = math.ceil(math.ceil(mean_kv / s) / 32) * 32
        cost = math.ceil(blocks * s / n_cu) * (chunk + overhead_keys)
        if best_cost is None or cost < best_cost:
            best, best_cost = s, cost
        if chunk <= 32:
            break
    return best


DL_BYTES = 512 * 4  # one fp32 latent output row


def _split_begin(prefix: int, num_splits: int, ratio: float, s: int) -> int:
    # host copy of the kernels' split boundaries (whole 32-key tiles, largest split first
    # for ratio < 1), used only by the schedule model below
    if s <= 0:
        return 0
    if s >= num_splits:
        return prefix
    if ratio >= 1.0:
        b = s * (((prefix + num_splits - 1) // num_splits + 31) // 32 * 32)
    else:
        f = (1.0 - ratio ** s) / (1.0 - ratio ** num_splits)
        b = (int(prefix * f) + 31) // 32 * 32
    return min(b, prefix)


def _schedule_makespan(batch: int, m_tiles: int, prefix: int, q: int, num_splits: int,
                       ratio: float, bf16: bool, n_xcd: int, cu_per_xcd: int,
                       overhead_keys: int) -> float:
    # Makespan (in key units) of one launch of equal requests: each workgroup costs its
    # split's keys (whole 32-key tiles) plus overhead_keys; workgroups are dealt to XCDs
    # as the kernels deal them and list-scheduled on each XCD's CUs.  inf when a split
    # would be empty (fewer splits would do the same work).
    cost = []
    for split in range(num_splits):
        kb = _split_begin(prefix, num_splits, ratio, split) & ~31
        ke = (prefix + q if split == num_splits - 1
              else _split_begin(prefix, num_splits, ratio, split + 1))
        if ke <= kb:
            return math.inf
        cost.append(math.ceil((ke - kb) / 32) * 32 + overhead_keys)
    geo = ratio < 1.0
    queues = [[] for _ in range(n_xcd)]
    for g in range(batch * num_splits):
        split = g // batch if geo else g % num_splits
        if bf16:  # groups of m_tiles row tiles, snake order over the XCDs
            rnd, x = divmod(g, n_xcd)
            queues[(n_xcd - 1 - x) if rnd & 1 else x] += [cost[split]] * m_tiles
        else:     # workgroup i on XCD i mod n_xcd
            for t in range(m_tiles):
                queues[(g * m_tiles + t) % n_xcd].append(cost[split])
    if bf16 and num_splits == 1 and cut_applies(queues, cu_per_xcd):
        # the library's last-round cut: units after an XCD's whole rounds run as pieces
        for i, queue in enumerate(queues):
            whole = len(queue) // cu_per_xcd * cu_per_xcd
            left = len(queue) - whole
            if left and cu_per_xcd // left >= 2:
                k = cu_per_xcd // left
                piece = math.ceil((prefix + q) / 32 / k) * 32 + overhead_keys
                queues[i] = queue[:whole] + [piece] * (left * k)
    worst = 0.0
    for queue in queues:
        cus = [0.0] * cu_per_xcd
        for c in queue:
            heapq.heappush(cus, heapq.heappop(cus) + c)
        worst = max(worst, max(cus))
    return worst


def launch_uses_cut(batch: int, num_heads: int, max_q_len: int, num_splits: int,
                    dtype: int = KDTREE_DTYPE_BF16) -> bool:
    """Whether kdtree_verify_attn runs this launch with the last-round cut (the library's
    rule, evaluated on the host from the same scalars): bf16 inputs, one split, every
    XCD's queue of row tiles at most two whole rounds of its 32 CUs, and some XCD with
    leftover row tiles that can each be cut into two or more pieces; not when
    KDTREE_DISABLE_CUT is set."""
    if dtype != KDTREE_DTYPE_BF16 or num_splits != 1:
        return False
    if os.environ.get("KDTREE_DISABLE_CUT", "0") not in ("", "0"):
        return False
    m_tiles = math.ceil(max_q_len * num_heads / 128)
    full_rounds, rem = divmod(batch, 8)
    cut = False
    for x in range(8):
        pos = 7 - x if full_rounds & 1 else x
        n = (full_rounds + (1 if pos < rem else 0)) * m_tiles
        whole = n // 32 * 32
        left = n - whole
        if whole > 2 * 32:
            return False
        if left and 32 // left >= 2:
            cut = True
    return cut


def cut_applies(queues, cu_per_xcd: int = 32, max_rounds: int = 2) -> bool:
    # the library's rule for the last-round cut of a one-split bf16 launch: every XCD's
    # queue has at most max_rounds whole rounds, and some XCD has units left over that
    # can be cut into at least two pieces each
    if any(len(qu) // cu_per_xcd > max_rounds for qu in queues):
        return False
    return any(0 < len(qu) % cu_per_xcd <= cu_per_xcd // 2 for qu in queues)


def choose_split_ratio(batch: int, num_heads: int, max_q_len: int, mean_kv: float,
                       num_splits: int, dtype: int = KDTREE_DTYPE_BF16, n_xcd: int = 8,
                       cu_per_xcd: int = 32, overhead_keys: int = 600) -> float:
    """Host-side choice of split_ratio for a given split count, from a schedule model.

    Each workgroup costs its split's keys (whole 32-key tiles) plus ~overhead_keys.  The
    model deals workgroups to XCDs as the kernels do (bf16: groups of row tiles of one
    request and split, snake order over the XCDs, request-major for equal splits and
    split-major for geometric ones; fp32: workgroup i to XCD i mod 8), list-schedules
    each XCD's queue on its CUs, and returns the ratio in {1, 0.95, ..., 0.05} with the
    shortest makespan (1 unless another is more than 1% shorter), among the ratios that
    leave no split empty.  Requests are taken as equal, mean_kv keys each.  On MI355X it
    reproduces the swept optima: 0.4 for 8 requests of 4096 + 65 keys at 2 splits, 0.85
    for 4 of 32768 + 65 at 16 splits."""
    if num_splits <= 1:
        return 1.0
    bf16 = dtype == KDTREE_DTYPE_BF16
    m_tiles = math.ceil(max_q_len * num_heads / (128 if bf16 else 64))
    prefix = max(0, int(round(mean_kv)) - max_q_len)
    span = lambda r: _schedule_makespan(batch, m_tiles, prefix, max_q_len, num_splits, r,
                                        bf16, n_xcd, cu_per_xcd, overhead_keys)
    equal = span(1.0)
    best, best_r = min((span(k / 20), -k / 20) for k in range(1, 20))
    return -best_r if best < 0.99 * equal else 1.0


def choose_splits(batch: int, num_heads: int, max_q_len: int, mean_kv: float,
                  n_xcd: int = 8, cu_per_xcd: int = 32, overhead_keys: int = 600,
                  us_per_key: float = 1.79 / 32, merge_gbs: float = 4300.0,
                  merge_fixed_us: float = 6.0) -> tuple:
    """(num_splits, split_ratio) for bf16 inputs: for each split count, the ratio of
    choose_split_ratio(), priced as the schedule model's makespan (us_per_key: one
    32-key tile per ~1.79 us on MI355X) plus the split path's fill and merge (its
    partials read once, the output written once, at ~merge_gbs GB/s).  Returns the
    cheapest pair, fewer splits on ties.  Its picks matched the fastest of those timed on
    MI355X for 4 requests with 65-node trees and 64 heads: 4 splits at ratio 0.75 for
    4096-key prefixes (0.251 ms; 3 equal splits 0.301 ms), 8 at 0.75 for 32768-key ones
    (1.148 ms; 16 at 0.85 1.247 ms); for 8 requests of 4096 keys, 1 split with the
    library's last-round cut (0.317 ms; 2 splits at 0.4 0.388 ms)."""
    m_tiles = math.ceil(max_q_len * num_heads / 128)
    prefix = max(0, int(round(mean_kv)) - max_q_len)
    rows = batch * max_q_len * num_heads
    best = None
    for s in range(1, 65):
        # a bound that only grows with s: the work spread evenly over every CU, plus the
        # merge; once it reaches the best time so far, no larger count can beat it
        bound = (batch * m_tiles * (prefix + max_q_len + s * overhead_keys) * us_per_key
                 / (n_xcd * cu_per_xcd))
        if s > 1:
            bound += (s + 1) * rows * (DL_BYTES + 4) / (merge_gbs * 1e3) + merge_fixed_us
        if best is not None and bound >= best[0]:
            break
        r = choose_split_ratio(batch, num_heads, max_q_len, mean_kv, s, KDTREE_DTYPE_BF16,
                               n_xcd, cu_per_xcd, overhead_keys)
        span = _schedule_makespan(batch, m_tiles, prefix, max_q_len, s, r, True, n_xcd,
                                  cu_per_xcd, overhead_keys)
        if span == math.inf:
            continue
        t = span * us_per_key
        if s > 1:
            t += (s + 1) * rows * (DL_BYTES + 4) / (merge_gbs * 1e3) + merge_fixed_us
        else:  # the last-round cut's piece merge, when the library applies it
            queues = [[0] * (m_tiles * (batch // n_xcd + (x < batch % n_xcd)))
                      for x in range(n_xcd)]
            if cut_applies(queues, cu_per_xcd):
                cut_rows = sum(len(qu) % cu_per_xcd for qu in queues) * 128
                t += cu_per_xcd * cut_rows * (DL_BYTES + 4) / (merge_gbs * 1e3) + merge_fixed_us
        if best is None or t < best[0]:
            best = (t, s, r)
        if (prefix + s - 1) // s <= 32:
            break
    return best[1], best[2]

class VerifyAttn:
    """Reusable call object: checks and caches shapes, allocates outputs / workspace with
    torch on the inputs' device, launches on the current stream."""

    def __init__(self):
        load_library()

    @staticmethod
    def _check(t, name, dtype, shape_tail, torch):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if t.dtype != dtype:
            raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if tuple(t.shape[1:]) != tuple(shape_tail):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected [*, {shape_tail}]")

    def __call__(self, q_lat, q_rope, kv_lat, k_rope, prefix_len, tree_parent, q_len, scale,
                 out_lat=None, out_lse=None, num_splits: int = 1,
                 max_q_len: int = KDTREE_MAX_QLEN, workspace=None, status=None,
                 phase: str = "all", mid_event=None, split_ratio: float = 1.0):
        """phase: "all" (kdtree_verify_attn), "prepare" or "attend" (the two halves; an
        "attend" call needs the `workspace` of a "prepare" call on the same inputs).
        mid_event: with phase "all", a torch.cuda.Event recorded on the stream between
        the two halves (the halves are then issued as two calls).
        split_ratio: 1 = equal split-KV chunks; r < 1 = geometric chunks, largest first."""
        import torch
        dtype = q_lat.dtype
        if dtype not in (torch.float32, torch.bfloat16):
            raise ValueError("inputs must be float32 or bfloat16")
        if q_lat.dim() != 3:
            raise ValueError("q_lat must be [total_q, H, 512]")
        total_q, h = int(q_lat.shape[0]), int(q_lat.shape[1])
        self._check(q_lat, "q_lat", dtype, (h, D_LATENT), torch)
        self._check(q_rope, "q_rope", dtype, (h, D_ROPE), torch)
        self._check(kv_lat, "kv_lat", dtype, (D_LATENT,), torch)
        self._check(k_rope, "k_rope", dtype, (D_ROPE,), torch)
        if int(q_rope.shape[0]) != total_q or int(k_rope.shape[0]) != int(kv_lat.shape[0]):
            raise ValueError("row counts of q_lat/q_rope or kv_lat/k_rope differ")
        batch = int(q_len.shape[0])
        for t, n, rows in ((prefix_len, "prefix_len", batch), (q_len, "q_len", batch),
                           (tree_parent, "tree_parent", total_q)):
            if not t.is_cuda or t.dtype != torch.int32 or not t.is_contiguous() or t.dim() != 1 \
                    or int(t.shape[0]) != rows:
                raise ValueError(f"{n} must be a contiguous int32 GPU vector of length {rows}")
        dev = q_lat.device
        if out_lat is None:
            out_lat = torch.empty((total_q, h, D_LATENT), dtype=torch.float32, device=dev)
        if out_lse is None:
            out_lse = torch.empty((total_q, h), dtype=torch.float32, device=dev)
        if out_lat.dtype != torch.float32 or out_lse.dtype != torch.float32 \
                or tuple(out_lat.shape) != (total_q, h, D_LATENT) or tuple(out_lse.shape) != (total_q, h) \
                or not out_lat.is_contiguous() or not out_lse.is_contiguous():
            raise ValueError("out_lat / out_lse must be contiguous float32 [total_q, H, 512] / [total_q, H]")
        total_kv = int(kv_lat.shape[0])
        dt = KDTREE_DTYPE_BF16 if dtype == torch.bfloat16 else KDTREE_DTYPE_FP32
        need = kdtree_verify_attn_workspace_bytes(total_q, total_kv, batch, h, int(num_splits), dt)
        if need and phase != "all":
            # the two halves must share the caller's buffer: a fresh one would hold no
            # pre-pass output (attend) or be thrown away (prepare)
            if workspace is None:
                raise ValueError(f"phase {phase!r} needs the caller's workspace "
                                 f"({need} bytes for num_splits={num_splits})")
            if workspace.numel() * workspace.element_size() < need:
                raise ValueError(f"workspace of {workspace.numel() * workspace.element_size()} "
                                 f"bytes, {need} needed for num_splits={num_splits}")
        if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        ws_ptr = workspace.data_ptr() if (workspace is not None and need) else 0
        ws_bytes = workspace.numel() * workspace.element_size() if ws_ptr else 0
        torch_stream = torch.cuda.current_stream(dev)
        args = (q_lat.data_ptr(), q_rope.data_ptr(), kv_lat.data_ptr(), k_rope.data_ptr(),
                prefix_len.data_ptr(), tree_parent.data_ptr(), q_len.data_ptr(), float(scale),
                out_lat.data_ptr(), out_lse.data_ptr(), torch_stream.cuda_stream, batch, h,
                int(max_q_len), total_q, total_kv, dt, int(num_splits), ws_ptr, ws_bytes,
                status.data_ptr() if status is not None else 0)
        if phase == "all" and mid_event is None:
            names = ["kdtree_verify_attn"]
        elif phase == "all":
            names = ["kdtree_verify_attn_prepare", "kdtree_verify_attn_attend"]
        elif phase in ("prepare", "attend"):
            names = ["kdtree_verify_attn_" + phase]
        else:
            raise ValueError(f"unknown phase {phase!r}")
        for i, name in enumerate(names):
            if i == 1:
                mid_event.record(torch_stream)
            rc = _raw(name, *args, split_ratio=float(split_ratio))
            if rc != 0:
                raise RuntimeError(f"{name} failed: {rc} ({ERRORS.get(rc, '?')})")
        return out_lat, out_lse


def verify_attn(*args, **kwargs):
    """verify_attn(q_lat, q_rope, kv_lat, k_rope, prefix_len, tree_parent, q_len, scale,
    out_lat=None, out_lse=None, num_splits=1, max_q_len=65, workspace=None, status=None,
    split_ratio=1.0) -> (out_lat [total_q, H, 512] fp32, out_lse [total_q, H] fp32)."""
    return VerifyAttn()(*args, **kwargs)


def decode_status(value: int):
    return [name for bit, name in STATUS_BITS.items() if value & bit]
