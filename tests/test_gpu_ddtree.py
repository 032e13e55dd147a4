"""GPU parity of the draft-tree builder, the tree packing and the greedy accept against the
CPU oracle (oracle/ddtree_f32.py), and the on-device build -> verify -> accept chain.

Bar: bit-exact.  Every integer output (parents, tokens, depths, child / sibling pointers,
q_len, accepted tokens and nodes, accept lengths) and the float32 node scores must equal
the oracle's exactly: the scores are the same float32 additions in the same order.
"""
import numpy as np
import pytest
import torch

from oracle import ddtree_f32 as O
from oracle import verify_attn as oracle_verify_attn
from tree_verify_mla_attn_amd import binding as B
from tree_verify_mla_attn_amd import synth

pytestmark = pytest.mark.gpu

FIELDS = ("parent", "token", "depth", "first_child", "next_sibling")


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.load_library()
    return torch.device("cuda:0")


def _i32(x, dev):
    return torch.from_numpy(np.ascontiguousarray(x, np.int32)).to(dev)


def _f32(x, dev):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev)


def gpu_build(logp, ids, root, budget, dev):
    t = B.build_ddtree(_f32(logp, dev), _i32(ids, dev), _i32(root, dev), budget)
    torch.cuda.synchronize(dev)
    return {k: v.cpu().numpy() for k, v in t.items()}


def check_build(name, logp, ids, root, budget, dev):
    print(f"case build/{name} batch={logp.shape[0]} depth={logp.shape[1]} "
          f"top_k={logp.shape[2]} budget={budget}", flush=True)
    g = gpu_build(logp, ids, root, budget, dev)
    r = O.build_ddtree_batch(logp, ids, root, budget)
    np.testing.assert_array_equal(g["q_len"], r["q_len"], err_msg=f"{name}: q_len")
    for k in FIELDS:
        np.testing.assert_array_equal(g[k], r[k], err_msg=f"{name}: {k}")
    # scores: bit-exact float32, -inf past q_len
    for b in range(logp.shape[0]):
        t = O.build_ddtree(logp[b], ids[b], int(root[b]), budget)
        n = len(t["parent"])
        assert g["score"][b, :n].view(np.uint32).tolist() == t["score"].view(np.uint32).tolist(), \
            f"{name}: scores of request {b}"
        assert np.all(np.isneginf(g["score"][b, n:])), f"{name}: score padding"
    print(f"[build/{name}] q_len {int(g['q_len'].min())}..{int(g['q_len'].max())} exact",
          flush=True)
    return g


# ------------------------------------------------------------------ builder
def test_build_max_budget_deep15_batch64(dev):
    """Budget 64 (q_len 65), depth 15, batch 64, top-K 8."""
    rng = np.random.default_rng(100)
    logp, ids, root = synth.draft_tables(rng, 64, 8, depth=15)
    g = check_build("maxbudget_deep15_b64", logp, ids, root, 64, dev)
    assert (g["q_len"] == 65).all()


def test_build_mixed_top_k_budget32(dev):
    """The mixed workload's trees: 32 requests at K=8 and 32 at K=2 (absent columns)."""
    rng = np.random.default_rng(101)
    logp, ids, root = synth.draft_tables(rng, 64, [8] * 32 + [2] * 32, depth=15)
    check_build("mixed_k8_k2_b64", logp, ids, root, 32, dev)


def test_build_chain(dev):
    """Top-1 tables: every tree is a chain of min(depth, budget) drafted nodes."""
    rng = np.random.default_rng(102)
    logp, ids, root = synth.draft_tables(rng, 8, 1, depth=15)
    g = check_build("chain_k1", logp, ids, root, 64, dev)
    assert (g["q_len"] == 16).all()
    assert (g["parent"][:, 1:16] == np.arange(15)).all()


def test_build_underfull(dev):
    """Tables with fewer paths than the budget: the whole candidate tree is drafted."""
    rng = np.random.default_rng(103)
    logp, ids, root = synth.draft_tables(rng, 5, 2, depth=3)
    g = check_build("underfull_d3_k2", logp, ids, root, 64, dev)
    assert (g["q_len"] == 1 + 2 + 4 + 8).all()


def test_build_deep_and_wide_limits(dev):
    """Depth 64 x top-K 64 (the 4096-entry table limit) and top-K 4095 at depth 1."""
    rng = np.random.default_rng(104)
    logp = np.stack([synth.logprob_table(rng, 64, 64).astype(np.float32) for _ in range(3)])
    ids = rng.integers(0, synth.VOCAB, size=logp.shape).astype(np.int32)
    root = rng.integers(0, synth.VOCAB, size=3).astype(np.int32)
    check_build("d64_k64", logp, ids, root, 64, dev)
    logp = np.stack([synth.logprob_table(rng, 4095, 1).astype(np.float32) for _ in range(2)])
    ids = rng.integers(0, synth.VOCAB, size=logp.shape).astype(np.int32)
    g = check_build("d1_k4095", logp, ids, root[:2], 64, dev)
    assert (g["depth"][:, 1:] == 1).all()


def test_build_budget_zero_and_one(dev):
    rng = np.random.default_rng(105)
    logp, ids, root = synth.draft_tables(rng, 3, 4, depth=5)
    g = check_build("budget0", logp, ids, root, 0, dev)
    assert (g["q_len"] == 1).all() and (g["token"][:, 0] == root).all()
    check_build("budget1", logp, ids, root, 1, dev)


def test_build_ties(dev):
    """Heavy ties: log-probabilities drawn from three values, so equal scores are common
    and the earliest-push rule decides the order."""
    rng = np.random.default_rng(106)
    vals = np.array([-0.5, -1.0, -1.5], np.float32)
    logp = -np.sort(-rng.choice(vals, size=(16, 8, 4)), axis=2).astype(np.float32)
    ids = rng.integers(0, synth.VOCAB, size=logp.shape).astype(np.int32)
    root = rng.integers(0, synth.VOCAB, size=16).astype(np.int32)
    check_build("ties", logp, ids, root, 48, dev)


def test_build_golden_tie_fixture(dev):
    import json
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "ddtree_tie_break.json")
    with open(path) as f:
        gd = json.load(f)
    logp = np.array(gd["logp"], np.float32)[None]
    ids = np.array(gd["token_ids"], np.int32)[None]
    g = check_build("golden_tie", logp, ids, np.array([gd["root_token"]], np.int32),
                    gd["budget"], dev)
    exp = np.array(gd["expected"]["parent"], np.int32)
    np.testing.assert_array_equal(g["parent"][0, :len(exp)], exp)


def test_build_absent_rows_and_extremes(dev):
    """-inf past a per-position length; very negative and very close log-probabilities."""
    rng = np.random.default_rng(107)
    logp, ids, root = synth.draft_tables(rng, 6, 6, depth=8)
    for b in range(6):
        for d in range(8):
            logp[b, d, int(rng.integers(1, 7)):] = -np.inf
    logp[0] *= np.float32(1e5)
    logp[1] = np.float32(-1e-6) * np.arange(1, 7, dtype=np.float32)[None, :].repeat(8, 0)
    logp[1, 3:, 2:] = -np.inf
    check_build("absent_extremes", logp, ids, root, 64, dev)


def test_build_no_first_candidate(dev):
    """A table whose first position has no candidate: the root alone."""
    logp = np.full((2, 3, 2), -np.inf, np.float32)
    logp[1] = -1.0
    ids = np.arange(12, dtype=np.int32).reshape(2, 3, 2)
    g = check_build("no_first", logp, ids, np.array([7, 9], np.int32), 5, dev)
    assert g["q_len"].tolist() == [1, 6]


# ------------------------------------------------------------------ packing
def test_pack_tree_layout(dev):
    rng = np.random.default_rng(110)
    logp, ids, root = synth.draft_tables(rng, 16, [8, 2, 1, 4] * 4, depth=15)
    t = B.build_ddtree(_f32(logp, dev), _i32(ids, dev), _i32(root, dev), 32)
    pp, pt, off = B.pack_tree(t["q_len"], t["parent"], t["token"])
    torch.cuda.synchronize(dev)
    r = O.build_ddtree_batch(logp, ids, root, 32)
    q = r["q_len"].astype(np.int64)
    exp_off = np.concatenate([[0], np.cumsum(q)])
    assert off.cpu().numpy().tolist() == exp_off.tolist()
    n = int(exp_off[-1])
    np.testing.assert_array_equal(pp.cpu().numpy()[:n],
                                  np.concatenate([r["parent"][b, :q[b]] for b in range(16)]))
    np.testing.assert_array_equal(pt.cpu().numpy()[:n],
                                  np.concatenate([r["token"][b, :q[b]] for b in range(16)]))


def test_pack_tree_capacity_bound(dev):
    """A request that would end past total_q is left unwritten; earlier ones are packed."""
    par = _i32(np.array([[-1, 0, 0], [-1, 0, 1]]), dev)
    q_len = _i32(np.array([3, 3]), dev)
    pp, _, off = B.pack_tree(q_len, par, total_q=4)
    torch.cuda.synchronize(dev)
    assert off.cpu().numpy().tolist() == [0, 3, 6]
    assert pp.cpu().numpy()[:3].tolist() == [-1, 0, 0]


# ------------------------------------------------------------------ accept
def _accept_case(rng, batch, top_k, depth, budget, p_follow):
    logp, ids, root = synth.draft_tables(rng, batch, top_k, depth=depth)
    tr = O.build_ddtree_batch(logp, ids, root, budget)
    width = budget + 1
    tn = np.full((batch, width), -1, np.int32)
    for b in range(batch):
        n = int(tr["q_len"][b])
        tn[b] = synth.target_next_tokens(rng, tr["parent"][b, :n], tr["token"][b, :n], p_follow,
                                         width)
    return tr, tn


def oracle_accept(tr, tn, max_accept):
    batch, _ = tn.shape
    acc_len = np.zeros(batch, np.int32)
    toks = np.full((batch, max_accept), -1, np.int32)
    nodes = np.full((batch, max_accept), -1, np.int32)
    for b in range(batch):
        nd, tk = O.tree_accept(tr["token"][b], tr["first_child"][b], tr["next_sibling"][b], tn[b])
        if len(nd) > max_accept - 1:  # at most max_accept - 1 drafts, then the bonus token
            nd = nd[:max_accept - 1]
            tk = tk[:max_accept - 1] + [int(tn[b, nd[-1] if nd else 0])]
        acc_len[b] = len(tk)
        toks[b, :len(tk)] = tk
        nodes[b, :len(nd)] = nd
    return acc_len, toks, nodes


def gpu_accept(tr, tn, max_accept, dev):
    al, at, an = B.tree_accept(_i32(tr["token"], dev), _i32(tr["first_child"], dev),
                               _i32(tr["next_sibling"], dev), _i32(tr["q_len"], dev),
                               _i32(tn, dev), max_accept)
    torch.cuda.synchronize(dev)
    return al.cpu().numpy(), at.cpu().numpy(), an.cpu().numpy()


@pytest.mark.parametrize("p_follow", [0.0, 0.6, 0.9, 1.0])
def test_accept_matches_oracle(dev, p_follow):
    rng = np.random.default_rng(int(p_follow * 100) + 120)
    tr, tn = _accept_case(rng, 64, [8] * 32 + [2] * 32, 15, 32, p_follow)
    print(f"case accept p_follow={p_follow}", flush=True)
    g = gpu_accept(tr, tn, 16, dev)
    r = oracle_accept(tr, tn, 16)
    for name, a, e in zip(("accept_len", "accept_tokens", "accept_nodes"), g, r):
        np.testing.assert_array_equal(a, e, err_msg=name)
    print(f"[accept p={p_follow}] lengths {np.bincount(g[0]).tolist()}", flush=True)
    if p_follow == 0.0:
        assert (g[0] == 1).all()
    if p_follow == 1.0:  # always a child to follow: the walk ends only at a leaf
        for b in range(64):
            last = int(g[2][b, g[0][b] - 2])
            assert tr["first_child"][b, last] == -1


def test_accept_lengths_span_1_to_8(dev):
    """Top-2 trees of depth >= 8: accept lengths 1..8 all occur, each matching the oracle."""
    rng = np.random.default_rng(130)
    tr, tn = _accept_case(rng, 64, 2, 15, 64, 0.8)
    g = gpu_accept(tr, tn, 32, dev)
    r = oracle_accept(tr, tn, 32)
    for a, e in zip(g, r):
        np.testing.assert_array_equal(a, e)
    seen = set(g[0].tolist())
    print(f"[accept span] lengths seen {sorted(seen)}", flush=True)
    assert set(range(1, 9)) <= seen


def test_accept_truncation(dev):
    rng = np.random.default_rng(131)
    tr, tn = _accept_case(rng, 32, 1, 15, 64, 1.0)  # chains, always followed
    for ma in (1, 2, 5, 16, 17):
        g = gpu_accept(tr, tn, ma, dev)
        r = oracle_accept(tr, tn, ma)
        for a, e in zip(g, r):
            np.testing.assert_array_equal(a, e, err_msg=f"max_accept={ma}")
        assert (g[0] == min(ma, 16)).all()


# ------------------------------------------------------------------ on-device chain
TOY_VOCAB = 8


def test_build_verify_accept_chain_graph(dev):
    """build -> pack -> verify attention -> toy greedy head -> accept, all on the device
    and captured in one HIP graph; every replay must equal the eager run, and each stage
    must match the oracle (the accept stage on the target tokens the head produced)."""
    rng = np.random.default_rng(140)
    batch, budget, heads, depth = 4, 32, 16, 15
    width = budget + 1
    logp, ids, root = synth.draft_tables(rng, batch, [4, 2, 8, 1], depth=depth, vocab=TOY_VOCAB)
    prefix = np.array([100, 31, 257, 64], np.int32)
    cap_q = batch * width
    cap_kv = int(prefix.sum()) + cap_q
    q_lat = synth.round_to_bf16(rng.standard_normal((cap_q, heads, 512)).astype(np.float32))
    q_rope = synth.round_to_bf16(rng.standard_normal((cap_q, heads, 64)).astype(np.float32))
    kv_lat = synth.round_to_bf16(rng.standard_normal((cap_kv, 512)).astype(np.float32))
    k_rope = synth.round_to_bf16(rng.standard_normal((cap_kv, 64)).astype(np.float32))
    scale = 1.0 / np.sqrt(192.0)

    def bf(x):
        return torch.from_numpy(synth.bf16_bits(x).view(np.int16)).to(dev).view(torch.bfloat16)

    d_logp, d_ids, d_root = _f32(logp, dev), _i32(ids, dev), _i32(root, dev)
    d_prefix = _i32(prefix, dev)
    d_q, d_qr, d_kv, d_kr = bf(q_lat), bf(q_rope), bf(kv_lat), bf(k_rope)
    out_lat = torch.empty((cap_q, heads, 512), dtype=torch.float32, device=dev)
    out_lse = torch.empty((cap_q, heads), dtype=torch.float32, device=dev)
    need = B.kdtree_verify_attn_workspace_bytes(cap_q, cap_kv, batch, heads, 1, 1)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    col = torch.arange(width, device=dev, dtype=torch.int64)

    def step():
        t = B.build_ddtree(d_logp, d_ids, d_root, budget, with_score=False)
        pp, _, off = B.pack_tree(t["q_len"], t["parent"])
        B.verify_attn(d_q, d_qr, d_kv, d_kr, d_prefix, pp, t["q_len"], scale, out_lat=out_lat,
                      out_lse=out_lse, max_q_len=width, workspace=ws)
        # toy greedy head: the target's next token at row i = argmax of head 0's first
        # TOY_VOCAB output features (a stand-in for the target model's LM head)
        nxt = torch.argmax(out_lat[:, 0, :TOY_VOCAB], dim=1).to(torch.int32)
        idx = (off[:-1, None] + col[None, :]).clamp(max=cap_q - 1)
        tn = torch.where(col[None, :] < t["q_len"][:, None], nxt[idx], -1).to(torch.int32)
        al, at, an = B.tree_accept(t["token"], t["first_child"], t["next_sibling"], t["q_len"],
                                   tn, 16)
        return t, off, tn, al, at, an

    print("case chain eager", flush=True)
    t, off, tn, al, at, an = step()
    torch.cuda.synchronize(dev)
    eager = [x.cpu().numpy().copy() for x in (t["parent"], t["token"], t["q_len"], off, tn, al,
                                               at, an)]
    eager_out = out_lat.cpu().numpy().copy()

    # oracle: tree, attention on the packed layout, accept on the head's tokens
    r = O.build_ddtree_batch(logp, ids, root, budget)
    np.testing.assert_array_equal(eager[0], r["parent"])
    np.testing.assert_array_equal(eager[1], r["token"])
    q = r["q_len"].astype(np.int64)
    sq, skv = int(q.sum()), int((prefix + q).sum())
    packed_par = np.concatenate([r["parent"][b, :q[b]] for b in range(batch)])
    r_out, r_lse = oracle_verify_attn(q_lat[:sq].astype(np.float64), q_rope[:sq].astype(np.float64),
                                      kv_lat[:skv].astype(np.float64),
                                      k_rope[:skv].astype(np.float64), prefix, packed_par,
                                      r["q_len"], scale)
    err = np.abs(eager_out[:sq] - r_out)
    assert (err <= 1e-3 + 2e-3 * np.abs(r_out)).all(), f"attention max err {err.max():.3e}"
    tr = dict(token=eager[1], first_child=r["first_child"], next_sibling=r["next_sibling"])
    e_len, e_tok, e_node = oracle_accept(tr, eager[4], 16)
    np.testing.assert_array_equal(eager[5], e_len)
    np.testing.assert_array_equal(eager[6], e_tok)
    np.testing.assert_array_equal(eager[7], e_node)
    print(f"[chain] q_len {r['q_len'].tolist()} accept_len {eager[5].tolist()} "
          f"attention max err {err.max():.3e}", flush=True)

    # graph: capture once, replay with eager work in between, compare every replay
    print("case chain graph", flush=True)
    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(s):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream(dev).wait_stream(s)
    torch.cuda.synchronize(dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gt, goff, gtn, gal, gat, gan = step()
    for rep in range(3):
        out_lat.fill_(float("nan"))
        for x in (gt["parent"], gt["token"], gt["q_len"], goff, gtn, gal, gat, gan):
            x.fill_(-7)
        torch.cuda.synchronize(dev)
        g.replay()
        torch.cuda.synchronize(dev)
        got = [x.cpu().numpy() for x in (gt["parent"], gt["token"], gt["q_len"], goff, gtn, gal,
                                          gat, gan)]
        for i, (a, e) in enumerate(zip(got, eager)):
            np.testing.assert_array_equal(a, e, err_msg=f"replay {rep} output {i}")
        assert np.array_equal(out_lat.cpu().numpy()[:sq], eager_out[:sq]), f"replay {rep} attention"
        print(f"[chain] replay {rep} identical", flush=True)
