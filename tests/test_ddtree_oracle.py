"""Pins of the CPU oracle for the draft-tree builder and the greedy accept walk.

Builder: a hand-worked tie-break fixture; brute force over every path of small tables
(the nodes are the top-`budget` paths by float32 score, popped in descending order);
a table where float32 accumulation orders the nodes differently from float64; chain,
underfull and absent-candidate trees.  Accept: brute force over root-to-node paths and
closed forms.  Planted mistakes in the oracle must fail these pins.
"""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import ddtree_f32 as D
from tree_verify_mla_attn_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _paths(logp, dtype):
    """Every path (rank tuple) with its score accumulated root -> leaf in `dtype`."""
    n_depth, k = logp.shape
    out = []
    for d in range(1, n_depth + 1):
        for ranks in itertools.product(range(k), repeat=d):
            if any(not np.isfinite(logp[i, r]) for i, r in enumerate(ranks)):
                continue
            s = dtype(0.0)
            for i, r in enumerate(ranks):
                s = dtype(s + dtype(logp[i, r]))
            out.append((ranks, s))
    return out


def _tree_paths(t):
    """Rank tuple of every drafted node (root excluded)."""
    paths = {0: ()}
    for i in range(1, len(t["parent"])):
        paths[i] = paths[int(t["parent"][i])] + (int(t["rank"][i]),)
    return [paths[i] for i in range(1, len(t["parent"]))]


def _brute_force_order(logp, budget, dtype=np.float32):
    ps = _paths(logp, dtype)
    scores = [float(s) for _, s in ps]
    assert len(set(scores)) == len(scores), "ties: brute force order undefined"
    ps.sort(key=lambda x: -float(x[1]))
    return [r for r, _ in ps[:budget]]


def test_golden_tie_break():
    with open(os.path.join(GOLDEN, "ddtree_tie_break.json")) as f:
        g = json.load(f)
    t = D.build_ddtree(np.array(g["logp"], np.float32), np.array(g["token_ids"], np.int32),
                       g["root_token"], g["budget"])
    for k, v in g["expected"].items():
        np.testing.assert_array_equal(t[k], np.array(v, t[k].dtype), err_msg=k)


@pytest.mark.parametrize("depth,k,budget,seed", [(3, 3, 10, 0), (4, 2, 15, 1), (2, 5, 12, 2),
                                                 (5, 2, 31, 3), (3, 4, 40, 4)])
def test_brute_force_best_first(depth, k, budget, seed):
    rng = np.random.default_rng(seed)
    logp = synth.logprob_table(rng, k, depth).astype(np.float32)
    ids = np.arange(depth * k, dtype=np.int32).reshape(depth, k)
    t = D.build_ddtree(logp, ids, 7, budget)
    expect = _brute_force_order(logp, budget)
    assert _tree_paths(t) == expect
    # structure: parents precede children, tokens from the tables, scores are path sums
    assert t["parent"][0] == -1 and (t["parent"][1:] < np.arange(1, len(t["parent"]))).all()
    for i, ranks in enumerate(expect, start=1):
        assert t["token"][i] == ids[len(ranks) - 1, ranks[-1]]
        assert t["depth"][i] == len(ranks)


def _rounding_chain():
    """Depth-3 chain [-1, -0.6u, -0.6u] (u = 2^-23): adding in float32 from the root down
    gives -1 - u, then -1 - 2u; the exact sum -1 - 1.2u rounds to -1 - u."""
    u = 2.0 ** -23
    return np.array([[-1.0], [-0.6 * u], [-0.6 * u]], np.float32)


def test_float32_accumulation():
    lp = _rounding_chain()
    t = D.build_ddtree(lp, np.zeros(lp.shape, np.int32), 0, 3)
    u = 2.0 ** -23
    expect = np.array([0.0, -1.0, -1.0 - u, -1.0 - 2 * u], np.float32)
    assert t["score"].tobytes() == expect.tobytes()
    assert np.float32(-1.0 - 1.2 * u) != expect[3]  # the exact sum rounds elsewhere


def test_chain_underfull_and_absent_candidates():
    lp = synth.logprob_table(np.random.default_rng(5), 1, 15).astype(np.float32)
    t = D.build_ddtree(lp, np.zeros((15, 1), np.int32), 1, 64)  # K = 1: a chain of 15
    np.testing.assert_array_equal(t["parent"], np.arange(-1, 15))
    np.testing.assert_array_equal(t["depth"], np.arange(16))
    lp = synth.logprob_table(np.random.default_rng(6), 2, 2).astype(np.float32)
    t = D.build_ddtree(lp, np.zeros((2, 2), np.int32), 1, 64)  # underfull: 2 + 4 nodes
    assert len(t["parent"]) == 7
    lp = np.array([[-0.5, -1.0, -np.inf], [-0.2, -np.inf, -np.inf]], np.float32)
    t = D.build_ddtree(lp, np.arange(6, dtype=np.int32).reshape(2, 3), 9, 64)
    assert len(t["parent"]) == 5 and t["rank"].max() <= 1  # 2 depth-1 nodes, 1 child each
    assert D.build_ddtree(lp, np.zeros((2, 3), np.int32), 9, 0)["parent"].tolist() == [-1]


def test_children_pointers_match_parents():
    lp, ids, root = synth.draft_tables(np.random.default_rng(7), 4, [8, 2, 4, 3])
    for b in range(4):
        t = D.build_ddtree(lp[b], ids[b], root[b], 64)
        kids = synth.children_lists(t["parent"])
        for i in range(len(t["parent"])):
            walk, c = [], int(t["first_child"][i])
            while c >= 0:
                walk.append(c)
                c = int(t["next_sibling"][c])
            assert walk == kids[i]


def _brute_force_accept(parent, token, target_next):
    """Longest root-to-node path whose every step takes the target's next token."""
    n = len(parent)
    best = []
    for i in range(n):
        path, x = [], i
        while x > 0:
            path.append(x)
            x = int(parent[x])
        path.reverse()
        prev, ok = 0, True
        for c in path:
            if token[c] != target_next[prev]:
                ok = False
                break
            prev = c
        if ok and len(path) > len(best):
            best = path
    last = best[-1] if best else 0
    return best, [int(token[c]) for c in best] + [int(target_next[last])]


@pytest.mark.parametrize("seed", range(6))
def test_accept_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    lp, ids, root = synth.draft_tables(rng, 1, [8, 2, 4, 3, 2, 6][seed])
    t = D.build_ddtree(lp[0], ids[0], root[0], 64)
    tn = synth.target_next_tokens(rng, t["parent"], t["token"], 0.85, len(t["parent"]))
    nodes, toks = D.tree_accept(t["token"], t["first_child"], t["next_sibling"], tn)
    assert (nodes, toks) == _brute_force_accept(t["parent"], t["token"], tn)


def test_accept_closed_forms():
    lp = synth.logprob_table(np.random.default_rng(8), 1, 10).astype(np.float32)
    ids = np.arange(10, dtype=np.int32).reshape(10, 1) + 100
    t = D.build_ddtree(lp, ids, 5, 64)  # chain 0 -> 1 -> ... -> 10, tokens 100..109
    full = np.append(t["token"][1:], 999).astype(np.int32)  # the target agrees everywhere
    nodes, toks = D.tree_accept(t["token"], t["first_child"], t["next_sibling"], full)
    assert nodes == list(range(1, 11)) and toks == list(range(100, 110)) + [999]
    none = np.full(11, 7, np.int32)  # the target agrees nowhere: only the bonus token
    assert D.tree_accept(t["token"], t["first_child"], t["next_sibling"], none) == ([], [7])


def test_planted_mistakes_fail_the_pins(monkeypatch):
    with open(os.path.join(GOLDEN, "ddtree_tie_break.json")) as f:
        g = json.load(f)
    args = (np.array(g["logp"], np.float32), np.array(g["token_ids"], np.int32),
            g["root_token"], g["budget"])
    real_push = D.heapq.heappush

    def lifo_push(heap, item):  # ties to the latest push
        neg, counter, *rest = item
        real_push(heap, (neg, -counter, *rest))
    monkeypatch.setattr(D.heapq, "heappush", lifo_push)
    assert D.build_ddtree(*args)["parent"].tolist() != g["expected"]["parent"]
    monkeypatch.setattr(D.heapq, "heappush", real_push)
    lp = _rounding_chain()
    monkeypatch.setattr(D.np, "float32", np.float64)  # float64 accumulation
    t = D.build_ddtree(lp, np.zeros(lp.shape, np.int32), 0, 3)
    monkeypatch.undo()
    assert np.float32(t["score"][3]) != np.float32(-1.0 - 2 * 2.0 ** -23)


def _mutant(old, new):
    """A copy of the oracle module with one planted mistake (source text replaced)."""
    import inspect
    import types
    src = inspect.getsource(D)
    assert src.count(old) == 1, old
    mod = types.ModuleType("ddtree_mutant")
    exec(compile(src.replace(old, new), "ddtree_mutant", "exec"), mod.__dict__)
    return mod


def _builder_pins_pass(mod):
    for depth, k, budget, seed in [(3, 3, 10, 0), (4, 2, 15, 1), (2, 5, 12, 2), (5, 2, 31, 3)]:
        logp = synth.logprob_table(np.random.default_rng(seed), k, depth).astype(np.float32)
        t = mod.build_ddtree(logp, np.zeros((depth, k), np.int32), 7, budget)
        if _tree_paths(t) != _brute_force_order(logp, budget):
            return False
        for i in range(1, len(t["parent"])):  # scores are the float32 path sums
            ranks = _tree_paths(t)[i - 1]
            s = np.float32(0.0)
            for d, r in enumerate(ranks):
                s = np.float32(s + logp[d, r])
            if s != t["score"][i]:
                return False
    return True


def _accept_pins_pass(mod):
    for seed in range(6):
        rng = np.random.default_rng(100 + seed)
        lp, ids, root = synth.draft_tables(rng, 1, [8, 2, 4, 3, 2, 6][seed])
        t = D.build_ddtree(lp[0], ids[0], root[0], 64)
        tn = synth.target_next_tokens(rng, t["parent"], t["token"], 0.85, len(t["parent"]))
        got = mod.tree_accept(t["token"], t["first_child"], t["next_sibling"], tn)
        if got != _brute_force_accept(t["parent"], t["token"], tn):
            return False
    return True


def test_unmodified_oracle_passes_the_mutation_harness():
    assert _builder_pins_pass(D) and _accept_pins_pass(D)


@pytest.mark.parametrize("old,new", [
    # the first child pushed under the parent instead of the popped node
    ("push(np.float32(score[node] + lp[d, 0]), d + 1, 0, node)",
     "push(np.float32(score[node] + lp[d, 0]), d + 1, 0, p)"),
    # the child scored from the parent's score
    ("push(np.float32(score[node] + lp[d, 0]), d + 1, 0, node)",
     "push(np.float32(score[p] + lp[d, 0]), d + 1, 0, node)"),
    # the sibling scored with its own rank's log-probability
    ("push(np.float32(score[p] + lp[d - 1, r + 1]), d, r + 1, p)",
     "push(np.float32(score[p] + lp[d - 1, r]), d, r + 1, p)"),
    # heap order by lowest score
    ("heapq.heappush(heap, (-float(s), counter, d, r, p))",
     "heapq.heappush(heap, (float(s), counter, d, r, p))"),
])
def test_planted_builder_mistakes_fail(old, new):
    assert not _builder_pins_pass(_mutant(old, new))


@pytest.mark.parametrize("old,new", [
    # the walk takes the first child whatever its token
    ("while c >= 0 and int(token[c]) != want:", "while False:"),
    # the bonus token taken from the current node instead of the target
    ("tokens.append(want)  # bonus token: the target's own next token",
     "tokens.append(int(token[cur]))"),
    # the walk stops one step early
    ("        nodes.append(c)\n        tokens.append(want)\n        cur = c",
     "        nodes.append(c)\n        tokens.append(want)\n        cur = c\n        tokens.append(int(target_next[cur]))\n        return nodes, tokens"),
])
def test_planted_accept_mistakes_fail(old, new):
    assert not _accept_pins_pass(_mutant(old, new))


# ------------------------------------------------------------------ batch helper
@pytest.mark.parametrize("budget", [0, 5, 32, 64])
def test_batch_helper_pads_per_request_trees(budget):
    """build_ddtree_batch = build_ddtree per request, written into rows of width
    budget + 1 with -1 past each tree, and q_len = the tree's node count."""
    rng = np.random.default_rng(700 + budget)
    logp, ids, root = synth.draft_tables(rng, 5, [8, 2, 4, 1, 3], depth=15, vocab=512)
    logp[4, 3:, :] = -np.inf  # a request whose table ends at depth 3 (underfull tree)
    got = D.build_ddtree_batch(logp, ids, root, budget)
    assert got["q_len"].shape == (5,)
    for b in range(5):
        t = D.build_ddtree(logp[b], ids[b], int(root[b]), budget)
        n = len(t["parent"])
        assert got["q_len"][b] == n
        for k in ("parent", "token", "depth", "first_child", "next_sibling"):
            row = got[k][b]
            assert row.shape == (budget + 1,) and row.dtype == np.int32
            np.testing.assert_array_equal(row[:n], t[k], err_msg=f"{k} b={b}")
            assert (row[n:] == -1).all(), f"{k} b={b} padding"
    # the underfull request (top-3 over 3 depths) has 3 + 9 + 27 candidate paths
    assert got["q_len"][4] == min(budget, 3 + 9 + 27) + 1
