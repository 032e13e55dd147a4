"""Pins of the float64 oracle against things other than itself.

The pages print no tensor values, so each pin is self-contained:
  * brute force: per (node, head) attention over an explicitly gathered key list
    (prefix + the node's ancestor chain), scalar math.fsum loops;
  * chain tree == bottom-right causal attention computed by torch's SDPA
    (a library routine, not our code), output and log-sum-exp;
  * closed forms: q = 0 / scale = 0 (uniform average), empty prefix root row,
    single-key ranges (lse = the score itself);
  * invariances: prefix permutation, head permutation, non-ancestor perturbation,
    request packing;
  * split + LSE-merge identity;
  * a hand-worked golden example (tests/golden/handworked_star_p1_t3.json);
  * pin sensitivity: deliberately wrong oracle variants (sibling leak, dropped self,
    scale on the latent part only) must fail the brute-force pin.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import verify_attn_f64 as O
from tree_verify_mla_attn_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ helpers
def _path_to_root(parent, i):
    """Explicit ancestor-or-self list of node i (independent of the oracle's mask)."""
    out = []
    while i != -1:
        out.append(int(i))
        i = int(parent[i])
    return out


def _brute_force(inp):
    """Per-row attention, scalar fsum loops over explicitly gathered keys."""
    q_off = inp.q_offsets()
    kv_off = inp.kv_offsets()
    h_n = inp.num_heads
    dl = inp.q_lat.shape[-1]
    out = np.zeros((inp.total_q, h_n, dl))
    lse = np.zeros((inp.total_q, h_n))
    for b in range(inp.batch):
        p = int(inp.prefix_len[b])
        t = int(inp.q_len[b])
        par = inp.parents_of(b)
        for i in range(t):
            keys = list(range(p)) + [p + j for j in _path_to_root(par, i)]
            for h in range(h_n):
                q = [float(x) for x in inp.q_lat[q_off[b] + i, h]] + \
                    [float(x) for x in inp.q_rope[q_off[b] + i, h]]
                scores = []
                for k in keys:
                    kr = [float(x) for x in inp.kv_lat[kv_off[b] + k]] + \
                         [float(x) for x in inp.k_rope[kv_off[b] + k]]
                    scores.append(inp.scale * math.fsum(a * c for a, c in zip(q, kr)))
                m = max(scores)
                w = [math.exp(s - m) for s in scores]
                l = math.fsum(w)
                for f in range(dl):
                    out[q_off[b] + i, h, f] = math.fsum(
                        wk * float(inp.kv_lat[kv_off[b] + k, f]) for wk, k in zip(w, keys)) / l
                lse[q_off[b] + i, h] = m + math.log(l)
    return out, lse


def _tiny_inputs(seed, parents, prefix, heads, dl=8, dr=4, dtype="fp32", scale=None):
    rng = np.random.default_rng(seed)
    return synth.make_inputs(rng, num_heads=heads, prefix_lens=prefix, parents=parents,
                             dtype=dtype, scale=scale, d_latent=dl, d_rope=dr)


def _oracle(inp, **kw):
    return O.verify_attn_inputs(inp, **kw)


# ------------------------------------------------------------------ golden
def test_golden_handworked():
    with open(os.path.join(GOLDEN, "handworked_star_p1_t3.json")) as f:
        g = json.load(f)
    env = {"e": math.e, "log": math.log}
    out, lse = O.verify_attn(np.array(g["q_lat"], float), np.array(g["q_rope"], float),
                             np.array(g["kv_lat"], float), np.array(g["k_rope"], float),
                             g["prefix_len"], g["tree_parent"], g["q_len"], g["scale"])
    exp_out = np.array([[[eval(x, env) for x in row] for row in node]
                        for node in g["expected_out_lat"]])
    exp_lse = np.array([[eval(x, env) for x in node] for node in g["expected_out_lse"]])
    np.testing.assert_allclose(out, exp_out, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, exp_lse, rtol=0, atol=1e-14)


# ------------------------------------------------------------------ brute force
@pytest.mark.parametrize("case", range(8))
def test_brute_force_tiny(case):
    rng = np.random.default_rng(100 + case)
    shapes = [synth.random_tree(rng, int(rng.integers(1, 10))) for _ in range(2)]
    if case == 0:
        shapes = [synth.chain_tree(9), synth.star_tree(6)]
    if case == 1:
        table = synth.logprob_table(rng, 3)
        shapes = [synth.best_first_tree(table, 8)[0], np.array([-1], np.int32)]
    prefix = [int(rng.integers(0, 17)), 0 if case % 2 else int(rng.integers(0, 17))]
    inp = _tiny_inputs(200 + case, shapes, prefix, heads=1 + case % 3,
                       dtype="bf16" if case % 4 == 3 else "fp32",
                       scale=[None, 0.3, 1.0, 0.05][case % 4])
    out, lse = _oracle(inp)
    bo, bl = _brute_force(inp)
    np.testing.assert_allclose(out, bo, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, bl, rtol=0, atol=1e-12)


def test_brute_force_full_mla_dims():
    rng = np.random.default_rng(7)
    parents = [synth.random_tree(rng, 4), synth.chain_tree(3)]
    inp = _tiny_inputs(8, parents, [3, 0], heads=2, dl=512, dr=64)
    out, lse = _oracle(inp)
    bo, bl = _brute_force(inp)
    np.testing.assert_allclose(out, bo, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, bl, rtol=0, atol=1e-12)


# ------------------------------------------------------------------ SDPA chain
@pytest.mark.parametrize("t,p,h", [(9, 7, 4), (17, 40, 2), (1, 5, 3), (6, 0, 2)])
def test_chain_tree_equals_causal_sdpa(t, p, h):
    rng = np.random.default_rng(t * 100 + p)
    inp = synth.make_inputs(rng, num_heads=h, prefix_lens=[p], parents=[synth.chain_tree(t)],
                            dtype="fp32")
    out, lse = _oracle(inp)
    q = torch.from_numpy(np.concatenate([inp.q_lat, inp.q_rope], -1).astype(np.float64))
    k = torch.from_numpy(np.concatenate([inp.kv_lat, inp.k_rope], -1).astype(np.float64))
    v = torch.from_numpy(inp.kv_lat.astype(np.float64))
    q = q.permute(1, 0, 2)[None]                      # [1, H, T, 576]
    k = k[None, None].expand(1, h, p + t, 576)
    v = v[None, None].expand(1, h, p + t, 512)
    causal = torch.tril(torch.ones(t, p + t, dtype=torch.bool), diagonal=p)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=causal,
                                                           scale=inp.scale)
    np.testing.assert_allclose(out, ref[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
    # log-sum-exp from torch's CPU flash kernel (needs equal head dims: pad V)
    v_pad = torch.nn.functional.pad(v, (0, 64))
    add_mask = torch.zeros(t, p + t, dtype=torch.float64).masked_fill(~causal, float("-inf"))
    o2, lse_ref = torch.ops.aten._scaled_dot_product_flash_attention_for_cpu(
        q.contiguous(), k.contiguous(), v_pad.contiguous(), 0.0, False, attn_mask=add_mask,
        scale=inp.scale)[:2]
    np.testing.assert_allclose(out, o2[0, :, :, :512].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref[0].permute(1, 0).numpy(), rtol=0, atol=1e-12)


# ------------------------------------------------------------------ normalisation / mask
def test_probabilities_normalised_and_masked():
    rng = np.random.default_rng(3)
    par = synth.random_tree(rng, 12)
    inp = synth.make_inputs(rng, num_heads=3, prefix_lens=[10], parents=[par], dtype="fp32")
    mask = O.visibility_mask(10, par)
    _, _, probs = O.attend_request(inp.q_lat, inp.q_rope, inp.kv_lat, inp.k_rope, mask,
                                   inp.scale, return_probs=True)
    np.testing.assert_allclose(probs.sum(-1), 1.0, rtol=0, atol=1e-12)
    assert np.all(probs[~np.broadcast_to(mask[:, None, :], probs.shape)] == 0.0)
    assert np.all(probs[np.broadcast_to(mask[:, None, :], probs.shape)] > 0.0)


@pytest.mark.parametrize("seed", range(5))
def test_mask_invariants(seed):
    rng = np.random.default_rng(seed)
    par = synth.random_tree(rng, int(rng.integers(1, 66)))
    m = O.ancestor_or_self_mask(par)
    t = len(par)
    assert m[:, 0].all(), "root visible to every node"
    assert np.diag(m).all(), "every node sees itself"
    depth = synth.tree_depths(par)
    np.testing.assert_array_equal(m.sum(1), depth + 1)
    for i in range(t):
        for j in np.nonzero(m[i])[0]:
            assert not np.any(m[j] & ~m[i]), "ancestor sets are closed"
    assert not np.any(np.triu(m, 1)), "with parent[i] < i only earlier nodes are ancestors"
    vm = O.visibility_mask(5, par)
    assert vm[:, :5].all() and vm.shape == (t, 5 + t)


def test_mask_rejects_malformed_parents():
    with pytest.raises(ValueError):
        O.ancestor_or_self_mask([0, 0])
    with pytest.raises(ValueError):
        O.ancestor_or_self_mask([-1, 2, 1])
    with pytest.raises(ValueError):
        O.ancestor_or_self_mask([-1, 5])


# ------------------------------------------------------------------ closed forms
def test_zero_query_is_mean_of_visible_rows():
    rng = np.random.default_rng(11)
    par = synth.random_tree(rng, 9)
    inp = synth.make_inputs(rng, num_heads=2, prefix_lens=[13], parents=[par], dtype="fp32")
    inp.q_lat[:] = 0.0
    inp.q_rope[:] = 0.0
    out, lse = _oracle(inp)
    for i in range(9):
        rows = list(range(13)) + [13 + j for j in _path_to_root(par, i)]
        for h in range(2):
            np.testing.assert_allclose(out[i, h], inp.kv_lat[rows].astype(np.float64).mean(0),
                                       rtol=0, atol=1e-14)
            assert abs(lse[i, h] - math.log(len(rows))) < 1e-14


def test_zero_scale_is_uniform():
    rng = np.random.default_rng(12)
    par = synth.star_tree(5)
    inp = synth.make_inputs(rng, num_heads=1, prefix_lens=[4], parents=[par], dtype="fp32",
                            scale=0.0)
    out, lse = _oracle(inp)
    for i in range(5):
        rows = list(range(4)) + [4 + j for j in _path_to_root(par, i)]
        np.testing.assert_allclose(out[i, 0], inp.kv_lat[rows].astype(np.float64).mean(0),
                                   rtol=0, atol=1e-14)
        assert abs(lse[i, 0] - math.log(len(rows))) < 1e-14


def test_root_with_empty_prefix_sees_only_itself():
    rng = np.random.default_rng(13)
    par = synth.random_tree(rng, 6)
    inp = synth.make_inputs(rng, num_heads=3, prefix_lens=[0], parents=[par], dtype="fp32")
    out, lse = _oracle(inp)
    for h in range(3):
        np.testing.assert_array_equal(out[0, h], inp.kv_lat[0].astype(np.float64))
        q = np.concatenate([inp.q_lat[0, h], inp.q_rope[0, h]]).astype(np.float64)
        k = np.concatenate([inp.kv_lat[0], inp.k_rope[0]]).astype(np.float64)
        assert abs(lse[0, h] - inp.scale * float(np.dot(q, k))) < 1e-12


def test_single_key_range_lse_is_the_score():
    rng = np.random.default_rng(14)
    par = synth.chain_tree(4)
    inp = synth.make_inputs(rng, num_heads=2, prefix_lens=[6], parents=[par], dtype="fp32")
    for k in range(10):
        out, lse = _oracle(inp, key_range=([k], [k + 1]))
        for i in range(4):
            visible = k < 6 or (k - 6) <= i
            for h in range(2):
                if visible:
                    q = np.concatenate([inp.q_lat[i, h], inp.q_rope[i, h]]).astype(np.float64)
                    kk = np.concatenate([inp.kv_lat[k], inp.k_rope[k]]).astype(np.float64)
                    assert abs(lse[i, h] - inp.scale * float(np.dot(q, kk))) < 1e-12
                    np.testing.assert_array_equal(out[i, h], inp.kv_lat[k].astype(np.float64))
                else:
                    assert lse[i, h] == -np.inf and not out[i, h].any()


# ------------------------------------------------------------------ invariances
def test_prefix_permutation_invariance():
    rng = np.random.default_rng(15)
    par = synth.random_tree(rng, 7)
    inp = synth.make_inputs(rng, num_heads=2, prefix_lens=[20], parents=[par], dtype="fp32")
    out, lse = _oracle(inp)
    perm = rng.permutation(20)
    inp.kv_lat[:20] = inp.kv_lat[perm]
    inp.k_rope[:20] = inp.k_rope[perm]
    out2, lse2 = _oracle(inp)
    np.testing.assert_allclose(out2, out, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, rtol=0, atol=1e-13)


def test_head_permutation_equivariance():
    rng = np.random.default_rng(16)
    par = synth.random_tree(rng, 5)
    inp = synth.make_inputs(rng, num_heads=6, prefix_lens=[9], parents=[par], dtype="fp32")
    out, lse = _oracle(inp)
    perm = rng.permutation(6)
    inp.q_lat = inp.q_lat[:, perm].copy()
    inp.q_rope = inp.q_rope[:, perm].copy()
    out2, lse2 = _oracle(inp)
    np.testing.assert_allclose(out2, out[:, perm], rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse2, lse[:, perm], rtol=0, atol=1e-13)


def test_non_ancestor_tail_row_is_invisible():
    rng = np.random.default_rng(17)
    par = np.array([-1, 0, 0, 1, 2, 1], np.int32)
    inp = synth.make_inputs(rng, num_heads=2, prefix_lens=[5], parents=[par], dtype="fp32")
    out, lse = _oracle(inp)
    # node 3's ancestors: 3, 1, 0; perturb the tail rows of nodes 2, 4, 5
    for j in (2, 4, 5):
        inp.kv_lat[5 + j] += 10.0
        inp.k_rope[5 + j] -= 3.0
    out2, lse2 = _oracle(inp)
    np.testing.assert_allclose(out2[3], out[3], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse2[3], lse[3], rtol=0, atol=1e-14)
    assert np.abs(out2[4] - out[4]).max() > 1e-3, "node 4 sees its own row"


def test_packing_matches_requests_alone():
    rng = np.random.default_rng(18)
    parents = [synth.random_tree(rng, n) for n in (3, 1, 7)]
    prefixes = [4, 0, 9]
    inp = synth.make_inputs(rng, num_heads=2, prefix_lens=prefixes, parents=parents, dtype="fp32")
    out, lse = _oracle(inp)
    qo, ko = inp.q_offsets(), inp.kv_offsets()
    for b in range(3):
        t, p = len(parents[b]), prefixes[b]
        o1, l1 = O.verify_attn(inp.q_lat[qo[b]:qo[b] + t], inp.q_rope[qo[b]:qo[b] + t],
                               inp.kv_lat[ko[b]:ko[b] + p + t], inp.k_rope[ko[b]:ko[b] + p + t],
                               [p], parents[b], [t], inp.scale)
        np.testing.assert_array_equal(out[qo[b]:qo[b] + t], o1)
        np.testing.assert_array_equal(lse[qo[b]:qo[b] + t], l1)


# ------------------------------------------------------------------ split + merge
@pytest.mark.parametrize("nsplit", [2, 3, 5])
def test_split_merge_identity(nsplit):
    rng = np.random.default_rng(19 + nsplit)
    parents = [synth.random_tree(rng, 8), synth.chain_tree(3)]
    inp = synth.make_inputs(rng, num_heads=3, prefix_lens=[30, 2], parents=parents, dtype="fp32")
    out, lse = _oracle(inp)
    n_keys = inp.prefix_len + inp.q_len
    cuts = [np.sort(rng.integers(0, n + 1, size=nsplit - 1)) for n in n_keys]
    bounds = [np.concatenate([[0], c, [n]]) for c, n in zip(cuts, n_keys)]
    outs, lses = [], []
    for s in range(nsplit):
        lo = [int(b[s]) for b in bounds]
        hi = [int(b[s + 1]) for b in bounds]
        o, l = _oracle(inp, key_range=(lo, hi))
        outs.append(o)
        lses.append(l)
    mo, ml = O.lse_merge(outs, lses)
    np.testing.assert_allclose(mo, out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(ml, lse, rtol=0, atol=1e-12)
    np.testing.assert_allclose(ml, np.logaddexp.reduce(np.stack(lses), axis=0), rtol=0, atol=1e-12)


def test_merge_with_empty_parts():
    o = np.ones((2, 4))
    out, lse = O.lse_merge([np.zeros((2, 4)), o * 3.0], [np.full(2, -np.inf), np.array([0.5, -2.0])])
    np.testing.assert_array_equal(out, o * 3.0)
    np.testing.assert_array_equal(lse, [0.5, -2.0])
    out, lse = O.lse_merge([np.zeros((1, 4))] * 2, [np.full(1, -np.inf)] * 2)
    assert lse[0] == -np.inf and not out.any()


# ------------------------------------------------------------------ pin sensitivity
_REAL_VISIBILITY = O.visibility_mask


def _wrong_visibility(kind):
    def vis(prefix_len, parent):
        m = _REAL_VISIBILITY(prefix_len, parent)
        t = len(parent)
        if kind == "sibling_leak":
            for i in range(t):
                if parent[i] >= 0:
                    for j in range(t):
                        if parent[j] == parent[i]:
                            m[i, prefix_len + j] = True
        elif kind == "drop_self":
            for i in range(1, t):
                m[i, prefix_len + i] = False
        elif kind == "descendant_mask":
            # tail block transposed: a node sees its descendants instead of its ancestors
            tail = m[:, prefix_len:].copy()
            m[:, prefix_len:] = tail.T
        return m
    return vis


_REAL_ATTEND = O.attend_request


def _wrong_attend(kind):
    def attend(q_lat, q_rope, kv_lat, k_rope, mask, scale, return_probs=False):
        q_rope = np.asarray(q_rope, float)
        kv_lat = np.asarray(kv_lat, float)
        if kind == "rope_unscaled":      # scale applied to the latent product only
            q_rope = q_rope / scale
        elif kind == "drop_rope":        # rope dims left out of the scores
            q_rope = np.zeros_like(q_rope)
        elif kind == "missing_scale":
            scale = 1.0
        elif kind == "latent_rope_row_skew":  # latent rows one key off from rope rows
            kv_lat = np.roll(kv_lat, 1, axis=0)
        res = _REAL_ATTEND(q_lat, q_rope, kv_lat, k_rope, mask, scale, return_probs)
        if kind == "log2_lse":
            res = (res[0], res[1] / math.log(2.0)) + tuple(res[2:])
        return res
    return attend


@pytest.mark.parametrize("kind", ["sibling_leak", "drop_self", "descendant_mask", "rope_unscaled",
                                  "drop_rope", "missing_scale", "latent_rope_row_skew",
                                  "log2_lse"])
def test_brute_force_catches_planted_mistakes(kind, monkeypatch):
    par = np.array([-1, 0, 0, 1, 1, 2], np.int32)
    inp = _tiny_inputs(22, [par], [4], heads=2, scale=0.4)
    bo, bl = _brute_force(inp)
    if kind in ("sibling_leak", "drop_self", "descendant_mask"):
        monkeypatch.setattr(O, "visibility_mask", _wrong_visibility(kind))
    else:
        monkeypatch.setattr(O, "attend_request", _wrong_attend(kind))
    out, lse = _oracle(inp)
    err = max(np.abs(out - bo).max(), np.abs(lse - bl).max())
    assert err > 1e-3, f"planted mistake {kind} went unnoticed"


# ------------------------------------------------------------------ row-selection helper
# verify_attn_rows is the checker used on selected rows of large batches.  It is pinned
# against the per-row brute force (independent code) on tiny inputs, and against the
# packed-batch oracle on selections that exercise its offsets: the last request, unsorted
# and repeated nodes and heads, a request after one with an empty prefix.
@pytest.mark.parametrize("seed", range(4))
def test_rows_helper_matches_brute_force(seed):
    rng = np.random.default_rng(500 + seed)
    parents = [synth.random_tree(rng, int(rng.integers(1, 8))) for _ in range(3)]
    prefix = [int(rng.integers(0, 12)), 0, int(rng.integers(1, 12))]
    inp = _tiny_inputs(600 + seed, parents, prefix, heads=3)
    bo, bl = _brute_force(inp)
    qo = inp.q_offsets()
    for b in range(inp.batch):
        t = int(inp.q_len[b])
        nodes = [int(x) for x in rng.integers(0, t, size=3)] + [t - 1, 0]
        heads = [2, 0, 2, 1]
        ro, rl = O.verify_attn_rows(inp, b, nodes, heads)
        rows = qo[b] + np.asarray(nodes)
        np.testing.assert_allclose(ro, bo[rows][:, heads], rtol=0, atol=1e-12)
        np.testing.assert_allclose(rl, bl[rows][:, heads], rtol=0, atol=1e-12)


def test_rows_helper_matches_packed_oracle():
    rng = np.random.default_rng(61)
    parents = [synth.random_tree(rng, n) for n in (5, 33, 1, 17)]
    inp = _tiny_inputs(62, parents, [40, 0, 7, 129], heads=8, dl=32, dr=8)
    fo, fl = _oracle(inp)
    qo = inp.q_offsets()
    for b, nodes, heads in ((3, [16, 0, 4, 4], [7, 0]), (1, [32, 31, 0], [5]),
                            (2, [0], list(range(8))), (0, [4, 2], [3, 6, 1])):
        ro, rl = O.verify_attn_rows(inp, b, nodes, heads)
        rows = qo[b] + np.asarray(nodes)
        np.testing.assert_allclose(ro, fo[rows][:, heads], rtol=0, atol=1e-13)
        np.testing.assert_allclose(rl, fl[rows][:, heads], rtol=0, atol=1e-13)
