"""Checks of the seeded input generator (trees, bf16 rounding, workload shapes)."""
import itertools

import numpy as np
import pytest
import torch

from tree_verify_mla_attn_amd import synth


def _node_paths(parent, rank):
    """Rank sequence (root excluded) of every drafted node."""
    paths = []
    for i in range(1, len(parent)):
        seq = []
        n = i
        while n > 0:
            seq.append(int(rank[n]))
            n = int(parent[n])
        paths.append(tuple(reversed(seq)))
    return paths


@pytest.mark.parametrize("depth,k,budget,seed", [(3, 3, 5, 0), (3, 3, 12, 1), (4, 2, 9, 2),
                                                 (2, 4, 30, 3), (3, 3, 39, 4), (3, 3, 50, 5),
                                                 (1, 1, 4, 6)])
def test_best_first_selects_top_paths(depth, k, budget, seed):
    rng = np.random.default_rng(seed)
    table = synth.logprob_table(rng, k, depth=depth)
    parent, dep, rank, cum = synth.best_first_tree(table, budget)
    # brute force: every rank sequence up to the table depth, scored by its sum
    scored = []
    for d in range(1, depth + 1):
        for seq in itertools.product(range(k), repeat=d):
            scored.append((sum(table[i, r] for i, r in enumerate(seq)), seq))
    scored.sort(key=lambda x: -x[0])
    want = {seq for _, seq in scored[:budget]}
    got = _node_paths(parent, rank)
    assert len(got) == min(budget, len(scored))
    assert set(got) == want
    # pop order is best-first: cumulative log-prob never increases
    assert np.all(np.diff(cum[1:]) <= 1e-12)
    for i, seq in enumerate(got, start=1):
        assert abs(cum[i] - sum(table[d, r] for d, r in enumerate(seq))) < 1e-12
        assert dep[i] == len(seq)


def test_tree_structure_and_budgets():
    for cfg in synth.CONFIGS:
        _, prefix, parents = synth.config_trees(cfg)
        c = synth.CONFIGS[cfg]
        assert len(parents) == c["batch"] and len(prefix) == c["batch"]
        for par in parents:
            assert par[0] == -1
            assert np.all(par[1:] >= 0) and np.all(par[1:] < np.arange(1, len(par)))
            assert len(par) == c["budget"] + 1 <= synth.MAX_QLEN
            assert synth.tree_depths(par).max() <= synth.MAX_DEPTH
    _, prefix, parents = synth.config_trees(4)
    assert prefix.min() >= 1024 and prefix.max() <= 8192
    # wide half (top-8) has more children at the root than the deep half (top-2)
    wide = [int((p == 0).sum()) for p in parents[:32]]
    deep = [int((p == 0).sum()) for p in parents[32:]]
    assert max(deep) <= 2 and max(wide) > 2
    _, _, parents3 = synth.config_trees(3)
    assert max(synth.tree_depths(p).max() for p in parents3) >= 12


def test_underfull_chain_tree():
    table = np.log(np.ones((synth.MAX_DEPTH, 1)))
    parent = synth.best_first_tree(table, 64)[0]
    np.testing.assert_array_equal(parent, synth.chain_tree(16))


def test_generator_is_deterministic():
    a = synth.config_inputs(1)
    b = synth.config_inputs(1)
    for f in ("q_lat", "q_rope", "kv_lat", "k_rope", "tree_parent", "prefix_len", "q_len"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))


def test_config1_shapes():
    inp = synth.config_inputs(1)
    assert inp.q_lat.shape == (9, 64, 512) and inp.q_rope.shape == (9, 64, 64)
    assert inp.kv_lat.shape == (265, 512) and inp.k_rope.shape == (265, 64)
    assert inp.q_lat.dtype == np.float32 and inp.dtype == "fp32"
    assert abs(inp.scale - 1 / np.sqrt(192)) < 1e-15


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0, np.inf, -np.inf, 3.4e38, 1e-40, -1e-39], np.float32)])
    # exact ties: mantissa low half == 0x8000, both parities of the kept bit
    ties = (np.arange(1000, dtype=np.uint32) << np.uint32(17)) | np.uint32(0x3F808000)
    ties2 = (np.arange(1000, dtype=np.uint32) << np.uint32(17)) | np.uint32(0x3F818000)
    x = np.concatenate([x, ties.view(np.float32), ties2.view(np.float32)])
    ours = synth.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    back = synth.bf16_to_f32(ours)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_bf16_inputs_hold_bf16_values():
    rng = np.random.default_rng(1)
    inp = synth.make_inputs(rng, num_heads=4, prefix_lens=[7], parents=[synth.chain_tree(3)],
                            dtype="bf16")
    for f in ("q_lat", "q_rope", "kv_lat", "k_rope"):
        a = getattr(inp, f)
        np.testing.assert_array_equal(synth.round_to_bf16(a), a)


def test_algorithmic_counts():
    rng = np.random.default_rng(2)
    par = np.array([-1, 0, 1, 0], np.int32)      # depths 0, 1, 2, 1
    inp = synth.make_inputs(rng, num_heads=2, prefix_lens=[10], parents=[par], dtype="bf16")
    pairs = (10 + 1) + (10 + 2) + (10 + 3) + (10 + 2)
    assert inp.algorithmic_flops() == pairs * 2 * 2 * (576 + 512)
    rows = 4 * 2
    assert inp.algorithmic_bytes() == rows * 576 * 2 + 14 * 576 * 2 + rows * 512 * 4 + rows * 4
