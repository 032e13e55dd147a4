"""GPU parity of the temperature draw (kdtree_sample_tokens) against the CPU oracle
(oracle/sample_f32.py), and of the temperature accept (draw, then the greedy walk).

Bar: every drawn token equals the oracle's, at T = 0 (an argmax with the lowest index on
ties) and at T > 0: both sides evaluate the keys with the same float32 operations, the
base-2 logarithm included (a fixed sequence of rounded operations), so the perturbed values
and their argmax agree bit for bit.  A frequency test on the GPU alone checks the draw
against softmax(logits / T).
"""
import numpy as np
import pytest
import torch

from oracle import ddtree_f32 as D
from oracle import sample_f32 as S
from tree_verify_mla_attn_amd import binding as B
from tree_verify_mla_attn_amd import synth

pytestmark = pytest.mark.gpu

VOCAB = synth.VOCAB


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.load_library()
    return torch.device("cuda:0")


def _bf16_exact(x):
    return synth.round_to_bf16(np.asarray(x, np.float32))


def gpu_draw(logits_np, temperature, seed, offset, dev, dtype="fp32", stride=None):
    rows, vocab = logits_np.shape
    stride = stride or vocab
    host = np.full((rows, stride), -7.0, np.float32)
    host[:, :vocab] = logits_np
    if dtype == "bf16":
        t = torch.from_numpy(synth.bf16_bits(host).view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        t = torch.from_numpy(host).to(dev)
    tok = B.sample_tokens(t, temperature, seed, offset, vocab=vocab)
    torch.cuda.synchronize(dev)
    return tok.cpu().numpy()


def compare(name, logits, temperature, seed, offset, got):
    want = S.sample_tokens(logits, temperature, seed, offset)
    bad = np.nonzero(got != want)[0]
    print(f"[{name}] T={temperature} rows={len(got)} differing={len(bad)}", flush=True)
    np.testing.assert_array_equal(got, want, err_msg=f"{name}: rows {bad[:8]}")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_greedy_exact_with_ties(dev, dtype):
    rng = np.random.default_rng(200)
    logits = rng.normal(0, 2, size=(8, VOCAB)).astype(np.float32)
    if dtype == "bf16":
        logits = _bf16_exact(logits)
    top = logits.max(axis=1)
    for r, cols in enumerate(([5, 99999], [163839, 0], [77, 78, 79], [12345])):
        logits[r, cols] = top[r] + 1.0  # equal maxima: the lowest index wins
    print(f"case greedy/{dtype}", flush=True)
    got = gpu_draw(logits, 0.0, 1, 2, dev, dtype)
    compare(f"greedy/{dtype}", logits, 0.0, 1, 2, got)
    assert got[0] == 5 and got[1] == 0 and got[2] == 77 and got[3] == 12345


@pytest.mark.parametrize("temperature", [0.7, 1.0, 1.5])
def test_draw_matches_oracle_fp32(dev, temperature):
    rng = np.random.default_rng(int(temperature * 10) + 201)
    logits = rng.normal(0, 3, size=(16, VOCAB)).astype(np.float32)
    print(f"case draw/fp32 T={temperature}", flush=True)
    got = gpu_draw(logits, temperature, 1234, 7, dev)
    compare("draw/fp32", logits, temperature, 1234, 7, got)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_draw_peaked_logits(dev, dtype):
    """LM-like rows: a flat bulk and a few far higher candidates, so most blocks of 8
    entries cannot hold the winner and the kernel skips their generator work; the draws
    must still equal the oracle's (which evaluates every entry)."""
    rng = np.random.default_rng(215)
    logits = rng.normal(0, 2, size=(16, VOCAB)).astype(np.float32)
    for r in range(16):
        top = rng.choice(VOCAB, size=12, replace=False)
        logits[r, top] = (18.0 if r % 2 else 24.0) + rng.normal(0, 1.5, size=12).astype(np.float32)
    if dtype == "bf16":
        logits = _bf16_exact(logits)
    print(f"case peaked/{dtype}", flush=True)
    for temperature in (0.6, 1.0):
        got = gpu_draw(logits, temperature, 4321, 9, dev, dtype)
        compare(f"peaked/{dtype}", logits, temperature, 4321, 9, got)


def test_draw_matches_oracle_bf16(dev):
    rng = np.random.default_rng(210)
    logits = _bf16_exact(rng.normal(0, 3, size=(16, VOCAB)))
    print("case draw/bf16", flush=True)
    got = gpu_draw(logits, 0.9, 99, 3, dev, "bf16")
    compare("draw/bf16", logits, 0.9, 99, 3, got)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_unaligned_stride_and_masks(dev, dtype):
    rng = np.random.default_rng(220)
    logits = rng.normal(0, 1, size=(40, 1001)).astype(np.float32)
    if dtype == "bf16":
        logits = _bf16_exact(logits)
    logits[3] = -np.inf                      # nothing to draw
    logits[4, :1000] = -np.inf               # only the last entry
    logits[5, ::2] = -np.inf                 # only odd entries
    print(f"case stride/{dtype}", flush=True)
    for temperature in (0.0, 1.3):
        got = gpu_draw(logits, temperature, 5, 6, dev, dtype, stride=1003)
        compare(f"stride/{dtype}", logits, temperature, 5, 6, got)
        assert got[3] == -1 and got[4] == 1000 and got[5] % 2 == 1


def test_frequencies_on_the_gpu(dev):
    logits = np.array([1.0, 0.2, -0.5, 2.0, -3.0, 0.0], np.float32)
    rows, temperature = 20000, 0.8
    print("case frequencies", flush=True)
    got = gpu_draw(np.tile(logits, (rows, 1)), temperature, 31, 4, dev)
    counts = np.bincount(got, minlength=6).astype(np.float64)
    p = np.exp(logits.astype(np.float64) / temperature)
    p /= p.sum()
    chi2 = float(((counts - rows * p) ** 2 / (rows * p)).sum())
    print(f"[frequencies] chi2={chi2:.2f} counts={counts.tolist()}", flush=True)
    assert chi2 < 30.0


def test_temperature_accept_chain(dev):
    """Build on the device, draw the target's token at every node, walk: the accepted
    tokens equal the oracle's chain (or, at a near-tie draw, the oracle walk over the
    device's draws)."""
    rng = np.random.default_rng(230)
    batch, budget = 8, 32
    logp, ids, root = synth.draft_tables(rng, batch, [8, 2] * 4, depth=15, vocab=4096)
    t = B.build_ddtree(torch.from_numpy(logp).to(dev), torch.from_numpy(ids).to(dev),
                       torch.from_numpy(root).to(dev), budget, with_score=False)
    torch.cuda.synchronize(dev)
    tree = {k: v.cpu().numpy() for k, v in t.items()}
    width = budget + 1
    logits = rng.normal(0, 1, size=(batch * width, 4096)).astype(np.float32)
    for b in range(batch):  # the target leans towards the first child of each node
        n = int(tree["q_len"][b])
        for i in range(n):
            c = int(tree["first_child"][b, i])
            if c > 0:
                logits[b * width + i, tree["token"][b, c]] += 10.0
    print("case temperature chain", flush=True)
    d_logits = torch.from_numpy(logits).to(dev)
    drawn = B.sample_tokens(d_logits, 0.8, 77, 1)
    al, at, an = B.tree_accept(t["token"], t["first_child"], t["next_sibling"], t["q_len"],
                               drawn.view(batch, width), 16)
    torch.cuda.synchronize(dev)
    drawn_np = drawn.cpu().numpy()
    compare("chain draw", logits, 0.8, 77, 1, drawn_np)
    lens = al.cpu().numpy()
    for b in range(batch):
        nd, tk = D.tree_accept(tree["token"][b], tree["first_child"][b], tree["next_sibling"][b],
                               drawn_np[b * width:(b + 1) * width])
        assert lens[b] == len(tk)
        np.testing.assert_array_equal(at.cpu().numpy()[b, :len(tk)], tk)
        np.testing.assert_array_equal(an.cpu().numpy()[b, :len(nd)], nd)
    print(f"[chain] accept lengths {lens.tolist()}", flush=True)
    assert lens.max() > 1
