"""Seeded random shapes for verify attention, compared with the float64 oracle element by
element: head counts the fixed cases do not use (1, 3, 7, 96, 160), random trees of 1..65
nodes, prefixes 0..3000, split counts 1..9, both input types.  Same bars as
test_gpu_parity.py."""
import numpy as np
import pytest
import torch

from oracle import verify_attn_inputs
from tree_verify_mla_attn_amd import binding as B
from tree_verify_mla_attn_amd import synth

pytestmark = pytest.mark.gpu

HEADS = (1, 3, 7, 16, 96, 160)


def _case(seed):
    rng = np.random.default_rng(5000 + seed)
    heads = int(HEADS[seed % len(HEADS)])
    dtype = "bf16" if seed % 2 else "fp32"
    batch = int(rng.integers(1, 5))
    parents, prefix = [], []
    for _ in range(batch):
        q = int(rng.choice([1, 2, 9, 33, 64, 65, int(rng.integers(1, 66))]))
        parents.append(synth.random_tree(rng, q))
        prefix.append(int(rng.choice([0, 1, 31, 32, 33, int(rng.integers(0, 3001))])))
    splits = int(rng.integers(1, 10))
    inp = synth.make_inputs(rng, num_heads=heads, prefix_lens=prefix, parents=parents,
                            dtype=dtype)
    return inp, splits


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.load_library()
    return torch.device("cuda:0")


@pytest.mark.parametrize("seed", range(24))
def test_random_shapes(dev, seed):
    inp, splits = _case(seed)
    print(f"case random/{seed}: dtype={inp.dtype} heads={inp.num_heads} q_len={inp.q_len.tolist()} "
          f"prefix={inp.prefix_len.tolist()} splits={splits}", flush=True)
    d = synth.device_tensors(inp, dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    out, lse = B.verify_attn(d["q_lat"], d["q_rope"], d["kv_lat"], d["k_rope"], d["prefix_len"],
                             d["tree_parent"], d["q_len"], inp.scale, num_splits=splits,
                             max_q_len=65, status=status)
    torch.cuda.synchronize(dev)
    assert int(status.item()) == 0
    r_out, r_lse = verify_attn_inputs(inp)
    g_out, g_lse = out.double().cpu().numpy(), lse.double().cpu().numpy()
    e_out, e_lse = np.abs(g_out - r_out), np.abs(g_lse - r_lse)
    if inp.dtype == "fp32":
        ratio = max(e_out.max(), e_lse.max()) / 1e-5
    else:
        ratio = max((e_out / (1e-3 + 2e-3 * np.abs(r_out))).max(),
                    (e_lse / (1e-3 + 2e-3 * np.abs(r_lse))).max())
    print(f"[random/{seed}] worst error/bound={ratio:.3f}", flush=True)
    assert np.isfinite(g_out).all() and np.isfinite(g_lse).all()
    assert ratio <= 1.0
