"""The allocation-free entry point kdtree_verify_attn_noalloc against kdtree_verify_attn.

Both run the same kernels, so the outputs must agree bit for bit; the no-alloc call
takes its scratch from the library's static device array instead of a workspace.  Two
calls in a row, the second on a smaller batch (the array keeps the first call's
contents), for bf16 inputs (pre-pass tiles, last-round cut pieces) and split launches
(partials), and fp32.
"""
import numpy as np
import pytest
import torch

from tree_verify_mla_attn_amd import binding as B
from tree_verify_mla_attn_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.load_library()
    return torch.device("cuda:0")


def _inputs(seed, n_req, heads, dtype):
    rng = np.random.default_rng(seed)
    parents = [synth.random_tree(rng, int(rng.integers(1, 66))) for _ in range(n_req)]
    prefix = rng.integers(0, 1500, size=n_req)
    return synth.make_inputs(rng, num_heads=heads, prefix_lens=prefix, parents=parents,
                             dtype=dtype)


def _noalloc(inp, d, dev, splits, ratio):
    out = torch.full((inp.total_q, inp.num_heads, 512), float("nan"), dtype=torch.float32,
                     device=dev)
    lse = torch.full((inp.total_q, inp.num_heads), float("nan"), dtype=torch.float32,
                     device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    dt = B.KDTREE_DTYPE_BF16 if inp.dtype == "bf16" else B.KDTREE_DTYPE_FP32
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = B.kdtree_verify_attn_noalloc(
        d["q_lat"].data_ptr(), d["q_rope"].data_ptr(), d["kv_lat"].data_ptr(),
        d["k_rope"].data_ptr(), d["prefix_len"].data_ptr(), d["tree_parent"].data_ptr(),
        d["q_len"].data_ptr(), float(inp.scale), out.data_ptr(), lse.data_ptr(), stream,
        inp.batch, inp.num_heads, inp.max_q_len, inp.total_q, inp.total_kv, dt, splits,
        status.data_ptr(), split_ratio=ratio)
    assert rc == 0, B.ERRORS.get(rc, rc)
    return out, lse, status


@pytest.mark.parametrize("dtype,splits,ratio", [("bf16", 1, 1.0), ("bf16", 3, 0.6),
                                                ("fp32", 1, 1.0), ("fp32", 4, 1.0)])
def test_noalloc_matches_workspace_call(dev, dtype, splits, ratio):
    for seed, n_req in ((11, 9), (12, 3)):  # the second call is smaller
        inp = _inputs(seed, n_req, 64 if dtype == "bf16" else 16, dtype)
        need = B.kdtree_verify_attn_workspace_bytes(inp.total_q, inp.total_kv, inp.batch,
                                                    inp.num_heads, splits,
                                                    B.KDTREE_DTYPE_BF16 if dtype == "bf16"
                                                    else B.KDTREE_DTYPE_FP32)
        assert need <= B.KDTREE_NOALLOC_SCRATCH_BYTES
        d = synth.device_tensors(inp, dev)
        print(f"case noalloc/{dtype} splits={splits} requests={n_req} need={need}", flush=True)
        ref_o, ref_l = B.verify_attn(d["q_lat"], d["q_rope"], d["kv_lat"], d["k_rope"],
                                     d["prefix_len"], d["tree_parent"], d["q_len"], inp.scale,
                                     num_splits=splits, max_q_len=inp.max_q_len,
                                     split_ratio=ratio)
        out, lse, status = _noalloc(inp, d, dev, splits, ratio)
        torch.cuda.synchronize(dev)
        assert int(status.item()) == 0
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"{dtype} {splits} {n_req}"
