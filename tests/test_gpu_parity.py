"""GPU parity of the HIP tree-verify attention against the float64 oracle.

Bars: fp32 inputs -> max |gpu - oracle| <= 1e-5 on out_lat and out_lse; bf16 inputs ->
|gpu - oracle| <= 1e-3 + 2e-3 |oracle| elementwise, oracle fed the same bf16 values.
Every case compares every element, the large workloads (batch 8 / 64 / 4 at H=64) too, in
the launch configuration the benchmark times.
"""
import numpy as np
import pytest
import torch

from oracle import verify_attn_inputs
from tree_verify_mla_attn_amd import binding as B
from tree_verify_mla_attn_amd import synth

pytestmark = pytest.mark.gpu

FP32_ATOL = 1e-5
BF16_ATOL, BF16_RTOL = 1e-3, 2e-3


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.load_library()
    return torch.device("cuda:0")


def run(inp, dev, num_splits=1, max_q_len=None, split_ratio=1.0):
    d = synth.device_tensors(inp, dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    out, lse = B.verify_attn(d["q_lat"], d["q_rope"], d["kv_lat"], d["k_rope"], d["prefix_len"],
                             d["tree_parent"], d["q_len"], inp.scale, num_splits=num_splits,
                             max_q_len=max_q_len or inp.max_q_len, status=status,
                             split_ratio=split_ratio)
    torch.cuda.synchronize(dev)
    return out, lse, int(status.item())


def check(name, inp, g_out, g_lse, r_out, r_lse):
    g_out = np.asarray(g_out, np.float64)
    g_lse = np.asarray(g_lse, np.float64)
    e_out = np.abs(g_out - r_out)
    e_lse = np.abs(g_lse - r_lse)
    if inp.dtype == "fp32":
        ratio = max(e_out.max(), e_lse.max()) / FP32_ATOL
    else:
        ratio = max((e_out / (BF16_ATOL + BF16_RTOL * np.abs(r_out))).max(),
                    (e_lse / (BF16_ATOL + BF16_RTOL * np.abs(r_lse))).max())
    print(f"[{name}] max|d out|={e_out.max():.3e} max|d lse|={e_lse.max():.3e} "
          f"worst error/bound={ratio:.3f}", flush=True)
    assert np.isfinite(g_out).all() and np.isfinite(g_lse).all()
    if inp.dtype == "fp32":
        assert e_out.max() <= FP32_ATOL, name
        assert e_lse.max() <= FP32_ATOL, name
    else:
        bad = e_out > BF16_ATOL + BF16_RTOL * np.abs(r_out)
        assert not bad.any(), f"{name}: {int(bad.sum())} out_lat elements outside tolerance"
        assert not (e_lse > BF16_ATOL + BF16_RTOL * np.abs(r_lse)).any(), name


def full_check(name, inp, dev, num_splits=1, split_ratio=1.0):
    print(f"case {name} splits={num_splits} ratio={split_ratio}", flush=True)
    out, lse, st = run(inp, dev, num_splits, split_ratio=split_ratio)
    assert st == 0, B.decode_status(st)
    r_out, r_lse = verify_attn_inputs(inp)
    check(name, inp, out.double().cpu().numpy(), lse.double().cpu().numpy(), r_out, r_lse)
    return out, lse


# ------------------------------------------------------------------ small / edge cases
def _mk(seed, parents, prefix, heads, dtype, scale=None):
    rng = np.random.default_rng(seed)
    return synth.make_inputs(rng, num_heads=heads, prefix_lens=prefix, parents=parents,
                             dtype=dtype, scale=scale)


def _ramp(seed, dtype, slope):
    """Scores that move steadily along each request's key stream: every latent key row is
    c_j + 0.25 N(0, 1) with c_j running linearly from -8 slope to 8 slope over the request's
    keys, and every query row 0.5 + 0.25 N(0, 1), so that q . k_j ~ 256 c_j.  At the
    default scale the running maximum then moves by about 14 log2 units per 32-key tile
    (slope 1: above the rescale threshold on every tile) or the first tile dominates and
    the later probabilities underflow (slope -1)."""
    rng = np.random.default_rng(seed)
    parents = [synth.random_tree(np.random.default_rng(seed + 1), 33), synth.chain_tree(9)]
    inp = synth.make_inputs(rng, num_heads=16, prefix_lens=[1000, 300], parents=parents,
                            dtype=dtype)
    fix = synth.round_to_bf16 if dtype == "bf16" else (lambda x: x.astype(np.float32))
    kv_off, q_off = inp.kv_offsets(), inp.q_offsets()
    for b in range(inp.batch):
        n = int(inp.prefix_len[b] + inp.q_len[b])
        c = np.linspace(-8.0 * slope, 8.0 * slope, n, dtype=np.float32)[:, None]
        rows = slice(int(kv_off[b]), int(kv_off[b]) + n)
        inp.kv_lat[rows] = fix(c + 0.25 * rng.standard_normal((n, 512), dtype=np.float32))
        qs = slice(int(q_off[b]), int(q_off[b]) + int(inp.q_len[b]))
        inp.q_lat[qs] = fix(0.5 + 0.25 * rng.standard_normal(inp.q_lat[qs].shape,
                                                             dtype=np.float32))
    return inp


EDGE = {
    "chain9_p37_h64": lambda dt: _mk(1, [synth.chain_tree(9)], [37], 64, dt),
    "star17_p0_h16": lambda dt: _mk(2, [synth.star_tree(17)], [0], 16, dt),
    "deep15_p100_h8": lambda dt: _mk(3, [synth.chain_tree(16)], [100], 8, dt),
    "root_only_p5_h64": lambda dt: _mk(4, [np.array([-1], np.int32)], [5], 64, dt),
    "qlen65_p300_h64": lambda dt: _mk(5, [synth.random_tree(np.random.default_rng(9), 65)], [300],
                                      64, dt),
    "ragged_batch5_h64": lambda dt: _mk(
        6, [synth.random_tree(np.random.default_rng(10 + i), n) for i, n in
            enumerate((1, 9, 33, 65, 17))], [0, 31, 64, 257, 1000], 64, dt),
    "tile_edges_h16": lambda dt: _mk(
        7, [synth.random_tree(np.random.default_rng(20 + i), 33) for i in range(4)],
        [31, 32, 33, 64], 16, dt),
    "zero_scale": lambda dt: _mk(8, [synth.random_tree(np.random.default_rng(30), 12)], [40], 64,
                                 dt, scale=0.0),
    "negative_scale": lambda dt: _mk(9, [synth.random_tree(np.random.default_rng(31), 12)], [40],
                                     64, dt, scale=-0.08),
}

# Softmax stress: scores of magnitude 50-160, where the running maximum moves on every
# tile (rising), or the first tile dominates and later probabilities underflow (falling).
# bf16 only: the fp32 bound is absolute (1e-5), below what float32 rounding of such
# scores allows; the bf16 bound scales with the values.
STRESS = {
    "large_scale": lambda: _mk(10, [synth.random_tree(np.random.default_rng(32), 33)], [700], 64,
                               "bf16", scale=1.0),
    "rising_scores": lambda: _ramp(11, "bf16", 1.0),
    "falling_scores": lambda: _ramp(13, "bf16", -1.0),
}


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("case", list(EDGE))
def test_edge_cases(dev, case, dtype):
    full_check(f"{case}/{dtype}", EDGE[case](dtype), dev)


@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("case", list(STRESS))
def test_softmax_stress(dev, case, splits):
    full_check(f"{case}/bf16", STRESS[case](), dev, num_splits=splits)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("splits,ratio", [(2, 1.0), (3, 1.0), (16, 1.0), (2, 0.45), (3, 0.5),
                                          (16, 0.7), (5, 0.05)])
def test_split_kv(dev, splits, ratio, dtype):
    """Equal splits, and geometric ones (ratio < 1: largest first, boundaries rounded up
    to whole tiles, so several splits of a short prefix may be empty)."""
    inp = EDGE["ragged_batch5_h64"](dtype)
    full_check(f"ragged_batch5/{dtype}", inp, dev, num_splits=splits, split_ratio=ratio)
    inp = EDGE["deep15_p100_h8"](dtype)
    full_check(f"deep15/{dtype}", inp, dev, num_splits=splits, split_ratio=ratio)


def test_bf16_best_first_trees_several_tiles(dev):
    rng = np.random.default_rng(40)
    parents = [synth.best_first_tree(synth.logprob_table(rng, k), 32)[0] for k in (8, 2, 4)]
    inp = synth.make_inputs(rng, num_heads=64, prefix_lens=[513, 200, 1030], parents=parents,
                            dtype="bf16")
    full_check("bestfirst3", inp, dev)
    full_check("bestfirst3", inp, dev, num_splits=4)


# ------------------------------------------------------------------ workloads
@pytest.mark.parametrize("cfg", [1, 2])
def test_small_workloads_full(dev, cfg):
    """Every element, unsplit and in the benchmark's launch configuration."""
    inp = synth.config_inputs(cfg)
    full_check(f"workload{cfg}", inp, dev)
    full_check(f"workload{cfg}", inp, dev, num_splits=inp.num_splits,
               split_ratio=inp.split_ratio)


@pytest.mark.parametrize("cfg", [3, 4, 5])
def test_large_workloads_full(dev, cfg):
    """Every element of the batch-8 / batch-64 / batch-4 workloads, in the launch
    configuration the benchmark times (workload 3 and 4: one split, workload 3 through the
    last-round cut; workload 5: 16 geometric splits at ratio 0.85), against the full
    float64 oracle on the same bf16 values."""
    inp = synth.config_inputs(cfg)
    full_check(f"workload{cfg}", inp, dev, num_splits=inp.num_splits,
               split_ratio=inp.split_ratio)


def test_workload4_metamorphic(dev):
    """Full-size checks that sampling cannot miss, on the batch-64 workload:
    * one tail key row per request (the last tree node's, a leaf) is replaced by new
      values; every row of a node that does not see that key is bit-identical, and the
      rows that do see it change;
    * reversing the head order of the queries reverses the heads of the outputs, bit for
      bit (every row is computed on its own)."""
    inp = synth.config_inputs(4)
    out, lse, st = run(inp, dev)
    assert st == 0
    out, lse = out.cpu(), lse.cpu()
    rng = np.random.default_rng(4004)
    kv_lat, k_rope = inp.kv_lat.copy(), inp.k_rope.copy()
    qo, ko = inp.q_offsets(), inp.kv_offsets()
    sees = np.zeros(inp.total_q, bool)
    for b in range(inp.batch):
        par = inp.parents_of(b)
        j = len(par) - 1
        row = ko[b] + int(inp.prefix_len[b]) + j
        kv_lat[row] = synth.round_to_bf16(rng.standard_normal(512).astype(np.float32) * 3)
        k_rope[row] = synth.round_to_bf16(rng.standard_normal(64).astype(np.float32) * 3)
        for i in range(len(par)):
            x = i
            while x != -1 and x != j:
                x = int(par[x])
            sees[qo[b] + i] = x == j
    pert = synth.VerifyInputs(**{**inp.__dict__, "kv_lat": kv_lat, "k_rope": k_rope})
    out2, lse2, st = run(pert, dev)
    assert st == 0
    out2, lse2 = out2.cpu(), lse2.cpu()
    keep = torch.from_numpy(~sees)
    print(f"rows seeing a perturbed key: {int(sees.sum())} of {inp.total_q}", flush=True)
    assert torch.equal(out2[keep], out[keep]) and torch.equal(lse2[keep], lse[keep])
    # rows that see the new key move (a row whose old and new scores are both tiny could
    # in principle stay the same in fp32, so this asks for nearly all of them)
    seen = torch.from_numpy(sees)
    moved = (out2[seen] != out[seen]).any(dim=2)
    assert moved.float().mean().item() > 0.99, moved.float().mean().item()
    flip = synth.VerifyInputs(**{**inp.__dict__, "q_lat": inp.q_lat[:, ::-1].copy(),
                                 "q_rope": inp.q_rope[:, ::-1].copy()})
    out3, lse3, st = run(flip, dev)
    assert st == 0
    assert torch.equal(out3.cpu(), out.flip(1)) and torch.equal(lse3.cpu(), lse.flip(1))


def test_one_split_without_cut_several_rounds(dev):
    """The uncut one-split path with more than two whole rounds of row tiles per XCD (24
    requests x 33 row tiles at q_len 65 and 64 heads), every element."""
    rng = np.random.default_rng(90)
    parents = [synth.random_tree(rng, 65) for _ in range(24)]
    prefix = rng.integers(0, 200, size=24)
    inp = synth.make_inputs(rng, num_heads=64, prefix_lens=prefix, parents=parents,
                            dtype="bf16")
    full_check("uncut24", inp, dev)


@pytest.mark.parametrize("case", [c for c in EDGE])
def test_edge_cases_bf16_cut_off(dev, case, monkeypatch):
    """The bf16 edge cases again with the last-round cut switched off, so that the uncut
    one-split path is covered on each of them (most small launches are cut)."""
    monkeypatch.setenv("KDTREE_DISABLE_CUT", "1")
    full_check(f"{case}/bf16/nocut", EDGE[case]("bf16"), dev)


# ------------------------------------------------------------------ robustness
def test_bf16_range_status(dev):
    """A bf16 latent value outside fp16's range (|x| >= 65504, or not finite) sets the
    range bit, in kv_lat (seen by the pre-pass) and in q_lat (seen by the Q load); the
    largest bf16 value below 65504 does not."""
    base = EDGE["ragged_batch5_h64"]("bf16")
    cases = []
    kv = base.kv_lat.copy()
    kv[40, 17] = 65280.0          # largest bf16 below 65504: in range
    cases.append(("in_range", dict(kv_lat=kv), 0))
    kv = base.kv_lat.copy()
    kv[40, 17] = 1.0e5
    cases.append(("kv_big", dict(kv_lat=kv), 32))
    kv = base.kv_lat.copy()
    kv[-1, 3] = -np.inf
    cases.append(("kv_inf", dict(kv_lat=kv), 32))
    q = base.q_lat.copy()
    q[7, 5, 100] = -7.0e4
    cases.append(("q_big", dict(q_lat=q), 32))
    for name, change, bit in cases:
        inp = synth.VerifyInputs(**{**base.__dict__, **change})
        print(f"case range/{name}", flush=True)
        _, _, st = run(inp, dev)
        print(f"range/{name}: status {st} {B.decode_status(st)}", flush=True)
        assert (st & 32) == bit, name


@pytest.mark.parametrize("splits", [1, 4])
def test_requests_before_a_malformed_one_are_computed(dev, splits):
    """q_len[2] = 0: requests 2.. are skipped and flagged, requests 0 and 1 are computed
    (their fp16 tiles converted by the pre-pass) and match the oracle."""
    base = EDGE["ragged_batch5_h64"]("bf16")
    bad_q = base.q_len.copy()
    bad_q[2] = 0
    inp = synth.VerifyInputs(**{**base.__dict__, "q_len": bad_q})
    d = synth.device_tensors(inp, dev)
    h = inp.num_heads
    n01 = int(base.q_len[0] + base.q_len[1])
    rows = base.total_q  # the packed rows the caller allocated (q_len no longer sums to it)
    out = torch.full((rows, h, 512), 7.25, dtype=torch.float32, device=dev)
    lse = torch.full((rows, h), 7.25, dtype=torch.float32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    print(f"case malformed_q2 splits={splits}", flush=True)
    B.verify_attn(d["q_lat"], d["q_rope"], d["kv_lat"], d["k_rope"], d["prefix_len"],
                  d["tree_parent"], d["q_len"], inp.scale, out_lat=out, out_lse=lse,
                  num_splits=splits, max_q_len=65, status=status)
    torch.cuda.synchronize(dev)
    assert int(status.item()) & 1
    assert (out[n01:] == 7.25).all() and (lse[n01:] == 7.25).all()
    first = synth.VerifyInputs(**{**base.__dict__, "q_len": base.q_len[:2].copy(),
                                  "prefix_len": base.prefix_len[:2].copy(),
                                  "tree_parent": base.tree_parent[:n01].copy(),
                                  "q_lat": base.q_lat[:n01], "q_rope": base.q_rope[:n01]})
    r_out, r_lse = verify_attn_inputs(first)
    check(f"malformed_q2/{splits}", first, out[:n01].double().cpu().numpy(),
          lse[:n01].double().cpu().numpy(), r_out, r_lse)


def test_phase_calls_need_the_callers_workspace(dev):
    inp = EDGE["chain9_p37_h64"]("bf16")
    d = synth.device_tensors(inp, dev)
    args = (d["q_lat"], d["q_rope"], d["kv_lat"], d["k_rope"], d["prefix_len"], d["tree_parent"],
            d["q_len"], inp.scale)
    for phase in ("prepare", "attend"):
        with pytest.raises(ValueError, match="workspace"):
            B.verify_attn(*args, max_q_len=inp.max_q_len, phase=phase)


def test_deterministic_and_guard_bands(dev):
    inp = EDGE["ragged_batch5_h64"]("bf16")
    d = synth.device_tensors(inp, dev)
    tq, h = inp.total_q, inp.num_heads
    results = []
    for splits in (1, 4, 1):
        big_o = torch.full((tq + 2, h, 512), 7.25, dtype=torch.float32, device=dev)
        big_l = torch.full((tq + 2, h), 7.25, dtype=torch.float32, device=dev)
        out, lse = big_o[1:tq + 1], big_l[1:tq + 1]
        B.verify_attn(d["q_lat"], d["q_rope"], d["kv_lat"], d["k_rope"], d["prefix_len"],
                      d["tree_parent"], d["q_len"], inp.scale, out_lat=out, out_lse=lse,
                      num_splits=splits, max_q_len=inp.max_q_len)
        torch.cuda.synchronize(dev)
        assert (big_o[0] == 7.25).all() and (big_o[-1] == 7.25).all()
        assert (big_l[0] == 7.25).all() and (big_l[-1] == 7.25).all()
        results.append((out.clone(), lse.clone()))
    assert torch.equal(results[0][0], results[2][0]) and torch.equal(results[0][1], results[2][1])


def test_malformed_inputs_set_status(dev):
    base = EDGE["ragged_batch5_h64"]("bf16")
    cases = []
    bad_parent = base.tree_parent.copy()
    bad_parent[3] = 7                               # request 1 node 2: parent must be < 2
    cases.append(("bad_parent", dict(tree_parent=bad_parent), 4))
    bad_q = base.q_len.copy()
    bad_q[2] = 0
    cases.append(("bad_qlen", dict(q_len=bad_q), 1))
    bad_p = base.prefix_len.copy()
    bad_p[1] = -3
    cases.append(("bad_prefix", dict(prefix_len=bad_p), 2))
    big_p = base.prefix_len.copy()
    big_p[4] = 10 ** 6
    cases.append(("overflow", dict(prefix_len=big_p), 8))
    for name, change, bit in cases:
        inp = synth.VerifyInputs(**{**base.__dict__, **change})
        d = synth.device_tensors(inp, dev)
        status = torch.zeros(1, dtype=torch.int32, device=dev)
        B.verify_attn(d["q_lat"], d["q_rope"], d["kv_lat"], d["k_rope"], d["prefix_len"],
                      d["tree_parent"], d["q_len"], inp.scale, num_splits=1,
                      max_q_len=65, status=status)
        torch.cuda.synchronize(dev)
        st = int(status.item())
        print(f"{name}: status {st} {B.decode_status(st)}", flush=True)
        assert st & bit, name


def test_hip_graph_capture_replays(dev):
    inp = EDGE["qlen65_p300_h64"]("bf16")
    d = synth.device_tensors(inp, dev)
    call = B.VerifyAttn()
    out = torch.empty((inp.total_q, inp.num_heads, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((inp.total_q, inp.num_heads), dtype=torch.float32, device=dev)
    ws = torch.empty(B.kdtree_verify_attn_workspace_bytes(inp.total_q, inp.total_kv, inp.batch,
                                                          inp.num_heads, 4, B.KDTREE_DTYPE_BF16),
                     dtype=torch.uint8, device=dev)
    args = (d["q_lat"], d["q_rope"], d["kv_lat"], d["k_rope"], d["prefix_len"], d["tree_parent"],
            d["q_len"], inp.scale)
    call(*args, out_lat=out, out_lse=lse, num_splits=4, max_q_len=65, workspace=ws)
    torch.cuda.synchronize(dev)
    ref_o, ref_l = out.clone(), lse.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            call(*args, out_lat=out, out_lse=lse, num_splits=4, max_q_len=65, workspace=ws)
    for i in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize(dev)
        g.replay()
        torch.cuda.synchronize(dev)
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"replay {i}"


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_prepare_then_attend(dev, dtype):
    """The two-phase calls give the one-call result bit for bit, and one prepare serves
    several attend calls (also with a different split count over the same workspace)."""
    inp = EDGE["ragged_batch5_h64"](dtype)
    d = synth.device_tensors(inp, dev)
    call = B.VerifyAttn()
    dt = B.KDTREE_DTYPE_BF16 if dtype == "bf16" else B.KDTREE_DTYPE_FP32
    ws_bytes = max(1, B.kdtree_verify_attn_workspace_bytes(inp.total_q, inp.total_kv, inp.batch,
                                                           inp.num_heads, 4, dt))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    args = (d["q_lat"], d["q_rope"], d["kv_lat"], d["k_rope"], d["prefix_len"], d["tree_parent"],
            d["q_len"], inp.scale)
    ref = {s: call(*args, num_splits=s, max_q_len=65, workspace=ws) for s in (1, 4)}
    torch.cuda.synchronize(dev)
    ref = {s: (o.clone(), l.clone()) for s, (o, l) in ref.items()}
    ws.fill_(0xAB)
    call(*args, num_splits=1, max_q_len=65, workspace=ws, phase="prepare")
    for s in (1, 4, 1):
        out = torch.full_like(ref[s][0], float("nan"))
        lse = torch.full_like(ref[s][1], float("nan"))
        call(*args, out_lat=out, out_lse=lse, num_splits=s, max_q_len=65, workspace=ws,
             phase="attend")
        torch.cuda.synchronize(dev)
        assert torch.equal(out, ref[s][0]) and torch.equal(lse, ref[s][1]), f"splits={s}"
    mid = torch.cuda.Event()
    out, lse = call(*args, num_splits=4, max_q_len=65, workspace=ws, mid_event=mid)
    torch.cuda.synchronize(dev)
    assert torch.equal(out, ref[4][0]) and torch.equal(lse, ref[4][1])


@pytest.mark.parametrize("splits", [1, 4])
def test_flagged_request_rows_left_unwritten(dev, splits):
    """A request flagged on the device keeps its output rows; the others are unchanged."""
    base = EDGE["ragged_batch5_h64"]("bf16")
    bad_parent = base.tree_parent.copy()
    bad_parent[3] = 7  # request 1, node 2: a parent must precede its node
    inp = synth.VerifyInputs(**{**base.__dict__, "tree_parent": bad_parent})
    h = inp.num_heads
    outs = {}
    for name, x in (("clean", base), ("bad", inp)):
        d = synth.device_tensors(x, dev)
        out = torch.full((x.total_q, h, 512), 7.25, dtype=torch.float32, device=dev)
        lse = torch.full((x.total_q, h), 7.25, dtype=torch.float32, device=dev)
        status = torch.zeros(1, dtype=torch.int32, device=dev)
        print(f"case flagged/{name} splits={splits}", flush=True)
        B.verify_attn(d["q_lat"], d["q_rope"], d["kv_lat"], d["k_rope"], d["prefix_len"],
                      d["tree_parent"], d["q_len"], x.scale, out_lat=out, out_lse=lse,
                      num_splits=splits, max_q_len=65, status=status)
        torch.cuda.synchronize(dev)
        outs[name] = (out.cpu(), lse.cpu(), int(status.item()))
    assert outs["clean"][2] == 0 and outs["bad"][2] & 4
    q0 = int(base.q_len[0])
    q1 = q0 + int(base.q_len[1])
    assert (outs["bad"][0][q0:q1] == 7.25).all() and (outs["bad"][1][q0:q1] == 7.25).all()
    for a, b in ((outs["bad"][0], outs["clean"][0]), (outs["bad"][1], outs["clean"][1])):
        assert torch.equal(a[:q0], b[:q0]) and torch.equal(a[q1:], b[q1:])


@pytest.mark.parametrize("splits", [1, 4])
def test_rows_past_the_packed_total_left_unwritten(dev, splits):
    """total_q larger than sum(q_len): the spare output rows keep their contents."""
    inp = EDGE["ragged_batch5_h64"]("bf16")
    d = synth.device_tensors(inp, dev)
    extra = 3
    h = inp.num_heads

    def pad(t, fill):
        tail = torch.full((extra,) + tuple(t.shape[1:]), fill, dtype=t.dtype, device=dev)
        return torch.cat([t, tail]).contiguous()
    q_lat, q_rope = pad(d["q_lat"], 0.5), pad(d["q_rope"], 0.5)
    parent = pad(d["tree_parent"], -1)
    out = torch.full((inp.total_q + extra, h, 512), 7.25, dtype=torch.float32, device=dev)
    lse = torch.full((inp.total_q + extra, h), 7.25, dtype=torch.float32, device=dev)
    print(f"case spare_rows splits={splits}", flush=True)
    B.verify_attn(q_lat, q_rope, d["kv_lat"], d["k_rope"], d["prefix_len"], parent, d["q_len"],
                  inp.scale, out_lat=out, out_lse=lse, num_splits=splits, max_q_len=65)
    torch.cuda.synchronize(dev)
    assert (out[inp.total_q:] == 7.25).all() and (lse[inp.total_q:] == 7.25).all()
    r_out, r_lse = verify_attn_inputs(inp)
    check(f"spare_rows/{splits}", inp, out[:inp.total_q].double().cpu().numpy(),
          lse[:inp.total_q].double().cpu().numpy(), r_out, r_lse)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_spare_kv_rows_ignored(dev, dtype):
    """total_kv larger than the packed total: the spare rows are never read, so filling
    them with huge values changes nothing."""
    inp = EDGE["ragged_batch5_h64"](dtype)
    d = synth.device_tensors(inp, dev)
    extra = 100

    def pad(t):
        tail = torch.full((extra,) + tuple(t.shape[1:]), 3.0e4, dtype=t.dtype, device=dev)
        return torch.cat([t, tail]).contiguous()
    print(f"case spare_kv/{dtype}", flush=True)
    ref = B.verify_attn(d["q_lat"], d["q_rope"], d["kv_lat"], d["k_rope"], d["prefix_len"],
                        d["tree_parent"], d["q_len"], inp.scale, max_q_len=65, num_splits=3)
    got = B.verify_attn(d["q_lat"], d["q_rope"], pad(d["kv_lat"]), pad(d["k_rope"]),
                        d["prefix_len"], d["tree_parent"], d["q_len"], inp.scale, max_q_len=65,
                        num_splits=3)
    torch.cuda.synchronize(dev)
    assert torch.equal(ref[0], got[0]) and torch.equal(ref[1], got[1])


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_large_batch_of_small_requests(dev, dtype):
    """300 requests with 1..9 nodes and prefixes 0..200 (the request ranking, offsets and
    tile bookkeeping at a batch far above the workloads')."""
    rng = np.random.default_rng(77)
    parents = [synth.random_tree(rng, int(rng.integers(1, 10))) for _ in range(300)]
    prefix = rng.integers(0, 201, size=300)
    inp = synth.make_inputs(rng, num_heads=8, prefix_lens=prefix, parents=parents, dtype=dtype)
    full_check(f"batch300/{dtype}", inp, dev)
    full_check(f"batch300/{dtype}", inp, dev, num_splits=2)


def test_batch_beyond_the_ranking_limit(dev):
    """4100 requests, more than the pre-pass ranks (4096): the work is then handed out in
    request order, and each workgroup sums the lengths of up to 4099 earlier requests."""
    rng = np.random.default_rng(78)
    n = 4100
    parents = [synth.random_tree(rng, int(rng.integers(1, 4))) for _ in range(n)]
    prefix = rng.integers(0, 40, size=n)
    inp = synth.make_inputs(rng, num_heads=2, prefix_lens=prefix, parents=parents, dtype="bf16")
    full_check("batch4100", inp, dev)
    full_check("batch4100", inp, dev, num_splits=3)
