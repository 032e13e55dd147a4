"""Host-side checks of the C ABI (no GPU needed: every call here fails validation before
anything is enqueued, or is a pure size query)."""
import ctypes
import os
import re
import subprocess

import pytest

from tree_verify_mla_attn_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kdtree_verify.h")
FAKE = 0x1000  # never dereferenced: these calls fail host validation first


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kdtree_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = B.load_library()
    names = _declared_functions()
    assert names == ["kdtree_build_ddtree", "kdtree_max_qlen", "kdtree_pack_tree",
                     "kdtree_sample_tokens", "kdtree_tree_accept",
                     "kdtree_verify_attn", "kdtree_verify_attn_attend",
                     "kdtree_verify_attn_noalloc", "kdtree_verify_attn_prepare",
                     "kdtree_verify_attn_workspace_bytes"]
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"
    out = subprocess.run(["nm", "-D", "--defined-only", B.lib_path()], capture_output=True,
                         text=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}$", out, flags=re.M), f"{n} not a defined text symbol"


def test_header_constants_match_binding():
    text = open(HEADER).read()
    assert re.search(r"#define KDTREE_MAX_QLEN 65\b", text)
    assert re.search(r"#define KDTREE_NOALLOC_SCRATCH_BYTES \(128u \* 1024u \* 1024u\)", text)
    assert B.KDTREE_NOALLOC_SCRATCH_BYTES == 128 * 1024 * 1024
    assert B.kdtree_max_qlen() == 65 == B.KDTREE_MAX_QLEN
    for code in B.ERRORS:
        if code:
            assert re.search(rf"\(({code})\)", text), f"error code {code} missing from header"


def test_workspace_bytes():
    def up(x):
        return -(-x // 256) * 256
    # fp32, one split: nothing
    assert B.kdtree_verify_attn_workspace_bytes(100, 5000, 2, 64, 1, 0) == 0
    # bf16, one split: the request records (64 bytes each), the fp16 latent tiles, and the area of the
    # last-round cut: 32 piece slots per XCD that receives work (min(batch, 8) XCDs),
    # each 128 rows x (512 + 1) fp32, then 2 int64 per slot
    def pieces(batch):
        slots = 32 * min(batch, 8)
        return slots * 128 * 513 * 4 + slots * 16
    assert B.kdtree_verify_attn_workspace_bytes(100, 5000, 2, 64, 1, 1) == up(2 * 64) + up((5000 // 32 + 2 + 1) * 32768) + pieces(2)
    assert B.kdtree_verify_attn_workspace_bytes(9, 300, 1, 64, 1, 1) == up(64) + up((300 // 32 + 1 + 1) * 32768) + pieces(1)
    assert B.kdtree_verify_attn_workspace_bytes(900, 9000, 30, 8, 1, 1) == up(30 * 64) + up((9000 // 32 + 30 + 1) * 32768) + pieces(30)
    # bf16, 16 splits: tiles + partial outputs + partial lse (larger than the cut area,
    # which shares their region)
    tq, tkv, b, h, s = 260, 131332, 4, 64, 16
    rows = tq * h
    want = up(b * 64) + up((tkv // 32 + b + 1) * 32768) + up(s * rows * 512 * 4) + up(s * rows * 4)
    assert B.kdtree_verify_attn_workspace_bytes(tq, tkv, b, h, s, 1) == want
    # bf16, 2 splits of a small batch: the partials (26 MB) outgrow the cut area (17 MB)
    assert B.kdtree_verify_attn_workspace_bytes(100, 5000, 2, 64, 2, 1) == \
        up(2 * 64) + up((5000 // 32 + 2 + 1) * 32768) + up(2 * 6400 * 512 * 4) + up(2 * 6400 * 4)
    # ... and with few rows the cut area is the larger
    assert B.kdtree_verify_attn_workspace_bytes(10, 500, 2, 8, 2, 1) == \
        up(2 * 64) + up((500 // 32 + 2 + 1) * 32768) + pieces(2)
    # never smaller for more splits
    for dt in (0, 1):
        sizes = [B.kdtree_verify_attn_workspace_bytes(165, 1500, 5, 64, k, dt) for k in range(1, 40)]
        assert sizes == sorted(sizes)
    # fp32, splits: partials only
    assert B.kdtree_verify_attn_workspace_bytes(tq, tkv, b, h, s, 0) == up(s * rows * 512 * 4) + up(s * rows * 4)
    for bad in [(0, 10, 1, 64, 2, 1), (10, 10, 1, 64, 0, 1), (10, 10, 1, 64, 257, 1),
                (10, 10, 1, 64, 2, 3), (10, 10, 0, 64, 2, 1)]:
        assert B.kdtree_verify_attn_workspace_bytes(*bad) == 0


def _call(entry="kdtree_verify_attn", **kw):
    args = dict(q_lat=FAKE, q_rope=FAKE, kv_lat=FAKE, k_rope=FAKE, prefix_len=FAKE,
                tree_parent=FAKE, q_len=FAKE, scale=0.07, out_lat=FAKE, out_lse=FAKE, stream=0,
                batch=2, num_heads=64, max_q_len=33, total_q=66, total_kv=2000, dtype=1,
                num_splits=1, workspace=0, workspace_bytes=0, status=0)
    args.update(kw)
    return getattr(B, entry)(**args)


ENTRIES = list(B.ENTRY_POINTS)


@pytest.mark.parametrize("entry", ENTRIES)
@pytest.mark.parametrize("field", ["q_lat", "q_rope", "kv_lat", "k_rope", "prefix_len",
                                   "tree_parent", "q_len", "out_lat", "out_lse"])
def test_null_pointer_rejected(entry, field):
    assert _call(entry, **{field: 0}) == -1


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), -2), (dict(num_heads=0), -2), (dict(total_q=1), -2),
    (dict(total_kv=10), -2), (dict(max_q_len=0), -3), (dict(max_q_len=66), -3),
    (dict(dtype=2), -4), (dict(dtype=-1), -4), (dict(num_splits=0), -5),
    (dict(num_splits=300), -5), (dict(num_splits=4), -5), (dict(dtype=1, num_splits=1), -5),
    (dict(num_splits=4, workspace=FAKE, workspace_bytes=16), -5),
    (dict(scale=float("nan")), -6), (dict(scale=float("inf")), -6),
    (dict(split_ratio=0.0), -5), (dict(split_ratio=-0.5), -5), (dict(split_ratio=1.5), -5),
    (dict(split_ratio=float("nan")), -5),
])
@pytest.mark.parametrize("entry", ENTRIES)
def test_bad_arguments_rejected(entry, kw, code):
    assert _call(entry, **kw) == code


def test_product_path_does_not_touch_the_oracle():
    pkg = os.path.join(ROOT, "tree_verify_mla_attn_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(from|import)\s+oracle\b", text, flags=re.M), f
                assert "oracle/" not in text, f


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setenv("KDTREE_LIB", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError):
        B.load_library()
    monkeypatch.setattr(B, "_lib", None)


def test_choose_num_splits():
    # few row tiles + long prefixes -> more splits; many tiles -> none
    # the counts a sweep on MI355X found fastest for the five workloads' shapes
    assert B.choose_num_splits(1, 64, 33, 2081, dtype=B.KDTREE_DTYPE_FP32) == 7
    assert 8 <= B.choose_num_splits(1, 64, 9, 265, dtype=B.KDTREE_DTYPE_FP32) <= 12
    assert B.choose_num_splits(8, 64, 65, 4161) == 2
    assert B.choose_num_splits(64, 64, 33, 4790) == 1
    assert B.choose_num_splits(4, 64, 65, 32833) > 1


def test_choose_split_ratio():
    # the ratios sweeps on MI355X found fastest (bf16): 0.35-0.4 for 8 requests of
    # 4096 + 65 keys at 2 splits, 0.85 (0.82-0.88 within noise) for 4 of 32768 + 65 at 16
    assert 0.35 <= B.choose_split_ratio(8, 64, 65, 4161, 2) <= 0.45
    assert 0.8 <= B.choose_split_ratio(4, 64, 65, 32833, 16) <= 0.9
    # nothing to balance: one split, or workgroups that fill whole rounds of every XCD
    assert B.choose_split_ratio(64, 64, 33, 4790, 1) == 1.0
    assert B.choose_split_ratio(8, 64, 64, 4096, 4) == 1.0
    # the fp32 launch of the 2048-key prefix fits one round at 7 splits
    assert B.choose_split_ratio(1, 64, 33, 2081, 7, dtype=B.KDTREE_DTYPE_FP32) == 1.0
    # a geometric ratio that would leave a split empty is never chosen (equal splits of
    # a short prefix may be, as the kernels allow)
    chosen = []
    for batch, mean_kv in ((8, 4161), (3, 2000), (2, 300)):
        for s in (2, 3, 4, 6, 8, 12, 16, 64):
            r = B.choose_split_ratio(batch, 64, 65, mean_kv, s)
            if r < 1.0:
                chosen.append(r)
                ends = [B._split_begin(mean_kv - 65, s, r, k) for k in range(s + 1)]
                assert all(b < e for b, e in zip(ends[:-2], ends[1:-1])), (s, r, ends)
    assert len(chosen) >= 5


def test_choose_splits():
    # (count, ratio) pairs that ran fastest of those timed on MI355X (bf16, 64 heads)
    assert B.choose_splits(4, 64, 65, 4161) == (4, 0.75)    # 2..8 splits timed
    assert B.choose_splits(8, 64, 65, 4161) == (1, 1.0)     # with the last-round cut
    assert B.choose_splits(4, 64, 65, 32833) == (8, 0.75)   # 8, 12, 16 timed
    assert B.choose_splits(64, 64, 33, 5120) == (1, 1.0)    # the batch-64 launch


# ---------------------------------------------------------------- builder and accept
def _build(**kw):
    args = dict(logp=FAKE, token_ids=FAKE, root_token=FAKE, batch=2, depth=15, top_k=8,
                budget=64, q_len=FAKE, tree_parent=FAKE, tree_token=FAKE, tree_depth=FAKE,
                first_child=FAKE, next_sibling=FAKE, tree_score=0, stream=0)
    args.update(kw)
    return B.kdtree_build_ddtree(**args)


@pytest.mark.parametrize("field", ["logp", "token_ids", "root_token", "q_len", "tree_parent",
                                   "tree_token", "tree_depth", "first_child", "next_sibling"])
def test_build_null_pointer_rejected(field):
    assert _build(**{field: 0}) == -1


@pytest.mark.parametrize("kw", [dict(batch=0), dict(depth=0), dict(depth=65), dict(top_k=0),
                                dict(top_k=4096, depth=1), dict(depth=64, top_k=65),
                                dict(budget=-1), dict(budget=65)])
def test_build_bad_shape_rejected(kw):
    assert _build(**kw) == -2


def test_build_limits_match_header():
    text = open(HEADER).read()
    for name in ("KDTREE_MAX_BUDGET", "KDTREE_MAX_DEPTH", "KDTREE_MAX_TABLE",
                 "KDTREE_MAX_ACCEPT_NODES"):
        m = re.search(rf"#define {name} (\d+)", text)
        assert m and int(m.group(1)) == getattr(B, name)
    src = open(os.path.join(ROOT, "tree_verify_mla_attn_amd", "csrc", "common.h")).read()
    for name, c in (("KDTREE_MAX_BUDGET", "MAX_DDTREE_BUDGET"), ("KDTREE_MAX_DEPTH", "MAX_DDTREE_DEPTH"),
                    ("KDTREE_MAX_TABLE", "MAX_DDTREE_TABLE"),
                    ("KDTREE_MAX_ACCEPT_NODES", "MAX_ACCEPT_NODES")):
        m = re.search(rf"constexpr int {c} = (\d+);", src)
        assert m and int(m.group(1)) == getattr(B, name)


def _accept(**kw):
    args = dict(tree_token=FAKE, first_child=FAKE, next_sibling=FAKE, q_len=FAKE,
                target_next=FAKE, batch=2, max_nodes=65, max_accept=16, accept_len=FAKE,
                accept_tokens=FAKE, accept_nodes=FAKE, stream=0)
    args.update(kw)
    return B.kdtree_tree_accept(**args)


@pytest.mark.parametrize("field", ["tree_token", "first_child", "next_sibling", "q_len",
                                   "target_next", "accept_len", "accept_tokens", "accept_nodes"])
def test_accept_null_pointer_rejected(field):
    assert _accept(**{field: 0}) == -1


@pytest.mark.parametrize("kw", [dict(batch=0), dict(max_nodes=0), dict(max_accept=0),
                                dict(max_nodes=B.KDTREE_MAX_ACCEPT_NODES + 1),
                                dict(max_accept=(1 << 20) + 1)])
def test_accept_bad_shape_rejected(kw):
    assert _accept(**kw) == -2


def _pack(**kw):
    args = dict(q_len=FAKE, tree_parent=FAKE, tree_token=FAKE, batch=2, width=33, total_q=66,
                packed_parent=FAKE, packed_token=FAKE, q_offsets=0, stream=0)
    args.update(kw)
    return B.kdtree_pack_tree(**args)


@pytest.mark.parametrize("kw", [dict(q_len=0), dict(tree_parent=0), dict(packed_parent=0),
                                dict(tree_token=0)])
def test_pack_null_pointer_rejected(kw):
    assert _pack(**kw) == -1


@pytest.mark.parametrize("kw", [dict(batch=0), dict(width=0), dict(width=(1 << 20) + 1),
                                dict(total_q=0)])
def test_pack_bad_shape_rejected(kw):
    assert _pack(**kw) == -2


def _sample(**kw):
    args = dict(logits=FAKE, dtype=0, rows=4, vocab=1000, row_stride=1000, temperature=1.0,
                seed=1, offset=0, tokens=FAKE, stream=0)
    args.update(kw)
    return B.kdtree_sample_tokens(**args)


@pytest.mark.parametrize("kw,code", [
    (dict(logits=0), -1), (dict(tokens=0), -1),
    (dict(rows=0), -2), (dict(rows=2 ** 31), -2), (dict(vocab=0), -2),
    (dict(row_stride=999), -2), (dict(dtype=2), -4),
    (dict(temperature=-0.5), -6), (dict(temperature=float("inf")), -6),
    (dict(temperature=float("nan")), -6)])
def test_sample_bad_arguments_rejected(kw, code):
    assert _sample(**kw) == code


def test_launch_uses_cut(monkeypatch):
    """The host copy of the library's cut rule on the workloads' shapes: batch 8 at q_len
    65 (33 row tiles a request, one request per XCD: one whole round + 1 left) is cut;
    batch 64 at q_len 33 (8 requests x 17 row tiles per XCD = 4.25 rounds) is not; one
    request of 9 nodes (5 row tiles on one XCD) is cut; split launches and fp32 never;
    the switch turns it off."""
    monkeypatch.delenv("KDTREE_DISABLE_CUT", raising=False)
    assert B.launch_uses_cut(8, 64, 65, 1)
    assert not B.launch_uses_cut(64, 64, 33, 1)
    assert B.launch_uses_cut(1, 64, 9, 1)
    assert not B.launch_uses_cut(8, 64, 65, 2)
    assert not B.launch_uses_cut(8, 64, 65, 1, B.KDTREE_DTYPE_FP32)
    # 24 requests of 65 nodes: 3 x 33 = 99 row tiles per XCD, 3 whole rounds
    assert not B.launch_uses_cut(24, 64, 65, 1)
    monkeypatch.setenv("KDTREE_DISABLE_CUT", "1")
    assert not B.launch_uses_cut(8, 64, 65, 1)


def test_noalloc_rejects_what_does_not_fit():
    """A call whose workspace need exceeds the static scratch is refused before anything
    touches the device (the need follows from host scalars alone)."""
    kw = dict(q_lat=FAKE, q_rope=FAKE, kv_lat=FAKE, k_rope=FAKE, prefix_len=FAKE,
              tree_parent=FAKE, q_len=FAKE, scale=0.07, out_lat=FAKE, out_lse=FAKE, stream=0,
              batch=64, num_heads=64, max_q_len=33, total_q=2112, total_kv=306580, dtype=1,
              num_splits=1, status=0)
    need = B.kdtree_verify_attn_workspace_bytes(2112, 306580, 64, 64, 1, 1)
    assert need > B.KDTREE_NOALLOC_SCRATCH_BYTES
    assert B.kdtree_verify_attn_noalloc(**kw) == -8
    kw.update(num_splits=16, dtype=0)
    assert B.kdtree_verify_attn_noalloc(**kw) == -8
    # argument errors keep their codes
    kw.update(num_splits=1, dtype=1, total_q=66, total_kv=2000, batch=2, q_lat=0)
    assert B.kdtree_verify_attn_noalloc(**kw) == -1
