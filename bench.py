"""Benchmark of the MI355X tree-verify MLA-absorb attention.

One step = one kdtree_verify_attn call over the whole batch (one layer's verify
attention for every request) of the batch-64 ragged workload: H=64, q_len 33,
prefixes uniform in [1024, 8192] stored contiguously, half wide (top-8) / half deep
(top-2) best-first trees, bf16 inputs, fp32 output.  Inputs are synthetic, seeded, and
resident in HBM before timing starts.

Prints ONE JSON line (rank 0):
  value      = algorithmic TFLOP/s (2*(576+512) flops per visible (row, key) pair)
  roofline   = the attention kernel vs the dense MFMA peak of its dtype (bf16 2.5
               PFLOP/s), from HIP events recorded on the launch stream around it in
               every timed step (the call is issued as its two phases for that)
  cpu_baseline = the float64 oracle on a bounded sample of the same workload
  call_ms_percentiles = per-call event times (p10 / median / p90) and a cold-cache median
               (an untimed 1 GB write before each of --cold-calls extra calls)
  measured_peaks = a large bf16 / fp32 GEMM and a 1 GiB copy on the same box, with the
               attention kernel's fraction of them beside the spec-peak fractions
  greedy_step  = per-launch device time of the draft-tree build, tree packing and greedy
               accept kernels at the workload's tree shape (graph-replayed), beside the
               host heap oracle's build time for the same batch; step_us = the whole
               build -> pack -> verify -> accept chain as one graph; sample_*_us = the
               temperature draw over the full vocabulary at every node, on flat N(0, 2)
               logits and on peaked (LM-like) ones
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "verify_attn TFLOP/s and tree-verify steps/s (H=64, q_len 33/65); % MFMA peak"
PEAK_TFLOPS = {"bf16": 2500.0, "fp32": 157.3}
HBM_PEAK_GBS = 8000.0


# the sources of the kernels whose HBM counters are stored (every kernel of a bf16 call)
KERNEL_SOURCES = ("tree_verify_mla_attn_amd/csrc/attn_bf16.hip",
                  "tree_verify_mla_attn_amd/csrc/common.h",
                  "tree_verify_mla_attn_amd/csrc/prepass.hip",
                  "tree_verify_mla_attn_amd/csrc/merge.hip",
                  "tree_verify_mla_attn_amd/csrc/capi.hip")
# what the path computes in: bf16 inputs, fp16 MFMA for the latent dims (Q and the latent
# rows converted exactly), bf16 MFMA for the rope dims, fp32 accumulation and softmax
DTYPE_LABEL = {"bf16": "bf16 in, fp16/bf16 MFMA, fp32 acc",
               "fp32": "fp32 in, fp32 MFMA, fp32 acc"}


def kernel_source_digest():
    """sha256 over the bf16 call's kernel sources: stored HBM counter readings are used
    only while it still matches the digest recorded with them."""
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


PHASE_KERNELS = ("fill_nan_kernel", "verify_attn_bf16_kernel", "verify_attn_f32_kernel",
                 "piece_merge_kernel", "lse_merge_kernel")


def measured_traffic(path, workload, splits):
    """HBM bytes per call from rocprofv3 FETCH_SIZE / WRITE_SIZE readings (KiB per
    dispatch of every kernel of the call, each counter scaled by the factor a plain
    256 MiB device copy gave): the attention phase's kernels (the roofline's kernel) and
    the whole call (pre-pass included).  None when absent, for another workload, or taken
    on other kernel sources."""
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            doc = json.load(f)
    except (OSError, ValueError):
        return None
    for e in doc.get("entries", []):
        if e.get("workload") != workload or e.get("num_splits") != splits \
                or e.get("kernel_source_sha256") != kernel_source_digest():
            continue
        ff, wf = e["fetch_copy_factor"] * 1024, e["write_copy_factor"] * 1024
        per = {k: {"fetch": round(v["fetch_kib"] * ff), "write": round(v["write_kib"] * wf)}
               for k, v in e["kernels"].items()}
        phase = [v for k, v in per.items() if k in PHASE_KERNELS]
        return {"bytes": sum(v["fetch"] + v["write"] for v in phase),
                "fetch_bytes": sum(v["fetch"] for v in phase),
                "write_bytes": sum(v["write"] for v in phase),
                "call_bytes": sum(v["fetch"] + v["write"] for v in per.values()),
                "per_kernel": per}
    return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=4, help="1..5 (default: batch-64 ragged)")
    ap.add_argument("--num-splits", type=int, default=None)
    ap.add_argument("--split-ratio", type=float, default=None,
                    help="split-KV chunk ratio (1 = equal; default: the workload's)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the oracle baseline sample (0 = skip)")
    ap.add_argument("--cold-calls", type=int, default=10,
                    help="extra calls, each after an untimed 1 GB write, for a cold-cache median")
    ap.add_argument("--no-measure-peaks", dest="measure_peaks", action="store_false",
                    help="skip the GEMM / copy reference measurements")
    ap.add_argument("--sharded-share", action="store_true",
                    help="also time one GPU's share of the 32768-key workload under 8-way "
                         "context parallelism (always on with --workload 5)")
    ap.add_argument("--no-greedy-step", action="store_true",
                    help="skip timing the tree build / pack / accept kernels")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after timing, run one 256 MiB device copy (reference for HBM counters)")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="measured HBM bytes per launch (from rocprofv3 counters), if present")
    return ap.parse_args()


def cpu_baseline(inp, seconds):
    """Time the float64 oracle request by request until `seconds` have elapsed."""
    import numpy as np
    from oracle import verify_attn_f64 as O
    from tree_verify_mla_attn_amd import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([x.get("num_threads", 1) for x in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    qo, ko = inp.q_offsets(), inp.kv_offsets()
    flops = 0
    done = 0
    t0 = time.perf_counter()
    for b in range(inp.batch):
        t, p = int(inp.q_len[b]), int(inp.prefix_len[b])
        O.verify_attn(inp.q_lat[qo[b]:qo[b] + t], inp.q_rope[qo[b]:qo[b] + t],
                      inp.kv_lat[ko[b]:ko[b] + p + t], inp.k_rope[ko[b]:ko[b] + p + t], [p],
                      inp.parents_of(b), [t], inp.scale)
        dep = synth.tree_depths(inp.parents_of(b)).astype(np.int64)
        flops += int((p + dep + 1).sum()) * inp.num_heads * 2 * (576 + 512)
        done += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")),
                         model)
    except OSError:  # pragma: no cover
        pass
    affinity = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"float64 numpy oracle on the first {done} of {inp.batch} requests "
                      f"({flops:.3e} algorithmic FLOPs in {dt:.2f} s, BLAS threads={threads}, "
                      f"host cpus={os.cpu_count()}, affinity={affinity}, cpu={model})"}


def sharded_share(B, synth, torch, dev, parts=8, steps=20):
    """One GPU's share of the 32768-key workload under context parallelism across `parts`
    GPUs: the same 4 requests and trees, 32768 / parts prefix keys each, giving that GPU's
    partial output and log-sum-exp (num_splits and split_ratio chosen by the host-side
    schedule model, as for a single GPU); the cross-GPU merge would be the same LSE merge
    the split path runs."""
    import numpy as np
    c = synth.CONFIGS[5]
    rng, prefix, parents = synth.config_trees(5)
    share = [int(x) // parts for x in prefix]
    inp = synth.make_inputs(rng, num_heads=c["heads"], prefix_lens=share, parents=parents,
                            dtype=c["dtype"])
    d = synth.device_tensors(inp, dev)
    mean_kv = float(np.mean(share)) + inp.max_q_len
    splits, ratio = B.choose_splits(inp.batch, inp.num_heads, inp.max_q_len, mean_kv)
    call = B.VerifyAttn()
    out = torch.empty((inp.total_q, inp.num_heads, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((inp.total_q, inp.num_heads), dtype=torch.float32, device=dev)
    ws_bytes = B.kdtree_verify_attn_workspace_bytes(inp.total_q, inp.total_kv, inp.batch,
                                                    inp.num_heads, splits, B.KDTREE_DTYPE_BF16)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

    def run():
        call(d["q_lat"], d["q_rope"], d["kv_lat"], d["k_rope"], d["prefix_len"],
             d["tree_parent"], d["q_len"], inp.scale, out_lat=out, out_lse=lse,
             num_splits=splits, max_q_len=inp.max_q_len, workspace=ws, split_ratio=ratio)
    for _ in range(3):
        run()
    torch.cuda.synchronize(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize(dev)
    ms = e0.elapsed_time(e1) / steps
    return {"workload": f"{c['name']} / {parts}-way context share", "prefix_per_gpu": share[0],
            "num_splits": splits, "split_ratio": ratio, "ms": round(ms, 5),
            "TFLOPs": round(inp.algorithmic_flops() / (ms * 1e-3) / 1e12, 2),
            "merge_message_MB_per_gpu": round(inp.total_q * inp.num_heads * 513 * 4 / 1e6, 1)}


def measured_peaks(torch, dev):
    """What the box reaches on plain work, beside the spec peaks: a large square GEMM
    through torch (hipBLASLt; 2-D, contiguous operands) in bf16 and fp32, and a 1 GiB
    device-to-device copy (bytes read + written per second)."""
    out = {}
    n = 8192
    for name, dt in (("gemm_bf16_TFLOPs", torch.bfloat16), ("gemm_fp32_TFLOPs", torch.float32)):
        a = torch.randn((n, n), device=dev).to(dt).contiguous()
        b = torch.randn((n, n), device=dev).to(dt).contiguous()
        c = torch.matmul(a, b)
        torch.cuda.synchronize(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 10 if dt == torch.bfloat16 else 3
        e0.record()
        for _ in range(reps):
            c = torch.matmul(a, b)
        e1.record()
        torch.cuda.synchronize(dev)
        out[name] = round(2.0 * n ** 3 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e12, 1)
        del a, b, c
    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize(dev)
    out["copy_GBs"] = round(2.0 * src.numel() * 4 * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    del src, dst
    return out


def greedy_step_timing(B, synth, torch, dev, cfg, reps=64, replays=5, cpu_oracle=True,
                       verify=None):
    """Per-launch device time of the steps around verify attention (draft-tree build, tree
    packing, greedy accept) at a workload's tree shape, each as `reps` launches captured
    in one HIP graph and replayed `replays` times between two events."""
    import numpy as np
    c = synth.CONFIGS[cfg]
    rng = np.random.default_rng(1000 + cfg)
    batch, budget = c["batch"], c["budget"]
    ks = list(c["top_k"])
    ks = ks * (batch // len(ks)) if len(ks) != batch else ks
    logp, ids, root = synth.draft_tables(rng, batch, ks, depth=synth.MAX_DEPTH)
    d_logp = torch.from_numpy(logp).to(dev)
    d_ids = torch.from_numpy(ids).to(dev)
    d_root = torch.from_numpy(root).to(dev)
    t = B.build_ddtree(d_logp, d_ids, d_root, budget, with_score=False)
    torch.cuda.synchronize(dev)
    par, tok, ql = (t[k].cpu().numpy() for k in ("parent", "token", "q_len"))
    width = budget + 1
    tn = np.stack([synth.target_next_tokens(rng, par[b, :ql[b]], tok[b, :ql[b]], 0.8, width)
                   for b in range(batch)])
    d_tn = torch.from_numpy(tn).to(dev)
    i32 = torch.int32
    o = {k: torch.empty((batch, width), dtype=i32, device=dev)
         for k in ("parent", "token", "depth", "first_child", "next_sibling")}
    o_q = torch.empty((batch,), dtype=i32, device=dev)
    pk_par = torch.empty((batch * width,), dtype=i32, device=dev)
    pk_off = torch.empty((batch + 1,), dtype=torch.int64, device=dev)
    a_len = torch.empty((batch,), dtype=i32, device=dev)
    a_tok = torch.empty((batch, 16), dtype=i32, device=dev)
    a_node = torch.empty((batch, 16), dtype=i32, device=dev)

    def build(s):
        return B.kdtree_build_ddtree(d_logp.data_ptr(), d_ids.data_ptr(), d_root.data_ptr(),
                                     batch, logp.shape[1], logp.shape[2], budget, o_q.data_ptr(),
                                     o["parent"].data_ptr(), o["token"].data_ptr(),
                                     o["depth"].data_ptr(), o["first_child"].data_ptr(),
                                     o["next_sibling"].data_ptr(), 0, s)

    def pack(s):
        return B.kdtree_pack_tree(o_q.data_ptr(), o["parent"].data_ptr(), 0, batch, width,
                                  batch * width, pk_par.data_ptr(), 0, pk_off.data_ptr(), s)

    def accept(s):
        return B.kdtree_tree_accept(o["token"].data_ptr(), o["first_child"].data_ptr(),
                                    o["next_sibling"].data_ptr(), o_q.data_ptr(), d_tn.data_ptr(),
                                    batch, width, 16, a_len.data_ptr(), a_tok.data_ptr(),
                                    a_node.data_ptr(), s)

    res = {"workload": c["name"], "batch": batch, "budget": budget, "depth": synth.MAX_DEPTH,
           "top_k": "per request, as the workload's trees"}
    for name, fn in (("build", build), ("pack", pack), ("accept", accept)):
        cs = torch.cuda.Stream(device=dev)
        cs.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(cs):
            assert fn(cs.cuda_stream) == 0
        torch.cuda.current_stream(dev).wait_stream(cs)
        torch.cuda.synchronize(dev)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            s = torch.cuda.current_stream(dev).cuda_stream
            for _ in range(reps):
                assert fn(s) == 0
        g.replay()
        torch.cuda.synchronize(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(replays):
            g.replay()
        e1.record()
        torch.cuda.synchronize(dev)
        res[f"{name}_us"] = round(e0.elapsed_time(e1) * 1e3 / (reps * replays), 3)
    acc = a_len.cpu().numpy()
    res["mean_accept_len"] = round(float(acc.mean()), 3)
    # the temperature path's draw: the target's next token at every node from logits over
    # the full vocabulary (synthetic N(0, 2) logits), fp32 and bf16, T = 0.8
    for dt_name, dt, peaked in (("fp32", torch.float32, False), ("bf16", torch.bfloat16, False),
                                ("fp32_peaked", torch.float32, True),
                                ("bf16_peaked", torch.bfloat16, True)):
        logits = torch.randn((batch * width, synth.VOCAB), device=dev) * 2.0
        if peaked:  # LM-like rows: an N(0, 2) bulk and 12 candidates near +24
            top = torch.randint(0, synth.VOCAB, (batch * width, 12), device=dev)
            logits.scatter_(1, top, 24.0 + 1.5 * torch.randn((batch * width, 12), device=dev))
        logits = logits.to(dt)
        toks = torch.empty((batch * width,), dtype=i32, device=dev)
        code = B.KDTREE_DTYPE_BF16 if dt == torch.bfloat16 else B.KDTREE_DTYPE_FP32

        def draw(s, logits=logits, toks=toks, code=code):
            return B.kdtree_sample_tokens(logits.data_ptr(), code, batch * width, synth.VOCAB,
                                          synth.VOCAB, 0.8, 1234, 5, toks.data_ptr(), s)
        assert draw(torch.cuda.current_stream(dev).cuda_stream) == 0
        torch.cuda.synchronize(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            assert draw(torch.cuda.current_stream(dev).cuda_stream) == 0
        e1.record()
        torch.cuda.synchronize(dev)
        us = e0.elapsed_time(e1) * 1e3 / 10
        nbytes = batch * width * synth.VOCAB * logits.element_size()
        res[f"sample_{dt_name}_us"] = round(us, 2)
        res[f"sample_{dt_name}_GBs"] = round(nbytes / (us * 1e-6) / 1e9, 1)
        del logits
    if verify is not None:
        # the whole step on the device: build -> pack -> verify attention over the built
        # trees (the workload's q / kv rows, which its trees fill exactly) -> accept on
        # fixed target tokens (the target model's argmax is outside this path)
        vq, vqr, vkv, vkr, vprefix, vout, vlse, vws, vsplits, vscale, vratio = verify
        if int(vq.shape[0]) != batch * width:
            res["step_us"] = None
        else:
            def chain(s):
                assert build(s) == 0 and pack(s) == 0
                B.VerifyAttn()(vq, vqr, vkv, vkr, vprefix, pk_par, o_q, vscale, out_lat=vout,
                               out_lse=vlse, num_splits=vsplits, max_q_len=width, workspace=vws,
                               split_ratio=vratio)
                assert accept(s) == 0
            cs = torch.cuda.Stream(device=dev)
            cs.wait_stream(torch.cuda.current_stream(dev))
            with torch.cuda.stream(cs):
                chain(cs.cuda_stream)
            torch.cuda.current_stream(dev).wait_stream(cs)
            torch.cuda.synchronize(dev)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                chain(torch.cuda.current_stream(dev).cuda_stream)
            g.replay()
            torch.cuda.synchronize(dev)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(replays * 4):
                g.replay()
            e1.record()
            torch.cuda.synchronize(dev)
            res["step_us"] = round(e0.elapsed_time(e1) * 1e3 / (replays * 4), 2)
    if cpu_oracle:
        from oracle import ddtree_f32 as O  # the host heap the device builder replaces
        t0 = time.perf_counter()
        n = 0
        while time.perf_counter() - t0 < 1.0:
            O.build_ddtree_batch(logp, ids, root, budget)
            n += 1
        res["cpu_baseline_build_us"] = {"value": round((time.perf_counter() - t0) * 1e6 / n, 1),
                                        "kind": "oracle", "cores": 1,
                                        "sample": f"{n} whole-batch builds in about 1 s"}
    return res


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the kernel works "
              "on one GPU's share and there is no multi-GPU path", file=sys.stderr)
        sys.exit(2)
    import torch
    from tree_verify_mla_attn_amd import binding as B
    from tree_verify_mla_attn_amd import synth

    B.load_library()
    dev = torch.device("cuda:0")
    inp = synth.config_inputs(args.workload)
    splits = args.num_splits or inp.num_splits
    ratio = args.split_ratio if args.split_ratio is not None else inp.split_ratio
    d = synth.device_tensors(inp, dev)
    flops = inp.algorithmic_flops()
    alg_bytes = inp.algorithmic_bytes()
    call = B.VerifyAttn()
    out = torch.empty((inp.total_q, inp.num_heads, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((inp.total_q, inp.num_heads), dtype=torch.float32, device=dev)
    ws_bytes = B.kdtree_verify_attn_workspace_bytes(
        inp.total_q, inp.total_kv, inp.batch, inp.num_heads, splits,
        B.KDTREE_DTYPE_BF16 if inp.dtype == "bf16" else B.KDTREE_DTYPE_FP32)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    argv = (d["q_lat"], d["q_rope"], d["kv_lat"], d["k_rope"], d["prefix_len"], d["tree_parent"],
            d["q_len"], inp.scale)

    def step(mid=None):
        call(*argv, out_lat=out, out_lse=lse, num_splits=splits, max_q_len=inp.max_q_len,
             workspace=ws, status=status, mid_event=mid, split_ratio=ratio)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)
    st = int(status.item())
    if st:
        raise RuntimeError(f"device status {B.decode_status(st)}")

    stream = torch.cuda.current_stream(dev)
    # Events on the launch stream: ev[i] -> mid[i] is the pre-pass (bf16 inputs),
    # mid[i] -> ev[i + 1] the attention kernel (+ the partial-lse fill and the merge when
    # num_splits > 1).
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    mid = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        step(mid[i])
        ev[i + 1].record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    st = int(status.item())
    if st:
        raise RuntimeError(f"device status {B.decode_status(st)}")
    ms = wall * 1e3 / args.steps
    call_each = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
    att_each = sorted(mid[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
    call_ms = sum(call_each) / args.steps
    pre_ms = sum(ev[i].elapsed_time(mid[i]) for i in range(args.steps)) / args.steps
    ev_ms = sum(att_each) / args.steps

    def pct(xs, q):
        return xs[min(len(xs) - 1, int(round(q * (len(xs) - 1))))]

    # cold caches: an untimed 1 GB write before each call evicts L2 and the MALL
    cold = []
    if args.cold_calls > 0:
        flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        for _ in range(args.cold_calls):
            flush.fill_(1.0)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step()
            e1.record(stream)
            torch.cuda.synchronize(dev)
            cold.append(e0.elapsed_time(e1))
        del flush
        cold.sort()
    measured = measured_peaks(torch, dev) if args.measure_peaks else None

    dtype = inp.dtype
    bf16_id = B.KDTREE_DTYPE_BF16 if dtype == "bf16" else B.KDTREE_DTYPE_FP32
    if splits > 1:
        kernel_label = "attention + merge"
    elif B.launch_uses_cut(inp.batch, inp.num_heads, inp.max_q_len, splits, bf16_id):
        kernel_label = "attention + piece merge"
    else:
        kernel_label = "attention"
    value = flops / (ms * 1e-3) / 1e12
    achieved = flops / (ev_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[dtype]
    traffic = measured_traffic(args.traffic_json, inp.name, splits)

    res = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "steps_per_s": round(1e3 / ms, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_LABEL[dtype],
        "data": "synthetic (seeded N(0,1) MLA tensors, best-first draft trees)",
        "config": {"workload": inp.name, "batch": inp.batch, "heads": inp.num_heads,
                   "q_len": int(inp.max_q_len), "total_q": inp.total_q, "total_kv": inp.total_kv,
                   "num_splits": splits, "split_ratio": ratio, "d_latent": 512, "d_rope": 64,
                   "algorithmic_flops": flops, "algorithmic_bytes": alg_bytes},
        "roofline": {"bound": "mfma", "kernel": kernel_label,
                     "achieved": round(achieved, 3), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": traffic["bytes"] if traffic else None},
        "hbm": {"achieved_GBs": round(alg_bytes / (ev_ms * 1e-3) / 1e9, 1),
                "peak_GBs": HBM_PEAK_GBS,
                "frac": round(alg_bytes / (ev_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "measured": traffic,
                "measured_GBs": round(traffic["bytes"] / (ev_ms * 1e-3) / 1e9, 1) if traffic else None,
                "call_bytes_over_algorithmic":
                    round(traffic["call_bytes"] / alg_bytes, 3) if traffic else None},
        "call_ms_percentiles": {"p10": round(pct(call_each, 0.1), 5),
                                "median": round(pct(call_each, 0.5), 5),
                                "p90": round(pct(call_each, 0.9), 5),
                                "cold_median": round(pct(cold, 0.5), 5) if cold else None,
                                "cold_calls": len(cold)},
        "kernel_ms": {"attention": round(ev_ms, 5), "prepass": round(pre_ms, 5),
                      "call": round(call_ms, 5)},
    }
    if measured:
        res["measured_peaks"] = measured
        key = "gemm_bf16_TFLOPs" if dtype == "bf16" else "gemm_fp32_TFLOPs"
        res["roofline"]["frac_of_measured_peak"] = round(achieved / measured[key], 4)
        res["hbm"]["frac_of_measured_copy"] = round(
            alg_bytes / (ev_ms * 1e-3) / 1e9 / measured["copy_GBs"], 4)
    if args.calibrate_copy:
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize(dev)
        dst.copy_(src)
        torch.cuda.synchronize(dev)
        print(f"calibration copy: {src.numel() * 4} bytes read, {dst.numel() * 4} bytes written",
              file=sys.stderr, flush=True)
    if args.cpu_seconds > 0:
        res["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    if args.workload == 5 or args.sharded_share:
        res["sharded_share"] = sharded_share(B, synth, torch, dev)
    if not args.no_greedy_step:
        res["greedy_step"] = greedy_step_timing(
            B, synth, torch, dev, args.workload, cpu_oracle=args.cpu_seconds > 0,
            verify=(d["q_lat"], d["q_rope"], d["kv_lat"], d["k_rope"], d["prefix_len"], out, lse,
                    ws, splits, inp.scale, ratio))
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
