#!/usr/bin/env python3
"""Benchmark of one query-aware sparse decode step on one MI355X.

Workload (the headline setting): a Llama-7B-like attention layer at 32K
context, B=1, Hq=Hkv=32, d=128, bf16 q/K/V ~ N(0,1) times per-channel scales
U(0.5, 2), 8 planted needles per head, 16-token pages, a 2048-token budget
(126 pages by score + sink page + recent page), Quest min/max scoring.

A step = score every page -> exact top-K -> split-K attention over the kept
pages (+ merge), i.e. one sa_decode_step call.  The page metadata is built
once per layer copy beforehand (the insert-time update, not part of a step).
Inputs are resident in HBM before timing starts.  R = 16 copies of the layer
(8.7 GB) are rotated, and every step uses a fresh seeded query, so neither
the 256 MB Infinity Cache nor a repeated selection can serve the reads.

value = effective HBM GB/s of the step = algorithmic bytes (metadata of every
page + K/V of the kept pages + q + out) / step time.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse decode-step µs + effective HBM GB/s (% of peak), 32K ctx, 2048-token budget"
PEAK_GBS = 8000.0  # MI355X HBM3E
STEP_KERNEL = "quest_step_kernel"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "quest_step_kernel_llama7b_32k_traffic.json")
CALIB_BYTES = 256 << 20  # the plain copy timed beside the step in a counter run
# sources the fused step kernel is compiled from: counters taken on other sources are stale
KERNEL_SOURCES = ["include/sa.h"] + [
    "query_aware_sparse_min_amd/csrc/" + f
    for f in ("sa_step.hip", "sa_step.h", "sa_dev_score.h", "sa_dev_topk.h", "sa_dev_attn.h",
              "sa_internal.h")]


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=16, help="layer copies rotated per step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--pmc-run", action="store_true",
                    help="run a few steps and a plain copy of known size, for a counter run")
    ap.add_argument("--configs", default="",
                    help="instead of the headline line, one line per listed workload "
                         "(1-5, 5d = config 5 with every page kept, 2p = config 2 selected by "
                         "probe sampling, 3h = config 3 with per-head selection, 2a / 4a = the "
                         "decode-time append on config 2 / 4), e.g. --configs 1,3,3h,4,5,5d,2p,2a,4a")
    ap.add_argument("--parse-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the HBM traffic record from two rocprofv3 --pmc outputs")
    ap.add_argument("--pmc-kernels", default="",
                    help="with --parse-pmc: print scaled bytes per launch of these kernels "
                         "(comma-separated name parts) instead of writing the step record")
    return ap.parse_args()


def parse_pmc(fetch_csv, write_csv, kernels=""):
    """HBM bytes per kernel launch from rocprofv3 counter files (FETCH_SIZE,
    WRITE_SIZE in KiB per dispatch), each scaled by what the same counter reads
    for the plain copy of CALIB_BYTES that the counter run also launches.  Without
    `kernels` this writes the record of the fused step kernel; with a list of kernel
    names it prints one line per kernel."""
    import csv

    def per_kernel(path, counter, name):
        """(values of kernels whose name contains `name`, last copy dispatch) in bytes."""
        step, copies = [], []
        with open(path) as fh:
            for r in csv.DictReader(fh):
                if r.get("Counter_Name") != counter:
                    continue
                v = float(r["Counter_Value"]) * 1024.0
                if name in r["Kernel_Name"]:
                    step.append(v)
                elif "copy" in r["Kernel_Name"].lower():
                    copies.append((int(r["Dispatch_Id"]), v))
        return step, max(copies)[1]  # the calibration copy is the last copy dispatched

    if kernels:
        for name in kernels.split(","):
            fs, fc = per_kernel(fetch_csv, "FETCH_SIZE", name)
            ws, wc = per_kernel(write_csv, "WRITE_SIZE", name)
            if not fs or not ws:
                print(json.dumps({"kernel": name, "dispatches": 0}))
                continue
            fk, wk = sum(fs) / len(fs), sum(ws) / len(ws)
            print(json.dumps({"kernel": name, "dispatches": len(fs),
                              "fetch_bytes_raw": round(fk), "write_bytes_raw": round(wk),
                              "fetch_scale": CALIB_BYTES / fc, "write_scale": CALIB_BYTES / wc,
                              "fetch_bytes": round(fk * CALIB_BYTES / fc),
                              "write_bytes": round(wk * CALIB_BYTES / wc)}))
        return
    fs, fc = per_kernel(fetch_csv, "FETCH_SIZE", STEP_KERNEL)
    ws, wc = per_kernel(write_csv, "WRITE_SIZE", STEP_KERNEL)
    fk, wk = sum(fs) / len(fs), sum(ws) / len(ws)
    rec = {"kernel": STEP_KERNEL, "kernel_src_sha": kernel_source_hash(),
           "fetch_bytes_raw": round(fk), "write_bytes_raw": round(wk),
           "copy_bytes": CALIB_BYTES, "copy_fetch_raw": round(fc), "copy_write_raw": round(wc),
           "fetch_scale": CALIB_BYTES / fc, "write_scale": CALIB_BYTES / wc,
           "fetch_bytes": round(fk * CALIB_BYTES / fc), "write_bytes": round(wk * CALIB_BYTES / wc)}
    rec["traffic_bytes"] = rec["fetch_bytes"] + rec["write_bytes"]
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec))


def load_traffic():
    """Counter-measured bytes per launch, or None when absent or taken on other sources."""
    import json
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    return rec.get("traffic_bytes") if rec.get("kernel_src_sha") == kernel_source_hash() else None


def main():
    args = parse()
    if args.parse_pmc:
        parse_pmc(*args.parse_pmc, kernels=args.pmc_kernels)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              f"(this path has no multi-GPU part)", file=sys.stderr)
        sys.exit(2)
    if args.configs:
        for name in args.configs.split(","):
            name = name.strip()
            (append_line if name.endswith("a") else config_line)(name, args)
        return
    import numpy as np
    import torch

    import query_aware_sparse_min_amd as sa
    import synth

    if not os.path.exists(sa.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    sa.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    t0 = time.time()
    wl = synth.make_config(2)
    d = synth.to_device(wl, dev)
    kv0 = sa.KVCache(d.k, d.v)
    seqs = sa.Seqs(d.page_table, d.seq_lens)
    cfg = sa.SelectCfg(sa.SA_MODE_QUEST, 16, wl.k_compete, wl.n_head_forced, wl.n_tail_forced)
    R = max(1, args.copies)
    copies = []
    for r in range(R):
        k = d.k if r == 0 else d.k.clone()
        v = d.v if r == 0 else d.v.clone()
        kv = sa.KVCache(k, v)
        meta, _ = sa.alloc_meta(kv, cfg)
        sa.sa_build_page_meta(kv, seqs, cfg, meta)
        copies.append((kv, meta))
    NQ = 64
    qs = [synth.q_to_device(wl, synth.fresh_q(wl, i), dev) for i in range(NQ)]
    ws = sa.alloc_workspace(sa.sa_decode_step_workspace_size(wl.Hq, kv0, seqs, cfg), dev)
    out = torch.empty((wl.B, wl.Hq, wl.d), dtype=torch.float32, device=dev)
    ms = sa.sa_max_selected(seqs, cfg)
    torch.cuda.synchronize()
    setup_s = time.time() - t0

    def step(i):
        kv, meta = copies[i % R]
        sa.sa_decode_step(qs[i % NQ], kv, seqs, cfg, meta, None, wl.softmax_scale, out, ws)

    if args.pmc_run:  # a few eager steps on cold copies, then the calibration copy
        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        for i in range(4):
            step(args.warmup + i)
        src = torch.empty(CALIB_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print("pmc run done", flush=True)
        return

    stream = torch.cuda.current_stream()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # eager: one ctypes call per step, per-step events (includes host launch gaps if any)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    ev[0].record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]) * 1e3  # us
    eager_ms = ev[0].elapsed_time(ev[-1]) / args.steps
    # graph: the same K steps captured once and replayed, so the GPU never waits on Python
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            for i in range(args.steps):
                step(args.warmup + i)
    stream.wait_stream(cap)
    graph.replay()  # untimed replay (warm-up)
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    g0.record(stream)
    graph.replay()
    g1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = g0.elapsed_time(g1) / args.steps

    # algorithmic bytes: selection sizes are fixed by the budget (126 + 2 pages per head)
    num = torch.empty((wl.B, wl.Hkv), dtype=torch.int32, device=dev)
    sel = torch.empty((wl.B, wl.Hkv, ms), dtype=torch.int32, device=dev)
    kv, meta = copies[0]
    sa.sa_decode_step(qs[0], kv, seqs, cfg, meta, None, wl.softmax_scale, out, ws, sel, num)
    torch.cuda.synchronize()
    nb = synth.step_bytes(wl, num.cpu().numpy())
    step_gbs = nb["total"] / (ms_per_step * 1e-3) / 1e9

    # per-entry-point timing on the same stream (scorer / top-K / attention+merge)
    mu = sa.sa_max_units(seqs, cfg)
    scores = torch.empty((wl.B, wl.Hkv, mu), dtype=torch.float32, device=dev)
    sels = []
    for r in range(R):
        kv, meta = copies[r]
        s_r = torch.empty((wl.B, wl.Hkv, ms), dtype=torch.int32, device=dev)
        n_r = torch.empty((wl.B, wl.Hkv), dtype=torch.int32, device=dev)
        sa.sa_score_pages(qs[r], kv, seqs, cfg, meta, None, scores)
        sa.sa_topk_pages(scores, wl.Hkv, seqs, cfg, s_r, n_r)
        sels.append((s_r, n_r))
    aws = sa.alloc_workspace(sa.sa_attn_workspace_size(wl.B, wl.Hq, wl.Hkv, wl.max_pages, ms), dev)
    dws = sa.alloc_workspace(sa.sa_attn_workspace_size(wl.B, wl.Hq, wl.Hkv, wl.max_pages, 0), dev)
    torch.cuda.synchronize()

    def timed(fn, n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for i in range(min(n, 10)):
            fn(i)
        torch.cuda.synchronize()
        a.record(stream)
        for i in range(n):
            fn(i)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n * 1e3  # us per call

    n_k = max(args.steps, 50)
    score_us = timed(lambda i: sa.sa_score_pages(qs[i % R], copies[i % R][0], seqs, cfg,
                                                 copies[i % R][1], None, scores), n_k)
    topk_us = timed(lambda i: sa.sa_topk_pages(scores, wl.Hkv, seqs, cfg, sels[0][0], sels[0][1]), n_k)
    attn_us = timed(lambda i: sa.sa_sparse_decode_attn(qs[i % R], copies[i % R][0], seqs,
                                                       sels[i % R][0], sels[i % R][1],
                                                       wl.softmax_scale, out, aws), n_k)
    dense_us = timed(lambda i: sa.sa_sparse_decode_attn(qs[i % NQ], copies[i % R][0], seqs, None,
                                                        None, wl.softmax_scale, out, dws),
                     max(20, args.steps // 4))
    dense_bytes = synth.dense_bytes(wl)
    stream_gbs = stream_read_gbs(dev, stream)
    # the step is one persistent kernel (score -> top-K -> attention -> merge), so it is the
    # dominant kernel; its launch duration is the graph's per-step time
    dom_name = "quest_step_kernel (fused decode step)"
    dom_gbs = nb["total"] / (ms_per_step * 1e-3) / 1e9

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, args.cpu_seconds, nb["total"])

    rec = {
        "metric": METRIC,
        "value": round(step_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "input_dtype": "bf16",
        "data": "synthetic (seeded N(0,1) x per-channel U(0.5,2), 8 needles/head)",
        "config": {"workload": "Llama-7B-like layer decode, 32K context, 2048-token budget",
                   "batch": wl.B, "num_q_heads": wl.Hq, "num_kv_heads": wl.Hkv, "head_dim": wl.d,
                   "context": int(wl.seq_lens[0]), "page_size": 16, "budget_pages": ms,
                   "scoring": "quest min/max bound", "layer_copies_rotated": R},
        "step_us": round(ms_per_step * 1e3, 2),
        "timing": "HIP graph of the K steps, replayed once between two events",
        "eager_step_us": round(eager_ms * 1e3, 2),
        "eager_step_us_p10_p50_p90": [round(float(np.percentile(per, p)), 2) for p in (10, 50, 90)],
        "step_bytes": nb["total"],
        "hbm_peak_frac": round(step_gbs / PEAK_GBS, 4),
        "stream_read_gbs": round(stream_gbs, 1),
        "stream_read_frac": round(step_gbs / stream_gbs, 4),
        "dense_us": round(dense_us, 2),
        "dense_gbs": round(dense_bytes / (dense_us * 1e-6) / 1e9, 1),
        "speedup_vs_dense": round(dense_us / (ms_per_step * 1e3), 2),
        "separate_entry_points_us": {"score_pages": round(score_us, 2),
                                     "topk_pages": round(topk_us, 2),
                                     "sparse_decode_attn": round(attn_us, 2)},
        "roofline": {"bound": "hbm", "kernel": dom_name, "achieved": round(dom_gbs, 1),
                     "peak": PEAK_GBS, "unit": "GB/s", "frac": round(dom_gbs / PEAK_GBS, 4),
                     "traffic": load_traffic()},
        "cpu_baseline": cpu,
        "setup_s": round(setup_s, 1),
    }
    print(json.dumps(rec), flush=True)


CONFIG_COPIES_BYTES = 4 << 30  # layer copies rotated: at least this many bytes of K/V in all
STREAM_BYTES = 4 << 30         # streaming-read probe: 16x the 256 MB Infinity Cache


def stream_read_gbs(dev, stream, reps=8):
    """GB/s of one plain streaming read of STREAM_BYTES (sa_stream_read), the best of reps
    timed launches: the bandwidth a pure HBM read reaches on this device."""
    import torch

    import query_aware_sparse_min_amd as sa

    src = torch.ones(STREAM_BYTES // 4, dtype=torch.float32, device=dev)
    sink = torch.zeros(1 << 14, dtype=torch.int32, device=dev)
    for _ in range(2):
        sa.sa_stream_read(src, sink)
    torch.cuda.synchronize()
    best = None
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        sa.sa_stream_read(src, sink)
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        best = ms if best is None else min(best, ms)
    del src, sink
    torch.cuda.empty_cache()
    return STREAM_BYTES / (best * 1e-3) / 1e9


def config_line(name, args):
    """One workload at full size on one GPU: the decode step (graph of K steps over
    rotated layer copies, fresh query each), its algorithmic bytes and GB/s, and
    dense flash-decode over every page of the same copies for comparison."""
    import numpy as np
    import torch

    import query_aware_sparse_min_amd as sa
    import synth

    if not os.path.exists(sa.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    sa.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.time()
    print(f"[bench] config {name}: generating inputs", file=sys.stderr, flush=True)
    wl = synth.make_config(int(name[0]), dense=name.endswith("d"), probe="p" in name[1:])
    per_head = "h" in name[1:]
    if per_head:
        wl.name += "-per-head"
    d = synth.to_device(wl, dev)
    print(f"[bench] config {name}: inputs on the GPU after {time.time() - t0:.0f} s", file=sys.stderr,
          flush=True)
    seqs = sa.Seqs(d.page_table, d.seq_lens)
    mode = {"quest": sa.SA_MODE_QUEST, "sals": sa.SA_MODE_SALS, "probe": sa.SA_MODE_PROBE}[wl.mode]
    cfg = sa.SelectCfg(mode, wl.unit_tokens, wl.k_compete, wl.n_head_forced, wl.n_tail_forced,
                       wl.rank, d.proj, wl.lse_scale, wl.n_probe, 1 if per_head else 0)
    kv_bytes = d.k.numel() * d.k.element_size() * 2
    R = int(max(2, min(args.copies, -(-CONFIG_COPIES_BYTES // kv_bytes))))
    copies = []
    for r in range(R):
        k = d.k if r == 0 else d.k.clone()
        v = d.v if r == 0 else d.v.clone()
        kv = sa.KVCache(k, v, d.k_scale, d.v_scale)
        meta, mscale = sa.alloc_meta(kv, cfg)
        sa.sa_build_page_meta(kv, seqs, cfg, meta, mscale)
        copies.append((kv, meta, mscale))
    NQ = 16
    qs = [synth.q_to_device(wl, synth.fresh_q(wl, i), dev) for i in range(NQ)]
    ws = sa.alloc_workspace(sa.sa_decode_step_workspace_size(wl.Hq, copies[0][0], seqs, cfg), dev)
    out = torch.empty((wl.B, wl.Hq, wl.d), dtype=torch.float32, device=dev)
    ms = sa.sa_max_selected(seqs, cfg)
    setup_s = time.time() - t0
    stream = torch.cuda.current_stream()

    def step(i):
        kv, meta, mscale = copies[i % R]
        sa.sa_decode_step(qs[i % NQ], kv, seqs, cfg, meta, mscale, wl.softmax_scale, out, ws)

    if args.pmc_run:  # eager steps on rotated copies, then the calibration copy
        for i in range(args.warmup + 4):
            step(i)
        torch.cuda.synchronize()
        n_lists = wl.Hq if per_head else wl.Hkv
        num = torch.empty((wl.B, n_lists), dtype=torch.int32, device=dev)
        sel = torch.empty((wl.B, n_lists, ms), dtype=torch.int32, device=dev)
        kv, meta, mscale = copies[0]
        sa.sa_decode_step(qs[0], kv, seqs, cfg, meta, mscale, wl.softmax_scale, out, ws, sel, num)
        num_np = num.cpu().numpy()
        src = torch.empty(CALIB_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)  # the last copy dispatched: the calibration
        torch.cuda.synchronize()
        if not per_head:
            print(json.dumps({"workload": wl.name, "bytes": {k2: int(v2) for k2, v2 in
                                                             synth.step_bytes(wl, num_np).items()}}))
        print("pmc run done", flush=True)
        return

    def graph_us(fn, n):
        for i in range(min(n, args.warmup)):
            fn(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                for i in range(n):
                    fn(args.warmup + i)
        stream.wait_stream(cap)
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n * 1e3

    K = max(10, min(args.steps, 100))
    step_us = graph_us(step, K)
    n_lists = wl.Hq if per_head else wl.Hkv
    num = torch.empty((wl.B, n_lists), dtype=torch.int32, device=dev)
    sel = torch.empty((wl.B, n_lists, ms), dtype=torch.int32, device=dev)
    kv, meta, mscale = copies[0]
    sa.sa_decode_step(qs[0], kv, seqs, cfg, meta, mscale, wl.softmax_scale, out, ws, sel, num)
    torch.cuda.synchronize()
    if per_head:  # the attention reads each group's union of its heads' pages once
        sel_np, num_np = sel.cpu().numpy(), num.cpu().numpy()
        groups = np.array([[len(set().union(*[set(sel_np[b, h * wl.G + g, :num_np[b, h * wl.G + g]].tolist())
                                              for g in range(wl.G)])) for h in range(wl.Hkv)]
                           for b in range(wl.B)])
        nb = synth.step_bytes(wl, groups)
    else:
        nb = synth.step_bytes(wl, num.cpu().numpy())
    # the same step on the workload's own query (its needles are planted for it): recall
    sa.sa_decode_step(d.q, kv, seqs, cfg, meta, mscale, wl.softmax_scale, out, ws, sel, num)
    torch.cuda.synchronize()
    quality = selection_quality(wl, sel.cpu().numpy(), num.cpu().numpy())
    dws = sa.alloc_workspace(sa.sa_attn_workspace_size(wl.B, wl.Hq, wl.Hkv, wl.max_pages, 0), dev)
    dense_us = graph_us(lambda i: sa.sa_sparse_decode_attn(qs[i % NQ], copies[i % R][0], seqs, None,
                                                           None, wl.softmax_scale, out, dws),
                        max(10, K // 4))
    gbs = nb["total"] / (step_us * 1e-6) / 1e9
    dense_b = synth.dense_bytes(wl)
    rec = {
        "metric": f"decode-step µs + effective HBM GB/s, {wl.name}",
        "workload": wl.name, "batch": wl.B, "num_q_heads": wl.Hq, "num_kv_heads": wl.Hkv,
        "context": [int(x) for x in np.unique(wl.seq_lens)][:4], "kv_dtype": wl.kv_dtype,
        "scoring": {"quest": "quest min/max bound", "sals": "sals int4 index + block lse",
                    "probe": f"probe sampling, {wl.n_probe} keys per {wl.unit_tokens}-token block"}[wl.mode],
        "kept_units": int(wl.n_head_forced + wl.k_compete + wl.n_tail_forced),
        "step_us": round(step_us, 2), "step_bytes": nb["total"],
        "bytes": {k2: int(v2) for k2, v2 in nb.items()},
        "gbs": round(gbs, 1), "hbm_peak_frac": round(gbs / PEAK_GBS, 4),
        "dense_us": round(dense_us, 2),
        "dense_gbs": round(dense_b / (dense_us * 1e-6) / 1e9, 1),
        "speedup_vs_dense": round(dense_us / step_us, 2),
        "layer_copies_rotated": R, "steps": K, "setup_s": round(setup_s, 1), **quality,
        "timing": "HIP graph of K steps, replayed once between two events",
    }
    print(json.dumps(rec), flush=True)
    del copies, d, ws, dws
    torch.cuda.empty_cache()


def selection_quality(wl, sel, num):
    """Needle recall (share of the planted keys whose page the step kept) and top-10
    recall (share of each query head's ten largest exact logits q . k_t over the whole
    sequence whose page the step kept), from the page lists of a step run on the
    workload's own query.  The logits are scored on the host, so the top-10 figure is
    given only where B * Hq * L <= 2^24.  With one list per query head (per-head
    selection) each head is judged by its own list, and the pages the group reads (the
    union of its heads' lists) are reported relative to one list's length."""
    import numpy as np

    import synth

    per_head = sel.shape[1] == wl.Hq and wl.Hq != wl.Hkv
    lists = [[set(sel[b, i, :num[b, i]].tolist()) for i in range(sel.shape[1])] for b in range(wl.B)]

    def kept(b, head):  # the pages query head `head` attends over
        return lists[b][head] if per_head else lists[b][head // wl.G]

    res = {}
    if per_head:
        union = [len(set().union(*lists[b][h * wl.G:(h + 1) * wl.G])) for b in range(wl.B)
                 for h in range(wl.Hkv)]
        longest = [max(len(lists[b][h * wl.G + g]) for g in range(wl.G)) for b in range(wl.B)
                   for h in range(wl.Hkv)]
        res["union_pages_per_list"] = round(float(np.mean(np.array(union) / np.array(longest))), 3)
    if wl.needles:
        res["needle_recall"] = round(sum(1 for (b, h, p, s) in wl.needles if p in kept(b, h * wl.G)) /
                                     len(wl.needles), 4)
    if wl.kv_dtype != "i8" and wl.B * wl.Hq * int(wl.seq_lens.max()) <= 1 << 24:
        q = (synth.bf16_to_f32(wl.q) if wl.q_dtype == "bf16" else wl.q).astype(np.float32)
        hits = total = 0
        for b in range(wl.B):
            L = int(wl.seq_lens[b])
            t = np.arange(L)
            pp, sl = wl.page_table[b, t // 16], t % 16
            for h in range(wl.Hkv):
                kk = wl.k[pp, sl, h]
                kk = (synth.bf16_to_f32(kk) if wl.kv_dtype == "bf16" else kk).astype(np.float32)
                for g in range(wl.G):
                    z = kk @ q[b, h * wl.G + g]
                    top = np.argpartition(-z, 10)[:10] if L > 10 else t
                    hits += sum(1 for x in top if (x // 16) in kept(b, h * wl.G + g))
                    total += len(top)
        res["top10_recall"] = round(hits / total, 4)
    return res


def append_line(name, args):
    """The decode-time append (sa_append_kv) on a workload's full-size cache: one
    token per sequence written into its page plus the incremental metadata
    update, timed as a HIP graph of K appends.  The appended token is each
    sequence's current last token again, which leaves cache and metadata
    unchanged (the max/min fold and the index key are idempotent), so every
    replay does the same work.  Algorithmic bytes: the new K/V rows read and
    written (int8: and their scales), plus the page metadata read and written
    (Quest: the page's max and min rows) or written (SALS: codes and scale)."""
    import numpy as np
    import torch

    import query_aware_sparse_min_amd as sa
    import synth

    if not os.path.exists(sa.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    sa.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] append on config {name[0]}: generating inputs", file=sys.stderr, flush=True)
    wl = synth.make_config(int(name[0]))
    d = synth.to_device(wl, dev)
    seqs = sa.Seqs(d.page_table, d.seq_lens)
    mode = sa.SA_MODE_QUEST if wl.mode == "quest" else sa.SA_MODE_SALS
    cfg = sa.SelectCfg(mode, wl.unit_tokens, wl.k_compete, wl.n_head_forced, wl.n_tail_forced,
                       wl.rank, d.proj, wl.lse_scale)
    kv = sa.KVCache(d.k, d.v, d.k_scale, d.v_scale)
    meta, mscale = sa.alloc_meta(kv, cfg)
    sa.sa_build_page_meta(kv, seqs, cfg, meta, mscale)
    t = wl.seq_lens.astype(np.int64) - 1
    pp = torch.from_numpy(wl.page_table[np.arange(wl.B), t // 16].astype(np.int64)).to(dev)
    sl = torch.from_numpy((t % 16).astype(np.int64)).to(dev)
    new = {n: getattr(d, n)[pp, sl].contiguous() for n in ("k", "v", "k_scale", "v_scale")
           if getattr(d, n) is not None}

    def append(i):
        sa.sa_append_kv(new["k"], new["v"], kv, seqs, cfg, meta, mscale, new.get("k_scale"),
                        new.get("v_scale"))

    stream = torch.cuda.current_stream()
    K = max(10, min(args.steps, 200))
    for i in range(5):
        append(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            for i in range(K):
                append(i)
    stream.wait_stream(cap)
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) / K * 1e3
    es = {"f32": 4, "bf16": 2, "i8": 1}[wl.kv_dtype]
    row = wl.B * wl.Hkv * wl.d * es
    nbytes = 2 * 2 * row  # K and V rows: read from the new-token buffers, written into the cache
    if wl.kv_dtype == "i8":
        nbytes += 2 * 2 * wl.B * wl.Hkv * 2
    if wl.mode == "quest":
        nbytes += 2 * 2 * row  # the page's max and min rows, read and written
    else:
        nbytes += wl.B * wl.Hkv * (wl.rank // 2 + 2)  # codes and scale of the token
    rec = {
        "metric": f"decode-time append µs + effective HBM GB/s, {wl.name}",
        "workload": wl.name + "-append", "batch": wl.B, "num_kv_heads": wl.Hkv,
        "kv_dtype": wl.kv_dtype,
        "metadata": "quest min/max fold" if wl.mode == "quest" else "sals int4 index key",
        "append_us": round(us, 2), "append_bytes": int(nbytes),
        "gbs": round(nbytes / (us * 1e-6) / 1e9, 1), "steps": K,
        "timing": "HIP graph of K appends, replayed once between two events",
    }
    print(json.dumps(rec), flush=True)
    del d, kv, meta, mscale, new
    torch.cuda.empty_cache()


def host_description():
    """Host cores and CPU model of the machine the oracle runs on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    affinity = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return {"nproc": os.cpu_count(), "cores_available": affinity, "cpu_model": model}


def cpu_baseline(wl, seconds, step_bytes):
    """The oracle's decode step on the host, on fresh queries for about `seconds` per leg:
    single-threaded, then with its OpenMP outer loops (one (b, kv-head) list or query head per
    iteration) over the cores the process may use (OMP_NUM_THREADS caps them)."""
    import oracle
    import synth

    host = host_description()
    omp = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or host["cores_available"]
    omp = max(1, min(omp, host["cores_available"]))
    meta, _ = oracle.build_meta(wl)  # amortised, like the GPU's metadata build

    def leg(threads, first_q):
        oracle.set_threads(threads)
        n, t_used = 0, 0.0
        while n < 400 and (t_used < seconds or n == 0):
            q = synth.fresh_q(wl, first_q + n)
            t = time.perf_counter()
            oracle.decode_step(wl, meta, None, q=q)
            t_used += time.perf_counter() - t
            n += 1
        oracle.set_threads(1)
        per_step = t_used / n
        return {"value": round(step_bytes / per_step / 1e9, 4), "unit": "GB/s", "cores": threads,
                "step_ms": round(per_step * 1e3, 2), "steps": n}

    one = leg(1, 0)
    many = leg(omp, 1000)
    return {**many, "kind": "oracle",
            "sample": (f"{many['steps']} full decode steps of the same workload (all {wl.Hkv} lists), "
                       f"fresh query each, OpenMP over the lists on {omp} threads; a single-threaded "
                       f"leg of {one['steps']} steps is under single_thread"),
            "label": "plain double-precision oracle (not a tuned CPU implementation)",
            "single_thread": one, "host": host}


if __name__ == "__main__":
    main()
