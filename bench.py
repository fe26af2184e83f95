#!/usr/bin/env python3
"""Decode-step benchmark of the block-scaled 8-bit paged KV cache on one MI355X.

One step = one decode token for every sequence through a 28-layer attention
stack of the Qwen3-1.7B shape (16 query / 8 KV heads, head_dim 128): for each
layer, the quantize-on-store of the new token's K and V and paged decode
attention over that layer's pool, as one kvq_paged_decode_append call (one
kernel launch: the work item that attends the new position quantizes and
writes it), batch 8 x 16384-token contexts, page size 16, random-permutation
page tables, fp8_e4m3 block-32 codes with fp16 scales.  The same step as two
calls per layer (kvq_store, then kvq_paged_decode) is timed beside it.  The 28 layers are 28 distinct
copies of one layer's pool (7.99 GB in all), so every step streams the whole
KV cache from HBM rather than from the 256 MB Infinity Cache.

Prints one JSON line: `value` is the step's algorithmic bytes (codes + scales
of every token read, Q, O, page-table entries, and the store's bf16 reads and
code/scale writes) per second, in GB/s; `roofline` is the append-decode
call (one kernel launch: split-K decode with its in-kernel merge and the new
token's store) against the 8 TB/s HBM peak: its average launch duration from
HIP events around replays of the step's graph, which holds the 28 layers'
launches back to back (gaps between launches included), on the stream the
kernels run on; `decode_call_us` is kvq_paged_decode alone, timed the same
way; `store_gbps` is
the quantize-on-store at the mixed workload's size (8192 new tokens x 8 kv
heads x 128, K and V in one call), timed from graph replays as the decode;
`cpu_baseline` is the CPU oracle on a
bounded sample of the same workload (repeated layer decodes for about 10 s),
timed on this host.

Other modes: `--workload tiny|ragged256|single256|mla|mixed` times kvq_paged_decode
alone on that workload and prints its own line; `--workload mla_sparse` times
kvq_sparse_mla_decode (256 listed positions per query over the mla slab);
`--workload extend` times kvq_extend_attention (the last 64 of 8 x 16384
tokens new, causal); `--only decode|copy` and
`--traffic-from DIR` serve the rocprofv3 counter passes (see profiles/).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_GBPS = 8000.0
METRIC = "fp8 paged-decode effective HBM GB/s (% of peak) + store GB/s, 1 GPU"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# Sources whose change invalidates a recorded counter measurement.
KERNEL_SOURCES = ["paged_decode_attention_amd/csrc/kvq_decode.hip",
                  "paged_decode_attention_amd/csrc/kvq_attn.h",
                  "paged_decode_attention_amd/csrc/kvq_internal.h",
                  "paged_decode_attention_amd/csrc/kvq_device.h",
                  "paged_decode_attention_amd/csrc/kvq_api.cpp"]
TRAFFIC_FILE = "profiles/gqa_decode_qwen3_b8_ctx16384_fp8_traffic.json"


def recorded_traffic():
    """HBM bytes per decode launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE passes (scaled by a 1 GiB copy), or None when the kernel
    sources changed since they were taken."""
    import hashlib
    try:
        rec = json.load(open(os.path.join(ROOT, TRAFFIC_FILE)))
        h = hashlib.sha256()
        for f in KERNEL_SOURCES:
            h.update(open(os.path.join(ROOT, f), "rb").read())
    except OSError:
        return None
    if h.hexdigest()[:16] != rec.get("source_hash"):
        return None
    return rec["traffic_bytes_per_launch"]


def _counter_means(path, name_re):
    """Per-dispatch sums of each counter (all instances) in a rocprofv3
    counter_collection.csv, averaged over the dispatches whose kernel name
    matches name_re."""
    import csv
    import re
    per = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if not re.search(name_re, r["Kernel_Name"]):
                continue
            key = (r["Dispatch_Id"], r["Counter_Name"])
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (d, c), v in per.items():
        out.setdefault(c, []).append(v)
    return {c: sum(v) / len(v) for c, v in out.items()}


def write_traffic(src_dir):
    """Turn four rocprofv3 --pmc runs (FETCH_SIZE and WRITE_SIZE, each over the
    decode launches and over a plain 1 GiB copy) into TRAFFIC_FILE: HBM bytes
    per decode launch, with the counters scaled by what they read for the copy
    of known size, tagged with the kernel sources' hash."""
    import hashlib
    j = os.path.join
    dec_f = _counter_means(j(src_dir, "decode_FETCH_SIZE", "run_counter_collection.csv"),
                           "gqa_decode_kernel")["FETCH_SIZE"]
    dec_w = _counter_means(j(src_dir, "decode_WRITE_SIZE", "run_counter_collection.csv"),
                           "gqa_decode_kernel")["WRITE_SIZE"]
    cp_f = _counter_means(j(src_dir, "copy_FETCH_SIZE", "run_counter_collection.csv"),
                          "(?i)copy")["FETCH_SIZE"]
    cp_w = _counter_means(j(src_dir, "copy_WRITE_SIZE", "run_counter_collection.csv"),
                          "(?i)copy")["WRITE_SIZE"]
    gib = float(1 << 30)
    ff, fw = gib / (cp_f * 1024), gib / (cp_w * 1024)
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    rec = {
        "kernel": "gqa_decode_kernel<fp8_e4m3, 128, 2, append> (kvq_paged_decode_append)",
        "workload": "qwen3_b8_ctx16384_h16x8_d128 (one layer's pool, batch 8 x 16384 tokens)",
        "source_hash": h.hexdigest()[:16],
        "fetch_size_kib": round(dec_f, 1),
        "write_size_kib": round(dec_w, 1),
        "copy_reference": {"bytes_read": 1 << 30, "bytes_written": 1 << 30,
                           "fetch_size_kib": round(cp_f, 1), "write_size_kib": round(cp_w, 1)},
        "fetch_factor": round(ff, 4),
        "write_factor": round(fw, 4),
        "traffic_bytes_per_launch": int(round(dec_f * 1024 * ff + dec_w * 1024 * fw)),
    }
    with open(os.path.join(ROOT, TRAFFIC_FILE), "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))
    return 0


def store_bytes(n_tokens, n_heads, head_dim, qtype, tensors=2):
    per = {"bf16": 2.0, "fp8_e4m3": 1 + 1 / 16, "q8_0": 1 + 1 / 16, "fp8_e4m3_cast": 1.0,
           "fp8_e5m2_cast": 1.0, "fp8_ds_mla": 656 / 576}[qtype]
    return int(tensors * n_tokens * n_heads * head_dim * (2 + per)) + 4 * n_tokens


CPU_SAMPLE_S = 10.0  # seconds of oracle decode timed (at least one full layer)


def cpu_baseline(wl, qtype, k_rows, v_rows, q_bits):
    """The oracle, as it stands, on the workload: store every slot of one
    layer's pool, then decode all rows of that layer repeatedly (each pass is
    one of the step's 28 layer decodes) until CPU_SAMPLE_S seconds have
    passed.  Reports the decode part in GB/s over the same algorithmic bytes
    as the GPU line."""
    import oracle
    from paged_decode_attention_amd import workloads as W
    threads = oracle.default_threads()
    H, D = wl.n_kv_heads, wl.head_dim_qk
    slots = np.arange(wl.n_slots, dtype=np.int32)
    code_t = np.uint16 if qtype == "bf16" else np.uint8
    kp = np.zeros((wl.num_pages, H, W.PAGE, D), code_t)
    vp = np.zeros_like(kp)
    ks = (np.zeros((wl.num_pages, H, W.PAGE, D // 32), np.uint16) if qtype in oracle.SCALED
          else None)
    vs = None if ks is None else np.zeros_like(ks)
    t0 = time.perf_counter()
    oracle.store(qtype, k_rows, slots, H, D, W.PAGE, wl.num_pages, kp, ks, threads=threads)
    oracle.store(qtype, v_rows, slots, H, D, W.PAGE, wl.num_pages, vp, vs, threads=threads)
    t1 = time.perf_counter()
    passes = 0
    while True:
        oracle.paged_decode(qtype, q_bits, kp, ks, vp, vs, wl.page_table, wl.seq_lens, H, D, D,
                            W.PAGE, wl.num_pages, wl.sm_scale, threads=threads)
        passes += 1
        t2 = time.perf_counter()
        if t2 - t1 >= CPU_SAMPLE_S:
            break
    dec_bytes = wl.algorithmic_bytes(qtype) * passes
    fill_bytes = store_bytes(wl.n_slots, H, D, qtype)
    return {
        "value": round(dec_bytes / (t2 - t1) / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": ("%d layer decodes (of the step's 28) of all %d sequences x %d heads over "
                   "%d tokens each: %.2f s, %.1f MB algorithmic; the oracle's fill of that "
                   "layer's pool took %.3f s (%.3f GB/s)" % (
                       passes, wl.batch, wl.n_q_heads, int(wl.seq_lens[0]), t2 - t1,
                       dec_bytes / 1e6, t1 - t0, fill_bytes / (t1 - t0) / 1e9)),
    }


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak


def arith_dtype(qtype: str) -> str:
    """What the path computes in: the stored codes meet bf16 queries as bf16
    operands (dot2 / MFMA) with fp32 accumulation and an fp32 softmax."""
    return "bf16 operands, fp32 accumulation (%s storage)" % qtype


def median_of_means(elapsed_ms, counts):
    """Median over groups of (milliseconds, calls) of the per-call mean."""
    means = sorted(t / n for t, n in zip(elapsed_ms, counts))
    return means[len(means) // 2]


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def timed_replays(graph, n_replays, groups=5):
    """Replay `graph` n_replays times split into `groups` runs, each between
    two HIP events on the current stream; returns (median per-replay ms,
    list of the group means)."""
    import torch
    groups = max(1, min(groups, n_replays))
    sizes = [n_replays // groups + (1 if i < n_replays % groups else 0) for i in range(groups)]
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in sizes]
    torch.cuda.synchronize()
    for (e0, e1), n in zip(ev, sizes):
        e0.record()
        for _ in range(n):
            graph.replay()
        e1.record()
    torch.cuda.synchronize()
    ms = [e0.elapsed_time(e1) for e0, e1 in ev]
    return median_of_means(ms, sizes), [round(t / n, 5) for t, n in zip(ms, sizes)]


SPARSE_K = 256  # tokens listed per query by the sparse MLA workload


def decode_only(args, wl, qtype, dev, sparse_k=0) -> int:
    """Time kvq_paged_decode alone on `wl`, sweeping pool replicas so that
    each call reads its KV from HBM, and print one JSON line.  sparse_k > 0:
    time kvq_sparse_mla_decode over the slab instead, each query listing
    sparse_k distinct random positions of its sequence, the calls of all
    replicas captured in one HIP graph (a call takes microseconds)."""
    import torch
    from paged_decode_attention_amd import kvq
    from paged_decode_attention_amd import workloads as W

    H, D, Dv = wl.n_kv_heads, wl.head_dim_qk, wl.head_dim_v
    one = kvq.pool_bytes(qtype, wl.num_pages, W.PAGE, H, D)[0] * (1 if wl.shared else 2)
    R = args.replicas or max(1, min(16, -(-(1 << 30) // one)))
    log("workload", wl.name, "qtype", qtype, "replicas", R, "pool bytes", one)

    def dev_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(
            torch.bfloat16)

    pools = []
    for _ in range(R):
        kp, ks = kvq.alloc_pool(qtype, wl.num_pages, H, D, device=dev)
        if wl.shared:
            pools.append((kp, ks, kp, ks))
        else:
            vp, vs = kvq.alloc_pool(qtype, wl.num_pages, H, D, device=dev)
            pools.append((kp, ks, vp, vs))
    # fill every slot of every replica, 2^17 slots at a time
    step = 1 << 17
    for lo in range(0, wl.n_slots, step):
        hi = min(lo + step, wl.n_slots)
        slots = torch.arange(lo, hi, dtype=torch.int32, device=dev)
        d_k = dev_bf16(wl.kv_rows(0, lo, hi))
        d_v = None if wl.shared else dev_bf16(wl.kv_rows(1, lo, hi))
        for kp, ks, vp, vs in pools:
            if wl.shared:
                kvq.store(qtype, d_k, None, slots, kp, ks)
            else:
                kvq.store(qtype, d_k, d_v, slots, kp, ks, vp, vs)
        torch.cuda.synchronize()
    del d_k, d_v, slots
    q = dev_bf16(wl.query())
    pt = torch.from_numpy(wl.page_table).to(dev)
    sl = torch.from_numpy(wl.seq_lens).to(dev)
    ws = None
    calls = []
    if sparse_k:
        rng = np.random.default_rng(sparse_k)
        topk_np = np.stack([rng.choice(int(L), sparse_k, replace=False) for L in wl.seq_lens])
        topk = torch.from_numpy(topk_np.astype(np.int32)).to(dev)
        # the calls are bound to the stream the graph captures
        strm = torch.cuda.Stream(device=dev)
        for kp, ks, _, _ in pools:
            d = kvq.PreparedSparse(qtype, q, kp, ks, pt, sl, topk, wl.sm_scale, workspace=ws,
                                   stream=strm)
            ws = d.workspace
            calls.append(d)
        return sparse_timing(args, wl, qtype, calls, topk_np, strm)
    if "q_start" in wl.new_tokens:
        q_start_np = wl.new_tokens["q_start"]
        T = int(q_start_np[-1])
        qx = dev_bf16(W.extend_queries(wl, T))
        qs = torch.from_numpy(q_start_np).to(dev)
        max_new = int(np.diff(q_start_np).max())
        strm = torch.cuda.Stream(device=dev)
        for kp, ks, vp, vs in pools:
            d = kvq.PreparedExtend(qtype, qx, qs, max_new, kp, ks, vp, vs, pt, sl, wl.sm_scale,
                                   workspace=ws, stream=strm)
            ws = d.workspace
            calls.append(d)
        return extend_timing(args, wl, qtype, calls, q_start_np, strm)
    # a call of the 1024-token correctness shape takes a few microseconds, less
    # than the host needs to issue it: its calls are timed as graph replays
    short = wl.name.startswith("tiny")
    strm = torch.cuda.Stream(device=dev) if short else None
    for kp, ks, vp, vs in pools:
        d = kvq.PreparedDecode(qtype, q, kp, ks, vp, vs, pt, sl, wl.sm_scale, head_dim_v=Dv,
                               workspace=ws, stream=strm)
        ws = d.workspace
        calls.append(d)
    if short and args.only is None:
        us = replay_us(args, calls, strm)
        nbytes = wl.algorithmic_bytes(qtype)
        print(json.dumps({
            "metric": "paged-decode call time, 1 GPU (decode only)", "value": round(us, 3),
            "unit": "us", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "higher_is_better": False, "dtype": arith_dtype(qtype), "data": "synthetic",
            "config": {"workload": wl.name, "kv_storage": qtype, "replicas": R},
            "timing": "graph replays of every replica's call, median of 5 group means",
            "decode_call_us": round(us, 3),
            "gbps": round(nbytes / (us * 1e-6) / 1e9, 2),
            "algorithmic_bytes_per_call": nbytes}), flush=True)
        return 0
    for _ in range(args.warmup):
        for c in calls:
            c()
    torch.cuda.synchronize()
    if args.only == "decode":
        for _ in range(args.steps):
            for c in calls:
                c()
        torch.cuda.synchronize()
        log("ran %d decode calls" % (args.steps * R))
        return 0
    K = args.steps
    # 5 runs of K sweeps over the replicas, an event pair around each run:
    # the median run's mean per call
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(5)]
    for e0, e1 in ev:
        e0.record()
        for _ in range(K):
            for c in calls:
                c()
        e1.record()
    torch.cuda.synchronize()
    us = median_of_means([e0.elapsed_time(e1) for e0, e1 in ev], [K * R] * 5) * 1e3
    nbytes = wl.algorithmic_bytes(qtype)
    n_tok = int(np.minimum(wl.seq_lens, wl.max_pages * W.PAGE).sum())
    res = {
        "metric": "paged-decode effective HBM GB/s, 1 GPU (decode only)",
        "value": round(nbytes / (us * 1e-6) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "higher_is_better": True,
        "dtype": arith_dtype(qtype),
        "data": "synthetic",
        "config": {"workload": wl.name, "kv_storage": qtype, "replicas": R},
        "decode_call_us": round(us, 3),
        "pct_of_hbm_peak": round(100 * nbytes / (us * 1e-6) / 1e9 / PEAK_GBPS, 2),
        "algorithmic_bytes_per_call": nbytes,
    }
    if wl.shared:
        flops = 2.0 * wl.n_q_heads * n_tok * (D + Dv)
        tf = flops / (us * 1e-6) / 1e12
        res["tflops"] = round(tf, 1)
        res["mfma_frac"] = round(tf / MFMA_BF16_PEAK_TFLOPS, 4)
        res["t_roof_us"] = round(max(nbytes / PEAK_GBPS / 1e3, flops / MFMA_BF16_PEAK_TFLOPS / 1e6), 3)
    print(json.dumps(res), flush=True)
    return 0


def replay_us(args, calls, strm) -> float:
    """Microseconds per call: every call (bound to stream strm) captured back
    to back in one graph, replayed args.steps times between two HIP events."""
    import torch
    for _ in range(args.warmup):
        for c in calls:
            c()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=strm):
        for c in calls:
            c()
    for _ in range(args.warmup):
        graph.replay()
    ms, _ = timed_replays(graph, 5 * args.steps)
    return ms * 1e3 / len(calls)


def extend_timing(args, wl, qtype, calls, q_start, strm) -> int:
    """Causal extend attention of every sequence's new tokens over the pool."""
    from paged_decode_attention_amd import kvq
    from paged_decode_attention_amd import workloads as W
    us = replay_us(args, calls, strm)
    H, D, Dv, Hq = wl.n_kv_heads, wl.head_dim_qk, wl.head_dim_v, wl.n_q_heads
    E = np.diff(q_start).astype(np.int64)
    T = int(q_start[-1])
    # algorithmic bytes: every sequence's K and V rows once, its page-table
    # entries, the new tokens' Q and O, seq_lens and q_start
    per_tok = kvq.pool_bytes(qtype, 1, W.PAGE, H, D)[0] / W.PAGE * (1 if wl.shared else 2)
    tokens = int(wl.seq_lens.astype(np.int64).sum())
    nbytes = (tokens * per_tok + 4 * sum((int(L) + W.PAGE - 1) // W.PAGE for L in wl.seq_lens)
              + T * Hq * (D + Dv) * 2 + 4 * wl.batch + 4 * (wl.batch + 1))
    # flops: each new token attends to its position + 1 rows, 2 D flops per
    # row for q.k and 2 D for p.v, per query head
    vis = sum(int(np.sum(int(L) - e + np.arange(e) + 1)) for L, e in zip(wl.seq_lens, E))
    flops = 2.0 * (D + Dv) * Hq * vis
    t_roof = max(nbytes / 8e12, flops / 2.5e15) * 1e6
    res = {
        "metric": "extend attention call time, 1 GPU",
        "value": round(us, 3),
        "unit": "us",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "higher_is_better": False,
        "dtype": arith_dtype(qtype),
        "data": "synthetic",
        "config": {"workload": "%s: %d sequences x %d tokens, the last %d of each new (causal), "
                               "%d q / %d kv heads, head_dim %d/%d" % (
                                   wl.name, wl.batch, int(wl.seq_lens.max()), int(E.max()), Hq,
                                   H, D, Dv),
                   "kv_storage": qtype, "replicas": len(calls)},
        "call_us": round(us, 3),
        "gbps": round(nbytes / (us * 1e-6) / 1e9, 2),
        "tflops": round(flops / (us * 1e-6) / 1e12, 2),
        "t_roof_us": round(t_roof, 3),
        "roof_frac": round(t_roof / us, 4),
        "algorithmic_bytes_per_call": int(nbytes),
        "flops_per_call": flops,
    }
    print(json.dumps(res), flush=True)
    return 0


def sparse_timing(args, wl, qtype, calls, topk_np, strm) -> int:
    """Replays of one graph holding every replica's sparse call, timed by HIP
    events around the replays (which run on the current stream)."""
    import torch
    for _ in range(args.warmup):
        for c in calls:
            c()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=strm):
        for c in calls:
            c()
    for _ in range(args.warmup):
        graph.replay()
    K, R = args.steps, len(calls)
    ms, _ = timed_replays(graph, 5 * K)
    us = ms * 1e3 / R
    # algorithmic bytes: the listed rows (codes + scales), their page-table
    # entries, the lists, seq_lens, Q and O
    per_row = {"bf16": 2 * 576, "fp8_e4m3": 612, "q8_0": 612, "fp8_e4m3_cast": 576,
               "fp8_e5m2_cast": 576, "fp8_ds_mla": 656}[qtype]
    n = topk_np.size
    nbytes = (n * (per_row + 4 + 4) + 4 * wl.batch +
              wl.batch * wl.n_q_heads * (wl.head_dim_qk + wl.head_dim_v) * 2)
    flops = 2.0 * wl.n_q_heads * n * (wl.head_dim_qk + wl.head_dim_v)
    res = {
        "metric": "sparse top-k MLA decode call time, 1 GPU",
        "value": round(us, 3),
        "unit": "us",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "higher_is_better": False,
        "dtype": arith_dtype(qtype),
        "data": "synthetic",
        "config": {"workload": "sparse top-%d decode over the %s slab (%d queries x %d heads, "
                               "%d distinct random positions each)" % (
                                   topk_np.shape[1], wl.name, wl.batch, wl.n_q_heads,
                                   topk_np.shape[1]),
                   "kv_storage": qtype, "replicas": R},
        "call_us": round(us, 3),
        "gbps": round(nbytes / (us * 1e-6) / 1e9, 2),
        "tflops": round(flops / (us * 1e-6) / 1e12, 2),
        "algorithmic_bytes_per_call": int(nbytes),
    }
    print(json.dumps(res), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # untimed replays before each timed phase: after the host-synchronised
    # eager phase the first ~15 graph replays of the step ran 3-4% slow, so
    # five left the first timed group of the default 20 steps slow
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--qtype", default="fp8_e4m3",
                    choices=["fp8_e4m3", "q8_0", "bf16", "fp8_e4m3_cast", "fp8_e5m2_cast",
                             "fp8_ds_mla"])
    ap.add_argument("--layers", type=int, default=28)
    ap.add_argument("--extend-new", type=int, default=64,
                    help="--workload extend: new tokens per sequence")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default="qwen3",
                    choices=["qwen3", "tiny", "ragged256", "single256", "mla", "mixed", "mla_sparse",
                             "extend", "mla_extend"],
                    help="qwen3 (default) is the decode step this benchmark reports; the others "
                         "time kvq_paged_decode alone on that workload and print their own line")
    ap.add_argument("--ctx", type=int, default=0,
                    help="--workload mla: tokens of the sequence (0: the workload's 163840)")
    ap.add_argument("--replicas", type=int, default=0,
                    help="pool copies swept by the decode-only workloads (0: enough for 1 GB)")
    ap.add_argument("--traffic-from", default=None, metavar="DIR",
                    help="write the decode kernel's HBM traffic record from rocprofv3 --pmc "
                         "FETCH_SIZE / WRITE_SIZE runs under DIR (decode_* and copy_*) and exit")
    ap.add_argument("--only", choices=["decode", "copy"], default=None,
                    help="counter passes: run just the timed decode calls, or a plain "
                         "1 GiB device copy (the reference for scaling FETCH_SIZE/WRITE_SIZE)")
    args = ap.parse_args()
    if args.traffic_from:
        return write_traffic(args.traffic_from)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this path has no multi-GPU form (each GPU would "
              "run the same kernels on its own sequences or KV heads); run with --gpus 1",
              file=sys.stderr)
        return 2

    import torch
    from paged_decode_attention_amd import kvq
    from paged_decode_attention_amd import workloads as W

    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    qtype = args.qtype
    if args.only == "copy":
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copied %d x %d bytes" % (args.steps, src.numel()))
        return 0
    if args.workload == "mla_sparse":
        return decode_only(args, W.mla(), qtype, dev, sparse_k=SPARSE_K)
    if args.workload == "extend":
        return decode_only(args, W.extend(new=args.extend_new), qtype, dev)
    if args.workload == "mla_extend":
        return decode_only(args, W.mla_extend(new=args.extend_new), qtype, dev)
    if args.workload == "mla" and args.ctx:
        return decode_only(args, W.mla(ctx=args.ctx), qtype, dev)
    if args.workload != "qwen3":
        return decode_only(args, W.BY_NAME[args.workload](), qtype, dev)
    wl = W.qwen3(replicas=args.layers)
    L, B, H, D = wl.layer_replicas, wl.batch, wl.n_kv_heads, wl.head_dim_qk
    log("workload", wl.name, "layers", L, "qtype", qtype)

    # ---- inputs, resident in HBM before timing ---------------------------------------
    k_rows = wl.kv_rows(0, 0, wl.n_slots)
    v_rows = wl.kv_rows(1, 0, wl.n_slots)
    q_bits = wl.query()

    def dev_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(
            torch.bfloat16)

    d_k, d_v = dev_bf16(k_rows), dev_bf16(v_rows)
    d_slots = torch.arange(wl.n_slots, dtype=torch.int32, device=dev)
    pools = []
    for layer in range(L):
        kp, ks = kvq.alloc_pool(qtype, wl.num_pages, H, D, device=dev)
        vp, vs = kvq.alloc_pool(qtype, wl.num_pages, H, D, device=dev)
        kvq.store(qtype, d_k, d_v, d_slots, kp, ks, vp, vs)
        pools.append((kp, ks, vp, vs))
    torch.cuda.synchronize()
    del d_k, d_v, d_slots
    q = dev_bf16(q_bits)
    pt = torch.from_numpy(wl.page_table).to(dev)
    sl = torch.from_numpy(wl.seq_lens).to(dev)
    # the new token of each sequence is its last position; K/V rows per layer
    rng = np.random.Generator(np.random.PCG64([wl.seed, 55]))
    last = wl.seq_lens.astype(np.int64) - 1
    new_slots = torch.from_numpy(
        (wl.page_table[np.arange(B), last // W.PAGE].astype(np.int64) * W.PAGE + last % W.PAGE)
        .astype(np.int32)).to(dev)
    new_kv = [dev_bf16(W.to_bf16_bits(rng.standard_normal((2, B, H, D), dtype=np.float32)))
              for _ in range(L)]
    ws = None
    # every call goes to one stream of the default priority, which a HIP graph
    # can capture
    strm = torch.cuda.Stream(device=dev)
    stores, decodes, appends = [], [], []
    for layer in range(L):
        kp, ks, vp, vs = pools[layer]
        stores.append(kvq.PreparedStore(qtype, new_kv[layer][0], new_kv[layer][1], new_slots,
                                        kp, ks, vp, vs, stream=strm))
        d = kvq.PreparedDecode(qtype, q, kp, ks, vp, vs, pt, sl, wl.sm_scale, workspace=ws,
                               stream=strm)
        ws = d.workspace
        decodes.append(d)
        # the layer's step: store the new token and decode, one launch
        appends.append(kvq.PreparedDecode(qtype, q, kp, ks, vp, vs, pt, sl, wl.sm_scale,
                                          workspace=ws, stream=strm, new_k=new_kv[layer][0],
                                          new_v=new_kv[layer][1]))

    dec_bytes = wl.algorithmic_bytes(qtype)
    st_bytes = store_bytes(B, H, D, qtype)
    step_bytes = L * (dec_bytes + st_bytes)

    def step(ev=None, s=None):
        for layer in range(L):
            if ev is not None:
                ev[s][layer][0].record(strm)
            appends[layer]()
            if ev is not None:
                ev[s][layer][1].record(strm)

    def step_two_calls():
        for layer in range(L):
            stores[layer]()
            decodes[layer]()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.only == "decode":
        for s_ in range(args.steps):
            step()
        torch.cuda.synchronize()
        log("ran %d append-decode calls" % (args.steps * L))
        return 0

    K = args.steps
    # (1) each call timed on its own with HIP events on the stream it runs on
    ev = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(L)]
          for _ in range(K)]
    torch.cuda.synchronize()
    for s in range(K):
        step(ev, s)
    torch.cuda.synchronize()
    app_avg = float(np.mean([ev[s][l][0].elapsed_time(ev[s][l][1]) for s in range(K)
                             for l in range(L)]))
    # (2) the step as a serving loop runs it: captured once into a HIP graph
    # (every layer's append-decode, nothing else) and replayed K times
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=strm):
        step()
    for _ in range(args.warmup):
        graph.replay()
    # exactly K steps, in 5 groups (one event pair each): the median group mean
    ms_step, step_means = timed_replays(graph, K)
    value = step_bytes / (ms_step * 1e-3) / 1e9
    # (2a) the same step as two calls per layer (kvq_store, then kvq_paged_decode)
    graph2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph2, stream=strm):
        step_two_calls()
    for _ in range(args.warmup):
        graph2.replay()
    ms_step2, _ = timed_replays(graph2, K)
    # (2b) kvq_paged_decode alone: the L layers' decodes captured back to back
    # into one graph, replayed between two events on their stream (gaps
    # between launches included; no event between two launches).  The
    # roofline's kernel is the step's own launch (the step graph above holds
    # exactly L of them back to back); this is the decode without the store.
    dgraph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(dgraph, stream=strm):
        for layer in range(L):
            decodes[layer]()
    for _ in range(args.warmup):
        dgraph.replay()
    # 5 runs of K replays: the median run's mean
    dg_ms, dec_means = timed_replays(dgraph, 5 * K)
    dec_graph = dg_ms / L  # ms per decode launch
    # (3) the store at the mixed workload's size: 8192 new tokens (the last 128
    # of 64 sequences) x 8 kv heads x 128, K and V in one fused kvq_store into
    # a 2^20-slot pool, timed alone: 8 calls captured back to back in one
    # graph (eager calls would time the host's launch rate), replayed K times
    # between two HIP events
    mw = W.mixed()
    new = dev_bf16(mw.new_rows())
    mkp, mks = kvq.alloc_pool(qtype, mw.num_pages, H, D, device=dev)
    mvp, mvs = kvq.alloc_pool(qtype, mw.num_pages, H, D, device=dev)
    mslots = torch.from_numpy(mw.new_tokens["slots"]).to(dev)
    big = kvq.PreparedStore(qtype, new[0], new[1], mslots, mkp, mks, mvp, mvs, stream=strm)
    for _ in range(args.warmup):
        big()
    torch.cuda.synchronize()
    sgraph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(sgraph, stream=strm):
        for _ in range(8):
            big()
    for _ in range(args.warmup):
        sgraph.replay()
    sg_ms, _ = timed_replays(sgraph, 5 * K)
    big_us = sg_ms * 1e3 / 8
    big_bytes = store_bytes(int(mslots.numel()), H, D, qtype)
    app_graph = ms_step / L  # ms per append-decode launch in the step's graph
    achieved = (dec_bytes + st_bytes) / (app_graph * 1e-3) / 1e9
    log("step %.3f ms (graph; %.3f ms as store + decode calls), append-decode launch %.2f us "
        "(%.2f us with an event pair around each eager call), decode alone %.2f us"
        % (ms_step, ms_step2, app_graph * 1e3, app_avg * 1e3, dec_graph * 1e3))

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": arith_dtype(qtype),
        "data": "synthetic",
        "config": {
            "workload": "decode step (replayed as one HIP graph), %d layers x (store 1 new token "
                        "+ paged decode, one kvq_paged_decode_append launch), batch %d "
                        "x %d-token contexts, %d q / %d kv heads, head_dim %d, page 16, "
                        "random-permutation page tables (%s)" % (L, B, int(wl.seq_lens[0]),
                                                                 wl.n_q_heads, H, D, wl.name),
            "kv_storage": qtype + (", fp16 scale per 32 elements" if qtype in ("fp8_e4m3", "q8_0")
                                   else "" if qtype == "bf16" else ", per-tensor scale 1.0"),
            "layers": L,
            "batch": B,
            "context": int(wl.seq_lens[0]),
            "kv_bytes_per_step": L * dec_bytes,
        },
        "pct_of_peak": round(100 * value / PEAK_GBPS, 2),
        "tokens_per_s": round(B / (ms_step * 1e-3), 1),
        "timing": "median of 5 group means (HIP events on the stream around graph replays): "
                  "the step over exactly %d steps (the two-call step likewise); the decode "
                  "alone and the store over 5 x %d replays" % (K, K),
        "step_ms_group_means": step_means,
        "step_ms_store_then_decode": round(ms_step2, 4),
        "append_call_us": round(app_graph * 1e3, 3),
        "append_call_us_eager_events": round(app_avg * 1e3, 3),
        "decode_call_us": round(dec_graph * 1e3, 3),
        "store_gbps": round(big_bytes / (big_us * 1e-6) / 1e9, 2),
        "store": {"workload": "8192 new tokens x 8 kv heads x 128, K and V in one call, into a "
                              "2^20-slot pool (mixed_b64 new tokens: zero and constant blocks, "
                              "+-1e4 outliers)",
                  "call_us": round(big_us, 3), "bytes": big_bytes,
                  "gbps": round(big_bytes / (big_us * 1e-6) / 1e9, 2),
                  "pct_of_hbm_peak": round(100 * big_bytes / (big_us * 1e-6) / 1e9 / PEAK_GBPS, 2)},
        "roofline": {
            "bound": "hbm",
            "kernel": "gqa_decode_kernel<%s, 128, 2, append> (one launch per "
                      "kvq_paged_decode_append: the layer's decode and its new token's store)"
                      % qtype,
            "achieved": round(achieved, 2),
            "peak": PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_GBPS, 4),
            "traffic": recorded_traffic() if qtype == "fp8_e4m3" and L == 28 else None,
            "algorithmic_bytes_per_launch": dec_bytes + st_bytes,
        },
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        res["cpu_baseline"] = cpu_baseline(wl, qtype, k_rows, v_rows, q_bits)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
