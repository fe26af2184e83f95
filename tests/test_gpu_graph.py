"""HIP-graph capture of decode steps: a step (store of one new token per
sequence, then paged decode) for the three decode kernels (separate K/V on
the VALU path, a wide query group on the matrix-core path, the MLA slab with
its merge kernel) is captured once and replayed; every replay, with other
work and synchronizations between replays, must reproduce the eager outputs
bit for bit.  The library issues no memset and no allocation, so a captured
step holds only its own kernels; split-K arrival counters reset themselves
inside each call, which is what makes replays repeatable.
"""
import numpy as np
import pytest
import torch

from paged_decode_attention_amd import workloads as W
from tests.gpu_util import dev_bf16, dev_i32, kvq, requires_gpu, say

pytestmark = [pytest.mark.gpu, requires_gpu]


def layer(qtype, wl, strm):
    k = kvq()
    H, D = wl.n_kv_heads, wl.head_dim_qk
    slots = torch.arange(wl.n_slots, dtype=torch.int32, device="cuda")
    kp, ks = k.alloc_pool(qtype, wl.num_pages, H, D)
    if wl.shared:
        vp, vs = kp, ks
        k.store(qtype, dev_bf16(wl.kv_rows(0, 0, wl.n_slots)), None, slots, kp, ks)
    else:
        vp, vs = k.alloc_pool(qtype, wl.num_pages, H, D)
        k.store(qtype, dev_bf16(wl.kv_rows(0, 0, wl.n_slots)), dev_bf16(wl.kv_rows(1, 0, wl.n_slots)),
                slots, kp, ks, vp, vs)
    last = wl.seq_lens.astype(np.int64) - 1
    new_slots = dev_i32((wl.page_table[np.arange(wl.batch), last // W.PAGE].astype(np.int64) * W.PAGE
                         + last % W.PAGE).astype(np.int32))
    rng = np.random.default_rng(wl.seed)
    newk = dev_bf16(W.to_bf16_bits(rng.standard_normal((wl.batch, H, D), dtype=np.float32)))
    newv = None if wl.shared else dev_bf16(W.to_bf16_bits(
        rng.standard_normal((wl.batch, H, D), dtype=np.float32)))
    st = k.PreparedStore(qtype, newk, newv, new_slots, kp, ks, None if wl.shared else vp,
                         None if wl.shared else vs, stream=strm)
    dec = k.PreparedDecode(qtype, dev_bf16(wl.query()), kp, ks, vp, vs, dev_i32(wl.page_table),
                           dev_i32(wl.seq_lens), wl.sm_scale, head_dim_v=wl.head_dim_v, stream=strm)
    return st, dec


def test_captured_step_replays_match_eager():
    torch.cuda.synchronize()
    strm = torch.cuda.Stream()
    layers = [
        layer("fp8_e4m3", W.qwen3(batch=4, ctx=2048, replicas=1), strm),
        layer("q8_0", W.ragged256(batch=3, lo=600, hi=3000), strm),
        layer("fp8_e4m3", W.mla(ctx=5000, n_q_heads=64), strm),
    ]
    torch.cuda.synchronize()

    def step():
        for st, dec in layers:
            st()
            dec()

    say("graph: eager step")
    step()
    torch.cuda.synchronize()
    ref = [(dec.out.clone(), dec.lse.clone()) for _, dec in layers]
    for _, dec in layers:
        dec.out.zero_()
        dec.lse.zero_()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=strm):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        say("graph: replay", rep)
        graph.replay()
        torch.cuda.synchronize()
        for (o, l), (_, dec) in zip(ref, layers):
            assert torch.equal(dec.out, o) and torch.equal(dec.lse, l), rep
            dec.out.fill_(7)  # eager work between replays
        x = torch.randn(256, 256, device="cuda")
        (x @ x).sum().item()
        torch.cuda.synchronize()


def test_captured_extend_and_sparse_replay_match_eager():
    """Extend attention (split units merged by their last workgroup, whose
    arrival counters reset themselves) and the sparse MLA decode (the slab
    decode over the listed rows, then the merge) captured once and replayed:
    every replay reproduces the eager outputs bit for bit."""
    k = kvq()
    torch.cuda.synchronize()
    strm = torch.cuda.Stream()
    # extend: 3 sequences, long enough that units split into several items
    wl = W.qwen3(batch=3, ctx=6000, replicas=1)
    slots = torch.arange(wl.n_slots, dtype=torch.int32, device="cuda")
    kp, ks = k.alloc_pool("fp8_e4m3", wl.num_pages, 8, 128)
    vp, vs = k.alloc_pool("fp8_e4m3", wl.num_pages, 8, 128)
    k.store("fp8_e4m3", dev_bf16(wl.kv_rows(0, 0, wl.n_slots)), dev_bf16(wl.kv_rows(1, 0, wl.n_slots)),
            slots, kp, ks, vp, vs)
    news = np.array([20, 3, 40], np.int32)
    q_start = np.concatenate([[0], np.cumsum(news)]).astype(np.int32)
    ext = k.PreparedExtend("fp8_e4m3", dev_bf16(W.extend_queries(wl, int(q_start[-1]))),
                           dev_i32(q_start), int(news.max()), kp, ks, vp, vs,
                           dev_i32(wl.page_table), dev_i32(wl.seq_lens), wl.sm_scale, stream=strm)
    # sparse: 2 queries over an MLA slab
    ml = W.mla(ctx=3000, n_q_heads=64)
    mslots = torch.arange(ml.n_slots, dtype=torch.int32, device="cuda")
    sp, ss = k.alloc_pool("fp8_e4m3", ml.num_pages, 1, 576)
    k.store("fp8_e4m3", dev_bf16(ml.kv_rows(0, 0, ml.n_slots)), None, mslots, sp, ss)
    rng = np.random.default_rng(9)
    topk = np.stack([rng.choice(3000, 200, replace=False) for _ in range(1)]).astype(np.int32)
    spa = k.PreparedSparse("fp8_e4m3", dev_bf16(ml.query()), sp, ss, dev_i32(ml.page_table),
                           dev_i32(ml.seq_lens), dev_i32(topk), ml.sm_scale, stream=strm)
    calls = [ext, spa]
    torch.cuda.synchronize()
    say("graph: eager extend + sparse")
    for c in calls:
        c()
    torch.cuda.synchronize()
    ref = [(c.out.clone(), c.lse.clone()) for c in calls]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=strm):
        for c in calls:
            c()
    torch.cuda.synchronize()
    for rep in range(3):
        for c in calls:
            c.out.fill_(3)
            c.lse.zero_()
        torch.cuda.synchronize()
        say("graph: replay", rep)
        graph.replay()
        torch.cuda.synchronize()
        for (o, l), c in zip(ref, calls):
            assert torch.equal(c.out, o) and torch.equal(c.lse, l), rep
        x = torch.randn(256, 256, device="cuda")
        (x @ x).sum().item()
        torch.cuda.synchronize()
