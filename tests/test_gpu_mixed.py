"""Mixed store + decode at full size: quantize-on-store of 8192 new tokens
(with all-zero blocks, constant blocks and +-1e4 outliers) into a 2^20-token
pool, then paged decode of 64 sequences with log-uniform contexts in
[1024, 131072], -1 masked page-table columns and pages shared between
sequences.

The background rows of every page the batch reads are drawn per page
(Workload.page_rows) and stored on both sides; the new tokens' codes and
scales must match the oracle's bit for bit, and the decode of all 64
sequences within the attention tolerance.

Page keys: [PR103] "feat(kvcache): 8-bit KV cache (q8_0 / fp8_e4m3) behind
--kv-cache-dtype" §What (store kernel, QUANT switch) and the review comment
§"A bug on sm_89" (saturation, rounding); [PR113] "feat(kvcache): 8-bit DSV4
window/compressed KV behind --kv-cache-dtype" §Testing (split-k decode,
masked (-1) columns).
"""
import numpy as np
import pytest
import torch

import oracle
from paged_decode_attention_amd import workloads as W
from tests.gpu_util import (bf16_to_f64, dev_bf16, dev_i32, host_u16, host_u8, kvq, np_pool,
                            rel_err, requires_gpu, say)

pytestmark = [pytest.mark.gpu, requires_gpu]

TOL = 2e-2


@pytest.mark.parametrize("qtype", ["fp8_e4m3", "q8_0"])
def test_mixed_store_then_decode(qtype):
    wl = W.mixed()
    H, D = wl.n_kv_heads, wl.head_dim_qk
    k = kvq()
    # background: every page any sequence reads, in chunks of pages
    pages = set()
    for b in range(wl.batch):
        n = (int(wl.seq_lens[b]) + W.PAGE - 1) // W.PAGE
        cols = wl.page_table[b, :n]
        pages.update(int(x) for x in cols[cols >= 0])
    pages = np.array(sorted(pages), np.int64)
    say("mixed", qtype, "background pages", len(pages))
    kp, ks = k.alloc_pool(qtype, wl.num_pages, H, D)
    vp, vs = k.alloc_pool(qtype, wl.num_pages, H, D)
    for t in (kp, ks, vp, vs):
        t.zero_()
    okp, oks = np_pool(qtype, wl.num_pages, H, D)
    ovp, ovs = np_pool(qtype, wl.num_pages, H, D)
    step = 4096
    for lo in range(0, len(pages), step):
        pg = pages[lo:lo + step]
        bg_slots = (pg[:, None] * W.PAGE + np.arange(W.PAGE)[None]).reshape(-1).astype(np.int32)
        bg_k, bg_v = wl.page_rows(0, pg), wl.page_rows(1, pg)
        k.store(qtype, dev_bf16(bg_k), dev_bf16(bg_v), dev_i32(bg_slots), kp, ks, vp, vs)
        oracle.store(qtype, bg_k, bg_slots, H, D, W.PAGE, wl.num_pages, okp, oks)
        oracle.store(qtype, bg_v, bg_slots, H, D, W.PAGE, wl.num_pages, ovp, ovs)
        torch.cuda.synchronize()
    del bg_k, bg_v

    # the step's new tokens: one fused K+V store call
    new = wl.new_rows()
    slots = wl.new_tokens["slots"]
    say("mixed store", len(slots), "tokens")
    k.store(qtype, dev_bf16(new[0]), dev_bf16(new[1]), dev_i32(slots), kp, ks, vp, vs)
    torch.cuda.synchronize()
    oracle.store(qtype, new[0], slots, H, D, W.PAGE, wl.num_pages, okp, oks)
    oracle.store(qtype, new[1], slots, H, D, W.PAGE, wl.num_pages, ovp, ovs)
    pg, off = slots // W.PAGE, slots % W.PAGE
    for gp, gs, op, os_ in ((kp, ks, okp, oks), (vp, vs, ovp, ovs)):
        gpc = host_u8(gp)[pg, :, off, :]
        assert np.array_equal(gpc, op[pg, :, off, :]), "codes differ at new slots"
        assert np.array_equal(host_u16(gs)[pg, :, off, :], os_[pg, :, off, :]), "scales differ"

    # decode the whole batch; every row against the oracle
    q = wl.query()
    say("mixed decode", qtype)
    out, lse = k.paged_decode(qtype, dev_bf16(q), kp, ks, vp, vs, dev_i32(wl.page_table),
                              dev_i32(wl.seq_lens), wl.sm_scale)
    torch.cuda.synchronize()
    g_out = bf16_to_f64(host_u16(out)).reshape(-1, D)
    g_lse = lse.cpu().numpy().astype(np.float64).reshape(-1)
    o_out, o_lse = oracle.paged_decode(qtype, q, okp, oks, ovp, ovs, wl.page_table, wl.seq_lens,
                                       H, D, D, W.PAGE, wl.num_pages, wl.sm_scale)
    err = rel_err(g_out, o_out)
    worst = max(rel_err(g_out[r], o_out[r]) for r in range(len(o_out)))
    say("  rel err %.3e (worst row %.3e)" % (err, worst))
    assert err <= TOL
    assert np.abs(g_lse - o_lse).max() < 1e-2
