"""GPU parity of kvq_paged_decode at extreme score ranges.

The decode kernels weigh every score against a softmax reference that stays
fixed over a pass (the largest score of a wave's first page, or 0 when that
page has no valid token) and stream a work item a second time when its
largest score lands more than 2^64 away from that reference.  These cases
reach that second pass: scores hundreds of nats apart inside one work item,
every score far below zero, and many masked first pages.  The expected values
are the oracle's double-precision softmax over the same quantized pool.

Page keys: [PR103] "feat(kvcache): 8-bit KV cache (q8_0 / fp8_e4m3) behind
--kv-cache-dtype" §What (attention over the dequantized pool); [PR113]
"feat(kvcache): 8-bit DSV4 window/compressed KV behind --kv-cache-dtype"
§Testing (split-k decode, masked (-1) columns).
"""
import numpy as np
import pytest
import torch

import oracle
from paged_decode_attention_amd import workloads as W
from tests.gpu_util import (bf16_to_f64, dev_bf16, dev_i32, host_u16, kvq, np_pool, rel_err,
                            requires_gpu, say)
from tests.test_gpu_decode import TOL, small_workload

pytestmark = [pytest.mark.gpu, requires_gpu]


def slots_of(wl):
    out = []
    for b in range(wl.batch):
        for t in range(int(wl.seq_lens[b])):
            p = wl.page_table[b, t // W.PAGE]
            if p >= 0:
                out.append(int(p) * W.PAGE + t % W.PAGE)
    return np.array(out, np.int32)


def run(wl, qtype, ksrc, vsrc, q_bits):
    """Store the same rows on both sides, decode the whole batch on the GPU
    and in the oracle, and compare outputs and lse."""
    k = kvq()
    H, D = wl.n_kv_heads, wl.head_dim_qk
    slots = slots_of(wl)
    kp, ks = k.alloc_pool(qtype, wl.num_pages, H, D)
    vp, vs = k.alloc_pool(qtype, wl.num_pages, H, D)
    say("range", wl.name, qtype, "tokens", len(slots))
    k.store(qtype, dev_bf16(ksrc), dev_bf16(vsrc), dev_i32(slots), kp, ks, vp, vs)
    out, lse = k.paged_decode(qtype, dev_bf16(q_bits), kp, ks, vp, vs, dev_i32(wl.page_table),
                              dev_i32(wl.seq_lens), wl.sm_scale)
    torch.cuda.synchronize()
    g = bf16_to_f64(host_u16(out)).reshape(-1, D)
    g_lse = lse.cpu().numpy().astype(np.float64).reshape(-1)
    okp, oks = np_pool(qtype, wl.num_pages, H, D)
    ovp, ovs = np_pool(qtype, wl.num_pages, H, D)
    oracle.store(qtype, ksrc, slots, H, D, W.PAGE, wl.num_pages, okp, oks)
    oracle.store(qtype, vsrc, slots, H, D, W.PAGE, wl.num_pages, ovp, ovs)
    o, o_lse = oracle.paged_decode(qtype, q_bits, okp, oks, ovp, ovs, wl.page_table, wl.seq_lens,
                                   H, D, D, W.PAGE, wl.num_pages, wl.sm_scale)
    err = rel_err(g, o)
    say("  rel err %.3e" % err)
    assert np.all(np.isfinite(g))
    assert err <= TOL, err
    fin = np.isfinite(o_lse)
    assert np.array_equal(np.isfinite(g_lse), fin)
    # lse is checked relative to its size here: a few hundred nats
    assert np.all(np.abs(g_lse[fin] - o_lse[fin]) <= 1e-2 + 1e-5 * np.abs(o_lse[fin]))
    return o_lse


# long enough that every wave streams several pages of each work item
LENS, WIDTH = [20000, 9000, 300], 1400
KERNEL_SHAPES = [(128, 16, 8),   # 2 query heads per kv head: VALU kernel
                 (64, 4, 4),     # 1 per kv head
                 (128, 8, 1),    # 8 per kv head on the VALU kernel's widest group
                 (256, 16, 2),   # 8 per kv head: matrix-core kernel
                 (64, 16, 1)]    # 16 per kv head: matrix-core kernel


@pytest.mark.parametrize("qtype", ["fp8_e4m3", "q8_0"])
@pytest.mark.parametrize("D,Hq,Hkv", KERNEL_SHAPES)
def test_scores_hundreds_of_nats_apart(qtype, D, Hq, Hkv):
    """q scaled by 150: scores ~ N(0, 150^2) nats, so within one work item the
    largest score sits hundreds of nats above the first page's (weights
    against the first reference would overflow fp32).  Long sequences give
    every wave several pages per work item."""
    wl = small_workload(D, Hq, Hkv, LENS, WIDTH, seed=D + Hq, mask_frac=0.3)
    n = len(slots_of(wl))
    rng = np.random.default_rng(D * 3 + Hq)
    ksrc = W.to_bf16_bits(rng.standard_normal((n, Hkv, D), dtype=np.float32))
    vsrc = W.to_bf16_bits(rng.standard_normal((n, Hkv, D), dtype=np.float32))
    q = W.to_bf16_bits(150.0 * rng.standard_normal((wl.batch, Hq, D), dtype=np.float32))
    o_lse = run(wl, qtype, ksrc, vsrc, q)
    assert np.nanmax(o_lse) > 300.0  # the case really has scores this large


@pytest.mark.parametrize("qtype", ["fp8_e4m3", "q8_0"])
@pytest.mark.parametrize("D,Hq,Hkv", KERNEL_SHAPES)
def test_all_scores_far_below_zero_with_masked_first_pages(qtype, D, Hq, Hkv):
    """Every key positive and every query element -4: all scores near -11 sqrt(D)
    nats, so weights against a reference of 0 underflow.  Half the pages are
    masked, so many waves start on a page with no valid token and take 0 as
    their first reference."""
    wl = small_workload(D, Hq, Hkv, LENS, WIDTH, seed=2 * D + Hq, mask_frac=0.5)
    n = len(slots_of(wl))
    rng = np.random.default_rng(D * 5 + Hq)
    ksrc = W.to_bf16_bits(np.abs(rng.standard_normal((n, Hkv, D), dtype=np.float32)) + 2.0)
    vsrc = W.to_bf16_bits(rng.standard_normal((n, Hkv, D), dtype=np.float32))
    q = W.to_bf16_bits(np.full((wl.batch, Hq, D), -4.0, np.float32))
    o_lse = run(wl, qtype, ksrc, vsrc, q)
    fin = np.isfinite(o_lse)
    assert fin.any() and np.max(o_lse[fin]) < -50.0
