"""GPU parity of kvq_extend_attention (causal extend / prefill attention over
the quantized pool) against the oracle's double-precision attention over the
same pool (filled by the GPU store and the oracle's store from the same rows).

Cases: prefill (every token new), extends after a prefix, a sequence with
more new tokens than its pool holds (the first ones see nothing), an empty
sequence, masked pages, query-row tiles that are full, partial or spread over
several tokens, head_dim 64 / 128 / 256, every storage type, and at the full
extend shape every row against the oracle.  Tolerance as the decode: max |o - r| / max |r| <=
2e-2, lse within 1e-2.

Page keys: [PR103] "feat(kvcache): 8-bit KV cache (q8_0 / fp8_e4m3) behind
--kv-cache-dtype" (§What: the quantized pool feeds the prefill / extend
attention kernels); [PR113] "feat(kvcache): 8-bit DSV4 window/compressed KV
behind --kv-cache-dtype" (§Testing: prefill, masked (-1) columns).
"""
import numpy as np
import pytest
import torch

import oracle
from paged_decode_attention_amd import workloads as W
from tests.gpu_util import (bf16_to_f64, dev_bf16, dev_i32, fill_both, host_u16, kvq, rel_err,
                            requires_gpu, say)

pytestmark = [pytest.mark.gpu, requires_gpu]

TOL = 2e-2


def ext_workload(Hq, Hkv, D, lens, width, seed, mask_frac=0.0, extra_pages=3):
    rng = np.random.default_rng(seed)
    lens = np.array(lens, np.int32)
    need = sum((int(x) + W.PAGE - 1) // W.PAGE for x in lens)
    n_pages = need + extra_pages
    perm = rng.permutation(n_pages).astype(np.int32)
    pt = np.full((len(lens), width), -1, np.int32)
    o = 0
    for b, L in enumerate(lens):
        n = (int(L) + W.PAGE - 1) // W.PAGE
        pt[b, :n] = perm[o:o + n]
        o += n
        if mask_frac:
            pt[b, :n][rng.random(n) < mask_frac] = -1
    return W.Workload("ext_h%dx%d_d%d" % (Hq, Hkv, D), len(lens), Hq, Hkv, D, D, n_pages, lens,
                      pt, seed)


def run(wl, qtype, news, max_new=None, pools=None, q_scale=None):
    k = kvq()
    pools = pools or fill_both(wl, qtype)
    q_start = np.concatenate([[0], np.cumsum(news)]).astype(np.int32)
    T = int(q_start[-1])
    q = W.extend_queries(wl, T)
    if q_scale is not None:  # scores q_scale times wider (bf16 of the scaled rows)
        q = W.to_bf16_bits(q_scale * W.bf16_bits_to_f32(q))
    max_new = max_new or max(1, int(max(news)))
    say("extend", wl.name, qtype, "news", list(news), "max_new", max_new)
    out, lse = k.extend_attention(qtype, dev_bf16(q), dev_i32(q_start), max_new, pools["kp"],
                                  pools["ks"], pools["vp"], pools["vs"], dev_i32(wl.page_table),
                                  dev_i32(wl.seq_lens), wl.sm_scale)
    torch.cuda.synchronize()
    g = bf16_to_f64(host_u16(out)).reshape(-1, wl.head_dim_v)
    g_lse = lse.cpu().numpy().astype(np.float64).reshape(-1)
    o, o_lse = oracle.extend_attention(qtype, q, q_start, pools["okp"], pools["oks"], pools["ovp"],
                                       pools["ovs"], wl.page_table, wl.seq_lens, wl.n_kv_heads,
                                       wl.head_dim_qk, W.PAGE, wl.num_pages, wl.sm_scale)
    err = rel_err(g, o)
    say("  rel err %.3e" % err)
    assert err <= TOL, err
    fin = np.isfinite(o_lse)
    assert np.array_equal(np.isfinite(g_lse), fin)
    if fin.any():  # (relative to its size for scores hundreds of nats wide)
        assert np.all(np.abs(g_lse[fin] - o_lse[fin]) <= 1e-2 + 1e-5 * np.abs(o_lse[fin]))
    return g, g_lse, o, q_start, o_lse


@pytest.mark.parametrize("qtype", ["fp8_e4m3", "q8_0", "bf16", "fp8_e4m3_cast", "fp8_e5m2_cast"])
def test_extend_matches_oracle(qtype):
    """16 q / 8 kv heads, head_dim 128: a 64-token extend after a prefix, a
    prefill (every token new), a short extend, an empty sequence and more new
    tokens than the pool holds; masked pages."""
    wl = ext_workload(16, 8, 128, [700, 130, 64, 0, 5], 48, seed=11, mask_frac=0.1)
    g, g_lse, o, q_start, _ = run(wl, qtype, [64, 9, 64, 0, 8])
    Hq = wl.n_q_heads
    s0 = int(q_start[4])  # sequence 4: 8 new tokens, 5 in the pool -> the first 3 see nothing
    assert np.all(g[s0 * Hq:(s0 + 3) * Hq] == 0) and np.all(np.isneginf(g_lse[s0 * Hq:(s0 + 3) * Hq]))


@pytest.mark.parametrize("Hq,Hkv,D,news", [(8, 2, 64, [3, 1, 2]), (16, 2, 256, [2, 1, 1]),
                                           (32, 4, 128, [1, 5, 3]), (4, 4, 128, [33, 17, 40]),
                                           (16, 2, 256, [5, 1, 4]), (8, 2, 64, [9, 16, 3]),
                                           (16, 8, 128, [9, 16, 1])])
def test_extend_head_groups(Hq, Hkv, D, news):
    """Tiles of G heads x a few tokens, a partial last tile, one head per kv
    head (G = 1, 16 tokens per tile), and 40-128 query rows per kv head
    (several tiles per unit, the last one partly padding)."""
    wl = ext_workload(Hq, Hkv, D, [400, 77, 1000], 70, seed=Hq + D, mask_frac=0.05)
    run(wl, "fp8_e4m3", news)


@pytest.mark.parametrize("Hq,Hkv,D,news", [(16, 8, 128, [64, 40]), (16, 2, 256, [20, 9])])
def test_extend_scores_hundreds_of_nats_apart(Hq, Hkv, D, news):
    """Queries scaled by 150: scores ~ N(0, 150^2) nats, so the largest score
    of a work item sits hundreds of nats above its first step's, and the item
    is streamed a second time against that score."""
    wl = ext_workload(Hq, Hkv, D, [3000, 1500], 200, seed=D + 150, mask_frac=0.2)
    *_, o_lse = run(wl, "fp8_e4m3", news, q_scale=150.0)
    assert np.nanmax(o_lse) > 300.0


def test_extend_max_new_above_every_sequence():
    wl = ext_workload(16, 8, 128, [300, 90], 30, seed=5)
    run(wl, "fp8_e4m3", [7, 12], max_new=40)


def test_extend_split_sequences_merge():
    """Long prefixes: a sequence splits into many items per query tile, merged
    by the last workgroup or the merge kernel."""
    wl = ext_workload(16, 8, 128, [20000, 9000], 1300, seed=21)
    run(wl, "fp8_e4m3", [16, 4])


def test_extend_merge_weights_at_twelve_columns():
    """4 q / 1 kv head, head_dim 64, 3 new tokens: 12 query columns per tile,
    which do not divide the merge's 4096 LDS weights.  One 21840-token
    sequence in a 1365-column page table splits into the most chunks the
    planner allows; the planner keeps chunks x 12 within the LDS array (an
    earlier bound allowed 342 chunks, 4104 weights)."""
    L = 21840
    wl = ext_workload(4, 1, 64, [L], 1365, seed=1365)
    k = kvq()
    plan = k.debug_plan("fp8_e4m3", 1, 4, 1, 64, 64, 1365, 3)
    assert -(-1365 // plan["min_pages"]) * plan["gt"] * plan["tn"] <= 4096
    run(wl, "fp8_e4m3", [3])


def test_extend_full_shape_all_rows():
    """8 sequences x 16384 tokens, the last 64 of each new (the bench shape):
    every new token's rows against the oracle's causal attention."""
    wl = W.extend()
    k = kvq()
    pools = fill_both(wl, "fp8_e4m3")
    q_start = wl.new_tokens["q_start"]
    T = int(q_start[-1])
    q = W.extend_queries(wl, T)
    say("extend full shape", wl.name)
    out, lse = k.extend_attention("fp8_e4m3", dev_bf16(q), dev_i32(q_start), 64, pools["kp"],
                                  pools["ks"], pools["vp"], pools["vs"], dev_i32(wl.page_table),
                                  dev_i32(wl.seq_lens), wl.sm_scale)
    torch.cuda.synchronize()
    g = bf16_to_f64(host_u16(out)).reshape(-1, wl.head_dim_v)
    g_lse = lse.cpu().numpy().astype(np.float64).reshape(-1)
    o, o_lse = oracle.extend_attention("fp8_e4m3", q, q_start, pools["okp"], pools["oks"],
                                       pools["ovp"], pools["ovs"], wl.page_table, wl.seq_lens,
                                       wl.n_kv_heads, wl.head_dim_qk, W.PAGE, wl.num_pages,
                                       wl.sm_scale)
    err = rel_err(g, o)
    say("  rel err %.3e" % err)
    assert err <= TOL
    assert np.abs(g_lse - o_lse).max() < 1e-2


def test_extend_rows_past_max_new_untouched_and_empty_pool_zeroed():
    """A sequence with more new tokens than max_new_tokens: its first
    max_new rows are computed (at their true positions), the rest are left
    as they were.  A sequence whose pool is empty but lists new tokens: those
    rows are 0 with lse -inf (no work item covers it)."""
    k = kvq()
    wl = ext_workload(16, 8, 128, [300, 0, 90], 20, seed=8)
    pools = fill_both(wl, "fp8_e4m3")
    news = [6, 3, 4]
    q_start = np.concatenate([[0], np.cumsum(news)]).astype(np.int32)
    T = int(q_start[-1])
    q = W.extend_queries(wl, T)
    out = torch.full((T, 16, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((T, 16), 5.0, dtype=torch.float32, device="cuda")
    say("extend max_new 4 with 6 new tokens")
    k.extend_attention("fp8_e4m3", dev_bf16(q), dev_i32(q_start), 4, pools["kp"], pools["ks"],
                       pools["vp"], pools["vs"], dev_i32(wl.page_table), dev_i32(wl.seq_lens),
                       wl.sm_scale, out=out, lse=lse)
    torch.cuda.synchronize()
    g = bf16_to_f64(host_u16(out)).reshape(T, 16, 128)
    gl = lse.cpu().numpy().astype(np.float64)
    o, ol = oracle.extend_attention("fp8_e4m3", q, q_start, pools["okp"], pools["oks"],
                                    pools["ovp"], pools["ovs"], wl.page_table, wl.seq_lens, 8, 128,
                                    W.PAGE, wl.num_pages, wl.sm_scale)
    o = o.reshape(T, 16, 128)
    ol = ol.reshape(T, 16)
    written = [0, 1, 2, 3] + [9, 10, 11, 12]          # sequences 0 (first 4) and 2
    assert rel_err(g[written], o[written]) <= TOL
    assert np.abs(gl[written] - ol[written]).max() < 1e-2
    assert np.all(g[4:6] == 7.0) and np.all(gl[4:6] == 5.0)   # past max_new: untouched
    assert np.all(g[6:9] == 0) and np.all(np.isneginf(gl[6:9]))  # empty pool


@pytest.mark.parametrize("qtype", ["fp8_e4m3", "bf16", "fp8_ds_mla"])
def test_extend_over_the_mla_slab(qtype):
    """The shared 576/512 slab, 64 query heads: extends after a prefix, a
    prefill, more new tokens than the pool holds, an empty sequence, masked
    pages, sequences long enough to split into several items."""
    from tests.test_gpu_mla import mla_workload
    k = kvq()
    wl = mla_workload(64, [900, 40, 3, 0, 3000], 200, seed=13, mask_frac=0.1)
    pools = fill_both(wl, qtype)
    news = [9, 40, 5, 0, 2]
    q_start = np.concatenate([[0], np.cumsum(news)]).astype(np.int32)
    T = int(q_start[-1])
    q = W.extend_queries(wl, T)
    say("extend over the slab", qtype)
    out, lse = k.extend_attention(qtype, dev_bf16(q), dev_i32(q_start), max(news), pools["kp"],
                                  pools["ks"], pools["kp"], pools["ks"], dev_i32(wl.page_table),
                                  dev_i32(wl.seq_lens), wl.sm_scale)
    torch.cuda.synchronize()
    g = bf16_to_f64(host_u16(out)).reshape(-1, 512)
    gl = lse.cpu().numpy().astype(np.float64).reshape(-1)
    o, ol = oracle.extend_attention(qtype, q, q_start, pools["okp"], pools["oks"], pools["okp"],
                                    pools["oks"], wl.page_table, wl.seq_lens, 1, 576, W.PAGE,
                                    wl.num_pages, wl.sm_scale, head_dim_v=512)
    assert rel_err(g, o) <= TOL
    fin = np.isfinite(ol)
    assert np.array_equal(np.isfinite(gl), fin)
    assert np.abs(gl[fin] - ol[fin]).max() < 1e-2
    s2 = int(q_start[2])  # 5 new tokens, 3 in the pool: the first 2 see nothing
    assert np.all(g[s2 * 64:(s2 + 2) * 64] == 0)


def long_prefill_workload(Hq, Hkv, D, seed, lens, width):
    return ext_workload(Hq, Hkv, D, lens, width, seed=seed, mask_frac=0.03)


# A long-prefill plan: max_new_tokens 4096 gives so many (sequence, kv head,
# tile group) units that the split plan's partials would pass 1 GiB, so each
# unit is one work item over its whole sequence (streamed in sub-chunks of
# 256 pages).  The sequences list fewer new tokens than that (the other tiles
# have no rows), so the oracle stays cheap; two of them reach 16384 and 9000
# tokens (4 and 3 sub-chunks), one has its new tokens on both sides of the
# 4096-token sub-chunk boundary.
LONG_LENS = [16384, 9000, 4200, 300, 1000, 77, 4096, 2500]
LONG_NEWS = [40, 17, 200, 300, 33, 77, 9, 64]


@pytest.mark.parametrize("Hq,Hkv,D", [(16, 8, 128), (16, 2, 256)])
def test_extend_long_prefill_whole_sequences(Hq, Hkv, D):
    """Whole-sequence work items, no split-K partials in the workspace;
    every row against the oracle."""
    wl = long_prefill_workload(Hq, Hkv, D, 4096 + D, LONG_LENS, 1030)
    plan = kvq().debug_plan("fp8_e4m3", wl.batch, Hq, Hkv, D, D, wl.max_pages, 4096)
    assert plan["whole"] and plan["bytes"] < 1 << 20
    run(wl, "fp8_e4m3", LONG_NEWS, max_new=4096)


def test_extend_long_prefill_scores_hundreds_of_nats_apart():
    """Whole-sequence items with queries scaled by 150: the largest score of
    an item can sit in a later sub-chunk, hundreds of nats above the first
    page's, and the item is streamed again over all its sub-chunks."""
    wl = long_prefill_workload(16, 8, 128, 4097, LONG_LENS, 1030)
    *_, o_lse = run(wl, "fp8_e4m3", LONG_NEWS, max_new=4096, q_scale=150.0)
    assert np.nanmax(o_lse) > 300.0
