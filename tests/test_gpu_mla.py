"""GPU parity of kvq_paged_decode on the shared MLA latent slab (one 576-wide
row per token is K; its first 512 elements are V; one KV head for all query
heads) against the oracle's double-precision attention over the same pool.

Tolerance: max |o_gpu - o_ref| / max |o_ref| <= 2e-2 per output; the GPU
multiplies bf16 operands on the matrix cores with fp32 accumulation and
rounds the probabilities to bf16 before P V, so the expected error is a few
1e-3.  lse is checked to 1e-2 absolute.

Page keys: [PR113] "feat(kvcache): 8-bit DSV4 window/compressed KV behind
--kv-cache-dtype" §What this adds (one slab, K and V from the same row) and
§Testing (split-k decode, masked (-1) columns); [PR25] "Experimental FP8 KV
Cache" (128 heads against one 576/512 latent row).
"""
import numpy as np
import pytest
import torch

import oracle
from paged_decode_attention_amd import workloads as W
from tests.gpu_util import (bf16_to_f64, decode_both, dev_bf16, dev_i32, fill_both, host_u16,
                            kvq, np_pool, rel_err, requires_gpu, say)

pytestmark = [pytest.mark.gpu, requires_gpu]

TOL = 2e-2


def mla_workload(Hq, lens, width, seed, mask_frac=0.0, extra_pages=3):
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
        if mask_frac and n > 1:
            drop = rng.random(n) < mask_frac
            pt[b, :n][drop] = -1
    return W.Workload("mla_small_h%d" % Hq, len(lens), Hq, 1, 576, 512, n_pages, lens, pt, seed,
                      kind="mla", shared=True)


def check(wl, qtype, rows=None, tol=TOL):
    pools = fill_both(wl, qtype)
    g_out, g_lse, o_out, o_lse, rows = decode_both(wl, qtype, pools, rows=rows)
    err = rel_err(g_out[rows], o_out)
    say("  rel err %.3e" % err)
    assert err <= tol, err
    fin = np.isfinite(o_lse)
    assert np.array_equal(np.isfinite(g_lse[rows]), fin)
    if fin.any():
        assert np.abs(g_lse[rows][fin] - o_lse[fin]).max() < 1e-2
    return g_out, pools


@pytest.mark.parametrize("qtype", ["fp8_e4m3", "q8_0", "bf16", "fp8_e4m3_cast", "fp8_e5m2_cast",
                                   "fp8_ds_mla"])
@pytest.mark.parametrize("Hq", [128, 64, 16])
def test_mla_small_matches_oracle(qtype, Hq):
    """Ragged lengths around the page (16) and tile (32) edges, masked pages,
    an empty sequence, and enough pages for several split-K chunks."""
    lens = [0, 1, 15, 16, 17, 31, 32, 33, 300, 1111]
    wl = mla_workload(Hq, lens, 80, seed=Hq + 3, mask_frac=0.1)
    g_out, _ = check(wl, qtype)
    assert np.all(g_out[:Hq] == 0)


def test_mla_one_chunk_per_sequence():
    """Short contexts only: every sequence fits one work item, so the kernel
    writes the output itself and no merge runs."""
    wl = mla_workload(128, [5, 40, 64, 70], 5, seed=21)
    check(wl, "fp8_e4m3")


@pytest.mark.parametrize("qtype", ["fp8_e4m3", "q8_0"])
def test_mla_poisoned_unused_slots_never_reach_the_output(qtype):
    wl = mla_workload(128, [33, 250, 17], 40, seed=5, mask_frac=0.2, extra_pages=7)
    k = kvq()
    pool, scl = k.alloc_pool(qtype, wl.num_pages, 1, 576)
    pool.fill_(0x7F)
    scl.fill_(0x7E00)
    slots = []
    for b in range(wl.batch):
        for t in range(int(wl.seq_lens[b])):
            p = wl.page_table[b, t // W.PAGE]
            if p >= 0:
                slots.append(int(p) * W.PAGE + t % W.PAGE)
    slots = np.array(slots, np.int32)
    rows = wl.kv_rows(0, 0, len(slots))
    say("mla poison", qtype)
    k.store(qtype, dev_bf16(rows), None, dev_i32(slots), pool, scl)
    q = wl.query()
    out, lse = k.paged_decode(qtype, dev_bf16(q), pool, scl, pool, scl, dev_i32(wl.page_table),
                              dev_i32(wl.seq_lens), wl.sm_scale, head_dim_v=512)
    torch.cuda.synchronize()
    g = bf16_to_f64(host_u16(out)).reshape(-1, 512)
    assert np.all(np.isfinite(g)) and np.all(np.isfinite(lse.cpu().numpy()))
    op, os_ = np_pool(qtype, wl.num_pages, 1, 576, fill_code=0x7F, fill_scale=0x7E00)
    oracle.store(qtype, rows, slots, 1, 576, W.PAGE, wl.num_pages, op, os_)
    o, _ = oracle.paged_decode(qtype, q, op, os_, op, os_, wl.page_table, wl.seq_lens, 1, 576,
                               512, W.PAGE, wl.num_pages, wl.sm_scale)
    assert rel_err(g, o) <= TOL


@pytest.mark.parametrize("jumps", [1, 2])
def test_mla_scores_far_above_the_first_tile(jumps):
    """Scores that rise by far more than the kernel's softmax headroom after
    the first tiles (a constant query against rows whose level steps up)
    must still give the oracle's result."""
    L = 900
    wl = mla_workload(32, [L], 64, seed=31)
    rng = np.random.default_rng(8)
    x = rng.standard_normal((wl.n_slots, 1, 576)).astype(np.float32) * 0.1
    # token t's row level: 0 before the first step, then 2 (and 4); slots are
    # laid out by the page table
    t = np.arange(L)
    level = np.where(t >= 300, 2.0, 0.0) + (np.where(t >= 700, 2.0, 0.0) if jumps == 2 else 0.0)
    slot = wl.page_table[0, t // W.PAGE].astype(np.int64) * W.PAGE + t % W.PAGE
    x[slot, 0, :] += level[:, None].astype(np.float32)
    rows = W.to_bf16_bits(x)
    q = W.to_bf16_bits(np.ones((1, 32, 576), np.float32))
    k = kvq()
    pool, scl = k.alloc_pool("fp8_e4m3", wl.num_pages, 1, 576)
    slots = np.arange(wl.n_slots, dtype=np.int32)
    say("mla jumps", jumps)
    k.store("fp8_e4m3", dev_bf16(rows), None, dev_i32(slots), pool, scl)
    sm = 0.1  # score steps of about 0.1 * 576 * 2 = 115 natural-log units
    out, lse = k.paged_decode("fp8_e4m3", dev_bf16(q), pool, scl, pool, scl,
                              dev_i32(wl.page_table), dev_i32(wl.seq_lens), sm, head_dim_v=512)
    torch.cuda.synchronize()
    g = bf16_to_f64(host_u16(out)).reshape(-1, 512)
    op, os_ = np_pool("fp8_e4m3", wl.num_pages, 1, 576)
    oracle.store("fp8_e4m3", rows, slots, 1, 576, W.PAGE, wl.num_pages, op, os_)
    o, ol = oracle.paged_decode("fp8_e4m3", q, op, os_, op, os_, wl.page_table, wl.seq_lens, 1,
                                576, 512, W.PAGE, wl.num_pages, sm)
    assert rel_err(g, o) <= TOL
    # K enters the dot as bf16(code * scale): each product moves by at most
    # 2^-9 of itself, so a score near 120 may move by ~0.03; bound the lse by
    # 2^-8 of its size
    assert np.abs(lse.cpu().numpy().reshape(-1) - ol).max() < 2.0 ** -8 * np.abs(ol).max()


def test_mla_page_permutation_gives_identical_bits():
    wl = mla_workload(128, [700, 333], 48, seed=9)
    pools = fill_both(wl, "fp8_e4m3")
    k = kvq()
    q = dev_bf16(wl.query())
    o1, l1 = k.paged_decode("fp8_e4m3", q, pools["kp"], pools["ks"], pools["kp"], pools["ks"],
                            dev_i32(wl.page_table), dev_i32(wl.seq_lens), wl.sm_scale,
                            head_dim_v=512)
    perm = np.random.default_rng(3).permutation(wl.num_pages)
    inv = torch.from_numpy(np.argsort(perm)).cuda()
    p2, s2 = pools["kp"][inv], pools["ks"][inv]
    pt2 = np.where(wl.page_table >= 0, perm[np.maximum(wl.page_table, 0)], -1).astype(np.int32)
    say("mla permutation")
    o2, l2 = k.paged_decode("fp8_e4m3", q, p2, s2, p2, s2, dev_i32(pt2), dev_i32(wl.seq_lens),
                            wl.sm_scale, head_dim_v=512)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("qtype", ["fp8_e4m3", "fp8_ds_mla"])
def test_mla_full_size_all_rows(qtype):
    """The 163840-token slab with 128 heads, in the launch configuration the
    benchmark times; every head against the oracle."""
    check(W.mla(), qtype)
