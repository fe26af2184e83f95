"""GPU parity of kvq_sparse_mla_decode (sparse top-k decode over the shared
MLA slab) against the oracle's double-precision attention over the listed
rows of the same pool.

Lists mix positions inside the sequence, -1 padding, positions at or past
the length, positions on masked pages and repeated positions; list lengths
are a multiple of a page or not.  Tolerance as the dense slab decode: max
|o_gpu - o_ref| / max |o_ref| <= 2e-2, lse within 1e-2.

Page keys: [PR25] "Experimental FP8 KV Cache" (SPARSE_MLA_DECODE: D=576,
Hq=128, Hkv=1, Dv=512, K=256); [PR113] "feat(kvcache): 8-bit DSV4
window/compressed KV behind --kv-cache-dtype" (§What this adds, §Testing:
masked (-1) columns).
"""
import numpy as np
import pytest
import torch

import oracle
from paged_decode_attention_amd import workloads as W
from tests.gpu_util import (bf16_to_f64, dev_bf16, dev_i32, fill_both, host_u16, kvq, rel_err,
                            requires_gpu, say)
from tests.test_gpu_mla import mla_workload

pytestmark = [pytest.mark.gpu, requires_gpu]

TOL = 2e-2


def make_lists(rng, wl, K, pad=0.1, past=0.05, dup=0.05):
    lists = np.empty((wl.batch, K), np.int32)
    for b in range(wl.batch):
        L = int(wl.seq_lens[b])
        t = rng.integers(0, max(L, 1), K) if L else np.full(K, -1)
        r = rng.random(K)
        t = np.where(r < pad, -1, t)
        t = np.where((r >= pad) & (r < pad + past), L + rng.integers(0, 40, K), t)
        if K > 4:
            d = rng.random(K) < dup
            t[d] = t[0]
        lists[b] = t
    return lists


def run(wl, qtype, topk, pools=None):
    k = kvq()
    pools = pools or fill_both(wl, qtype)
    q = wl.query()
    say("sparse", wl.name, qtype, "k", topk.shape[1])
    out, lse = k.sparse_mla_decode(qtype, dev_bf16(q), pools["kp"], pools["ks"],
                                   dev_i32(wl.page_table), dev_i32(wl.seq_lens), dev_i32(topk),
                                   wl.sm_scale)
    torch.cuda.synchronize()
    g = bf16_to_f64(host_u16(out)).reshape(-1, 512)
    g_lse = lse.cpu().numpy().astype(np.float64).reshape(-1)
    o, o_lse = oracle.sparse_mla_decode(qtype, q, pools["okp"], pools["oks"], wl.page_table,
                                        wl.seq_lens, topk, 576, 512, W.PAGE, wl.num_pages,
                                        wl.sm_scale)
    err = rel_err(g, o)
    say("  rel err %.3e" % err)
    assert err <= TOL, err
    fin = np.isfinite(o_lse)
    assert np.array_equal(np.isfinite(g_lse), fin)
    if fin.any():
        assert np.abs(g_lse[fin] - o_lse[fin]).max() < 1e-2
    return g, g_lse, pools


@pytest.mark.parametrize("qtype", ["fp8_e4m3", "q8_0", "bf16", "fp8_e4m3_cast", "fp8_e5m2_cast",
                                   "fp8_ds_mla"])
@pytest.mark.parametrize("K", [256, 100, 33])
def test_sparse_matches_oracle(qtype, K):
    wl = mla_workload(128, [0, 700, 2000, 45], 140, seed=K + 5, mask_frac=0.15)
    topk = make_lists(np.random.default_rng(K), wl, K)
    g, g_lse, _ = run(wl, qtype, topk)
    assert np.all(g[:128] == 0) and np.all(np.isneginf(g_lse[:128]))  # the empty sequence


@pytest.mark.parametrize("Hq", [64, 16])
def test_sparse_fewer_heads_and_a_list_past_one_chunk(Hq):
    wl = mla_workload(Hq, [3000, 1200], 200, seed=Hq, mask_frac=0.1)
    run(wl, "fp8_e4m3", make_lists(np.random.default_rng(Hq), wl, 1500))


def test_sparse_list_of_every_position_matches_the_dense_decode():
    """A list naming each position once is the dense decode of the sequence."""
    wl = mla_workload(128, [333, 1024, 90], 70, seed=77, mask_frac=0.1)
    K = int(wl.seq_lens.max())
    topk = np.full((wl.batch, K), -1, np.int32)
    for b, L in enumerate(wl.seq_lens):
        topk[b, :L] = np.random.default_rng(b).permutation(int(L))
    g, g_lse, pools = run(wl, "fp8_e4m3", topk)
    k = kvq()
    out, lse = k.paged_decode("fp8_e4m3", dev_bf16(wl.query()), pools["kp"], pools["ks"],
                              pools["kp"], pools["ks"], dev_i32(wl.page_table),
                              dev_i32(wl.seq_lens), wl.sm_scale, head_dim_v=512)
    torch.cuda.synchronize()
    d = bf16_to_f64(host_u16(out)).reshape(-1, 512)
    assert rel_err(g, d) <= TOL
    assert np.abs(lse.cpu().numpy().reshape(-1) - g_lse).max() < 1e-2


def test_sparse_full_size_slab():
    """The 163840-token slab, 128 heads, 256 distinct positions per query: the
    shape the page profiles."""
    wl = W.mla()
    rng = np.random.default_rng(256)
    topk = np.stack([rng.choice(int(L), 256, replace=False) for L in wl.seq_lens]).astype(np.int32)
    run(wl, "fp8_e4m3", topk)


def test_sparse_longest_lists_in_the_largest_items():
    """130 lists of the most entries a call takes (2048), 16 heads: 130 x 64
    tiles over 256 workgroups asks for 33 tiles per work item, so items
    reach their cap of 1024 entries; each list is two items, and an item's
    row list fills the kernel's LDS array."""
    lens = np.random.default_rng(9).integers(0, 2500, 130)
    lens[3] = 0
    wl = mla_workload(16, lens.tolist(), 160, seed=9, mask_frac=0.1)
    run(wl, "fp8_e4m3", make_lists(np.random.default_rng(2048), wl, 2048))
