"""GPU parity of kvq_paged_decode against the oracle's double-precision
attention over the same quantized pool (which the store tests show is
bit-identical on both sides).

Tolerance: max |o_gpu - o_ref| / max |o_ref| <= 2e-2 over each output, the
bar the target states; the GPU result is bf16 and accumulates in fp32, so the
expected error is a few 1e-3.  lse is checked to 1e-2 absolute.

Page keys: [PR103] "feat(kvcache): 8-bit KV cache (q8_0 / fp8_e4m3) behind
--kv-cache-dtype" §What (QUANT switch; dequantize before the dot); [PR113]
"feat(kvcache): 8-bit DSV4 window/compressed KV behind --kv-cache-dtype"
§Testing (split-k decode against the reference, masked (-1) columns).
"""
import numpy as np
import pytest
import torch

from paged_decode_attention_amd import workloads as W
from tests.gpu_util import (bf16_to_f64, decode_both, dev_bf16, dev_i32, fill_both, host_u16,
                            kvq, rel_err, requires_gpu, say)

pytestmark = [pytest.mark.gpu, requires_gpu]

TOL = 2e-2


def small_workload(D, Hq, Hkv, lens, width, seed, kind="normal", mask_frac=0.0, extra_pages=5):
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
    return W.Workload("small_d%d_h%dx%d" % (D, Hq, Hkv), len(lens), Hq, Hkv, D, D, n_pages, lens,
                      pt, seed, kind=kind)


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


@pytest.mark.parametrize("qtype", ["fp8_e4m3", "q8_0", "bf16", "fp8_e4m3_cast", "fp8_e5m2_cast"])
@pytest.mark.parametrize("D,Hq,Hkv", [(32, 4, 4), (64, 8, 2), (128, 16, 8), (128, 8, 1),
                                      (256, 16, 2), (128, 12, 2), (64, 6, 2),
                                      # 8+ query heads per kv head: the matrix-core kernel
                                      (64, 16, 1), (128, 32, 2), (128, 32, 1), (256, 40, 4)])
def test_decode_small_matches_oracle(qtype, D, Hq, Hkv):
    lens = [0, 1, 15, 16, 17, 300, 1111]
    wl = small_workload(D, Hq, Hkv, lens, 80, seed=D * 7 + Hq, mask_frac=0.1)
    g_out, _ = check(wl, qtype)
    # empty sequence: zeros
    assert np.all(g_out[: Hq] == 0)


@pytest.mark.parametrize("qtype", ["fp8_e4m3", "q8_0"])
@pytest.mark.parametrize("D,Hq,Hkv", [(128, 16, 8), (256, 16, 2), (64, 16, 1)])
def test_poisoned_unused_slots_never_reach_the_output(qtype, D, Hq, Hkv):
    """NaN codes and NaN scales in unwritten slots, masked pages and pages the
    table never names must not leak: the output stays finite and equal to
    the oracle's (which reads only valid tokens)."""
    wl = small_workload(D, Hq, Hkv, [33, 250, 17], 40, seed=5, mask_frac=0.2, extra_pages=7)
    k = kvq()
    H, D = wl.n_kv_heads, wl.head_dim_qk
    kp, ks = k.alloc_pool(qtype, wl.num_pages, H, D)
    vp, vs = k.alloc_pool(qtype, wl.num_pages, H, D)
    for p_, s_ in ((kp, ks), (vp, vs)):
        p_.fill_(0x7F)                     # e4m3 NaN (and 127 for q8_0)
        s_.fill_(0x7E00)                   # fp16 NaN
    # store only the valid tokens of each sequence
    slots = []
    for b in range(wl.batch):
        for t in range(int(wl.seq_lens[b])):
            p = wl.page_table[b, t // W.PAGE]
            if p >= 0:
                slots.append(int(p) * W.PAGE + t % W.PAGE)
    slots = np.array(slots, np.int32)
    ksrc, vsrc = wl.kv_rows(0, 0, len(slots)), wl.kv_rows(1, 0, len(slots))
    say("poison", qtype)
    k.store(qtype, dev_bf16(ksrc), dev_bf16(vsrc), dev_i32(slots), kp, ks, vp, vs)
    q = wl.query()
    out, lse = k.paged_decode(qtype, dev_bf16(q), kp, ks, vp, vs, dev_i32(wl.page_table),
                              dev_i32(wl.seq_lens), wl.sm_scale)
    torch.cuda.synchronize()
    g = bf16_to_f64(host_u16(out)).reshape(-1, D)
    assert np.all(np.isfinite(g)) and np.all(np.isfinite(lse.cpu().numpy()))
    import oracle
    from tests.gpu_util import np_pool
    okp, oks = np_pool(qtype, wl.num_pages, H, D, fill_code=0x7F, fill_scale=0x7E00)
    ovp, ovs = np_pool(qtype, wl.num_pages, H, D, fill_code=0x7F, fill_scale=0x7E00)
    oracle.store(qtype, ksrc, slots, H, D, W.PAGE, wl.num_pages, okp, oks)
    oracle.store(qtype, vsrc, slots, H, D, W.PAGE, wl.num_pages, ovp, ovs)
    o, _ = oracle.paged_decode(qtype, q, okp, oks, ovp, ovs, wl.page_table, wl.seq_lens, H, D, D,
                               W.PAGE, wl.num_pages, wl.sm_scale)
    assert rel_err(g, o) <= TOL


def test_page_permutation_gives_identical_bits():
    wl = small_workload(128, 16, 8, [700, 333], 48, seed=9)
    pools = fill_both(wl, "fp8_e4m3")
    k = kvq()
    q = dev_bf16(wl.query())
    args = (dev_i32(wl.seq_lens), wl.sm_scale)
    o1, l1 = k.paged_decode("fp8_e4m3", q, pools["kp"], pools["ks"], pools["vp"], pools["vs"],
                            dev_i32(wl.page_table), *args)
    rng = np.random.default_rng(3)
    perm = rng.permutation(wl.num_pages)
    inv = torch.from_numpy(np.argsort(perm)).cuda()  # new page j holds old page inv[j]
    kp2, ks2 = pools["kp"][inv], pools["ks"][inv]
    vp2, vs2 = pools["vp"][inv], pools["vs"][inv]
    pt2 = np.where(wl.page_table >= 0, perm[np.maximum(wl.page_table, 0)], -1).astype(np.int32)
    say("permutation")
    o2, l2 = k.paged_decode("fp8_e4m3", q, kp2, ks2, vp2, vs2, dev_i32(pt2), *args)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # and a second run of the same call is bitwise identical
    o3, _ = k.paged_decode("fp8_e4m3", q, kp2, ks2, vp2, vs2, dev_i32(pt2), *args)
    assert torch.equal(o2, o3)


def test_split_plan_does_not_change_the_result():
    """A wider page table (more -1 padding) changes the split-K chunking; the
    result must agree with the narrow one within tolerance."""
    narrow = small_workload(128, 16, 8, [2000, 1500, 40], 128, seed=11)
    wide = W.Workload(narrow.name, narrow.batch, 16, 8, 128, 128, narrow.num_pages,
                      narrow.seq_lens, np.pad(narrow.page_table, ((0, 0), (0, 1920)),
                                              constant_values=-1), narrow.seed)
    k = kvq()
    pools = fill_both(narrow, "q8_0")
    assert (k.debug_plan("q8_0", 3, 16, 8, 128, 128, 128)["max_items"] !=
            k.debug_plan("q8_0", 3, 16, 8, 128, 128, 2048)["max_items"])
    g1, *_ = decode_both(narrow, "q8_0", pools)
    g2, _, o2, _, _ = decode_both(wide, "q8_0", pools)
    assert rel_err(g1, g2) <= TOL and rel_err(g2, o2) <= TOL


# ---- full-size workloads, in the bench's launch configuration: every row ---------------

@pytest.mark.parametrize("qtype", ["fp8_e4m3", "q8_0"])
def test_tiny_workload_all_rows(qtype):
    check(W.tiny(), qtype)


@pytest.mark.parametrize("qtype", ["fp8_e4m3", "q8_0", "bf16", "fp8_e4m3_cast", "fp8_e5m2_cast"])
def test_qwen3_workload_all_rows(qtype):
    """8 x 16384 tokens, 16 q / 8 kv heads: all 128 output rows."""
    check(W.qwen3(replicas=1), qtype)


@pytest.mark.parametrize("qtype", ["fp8_e4m3", "q8_0"])
def test_ragged256_workload_all_rows(qtype):
    check(W.ragged256(), qtype)


@pytest.mark.parametrize("qtype", ["fp8_e4m3", "q8_0"])
def test_single256_workload_all_rows(qtype):
    check(W.single256(), qtype)


def test_host_lengths_size_the_launch_without_changing_bits():
    """seq_lens_host only sizes the grid: the same bits with and without it,
    for the VALU kernel (qwen3 shape), the matrix-core kernel (head_dim 256,
    8 heads per kv head) and ragged batches with empty sequences."""
    k = kvq()
    for wl in (W.qwen3(replicas=1), small_workload(256, 16, 2, [0, 5000, 17, 3000], 400, seed=4),
               small_workload(128, 16, 8, [0, 1, 2000, 0], 200, seed=6)):
        pools = fill_both(wl, "fp8_e4m3")
        q = dev_bf16(wl.query())
        args = (pools["kp"], pools["ks"], pools["vp"], pools["vs"], dev_i32(wl.page_table),
                dev_i32(wl.seq_lens), wl.sm_scale)
        say("host lengths", wl.name)
        o1, l1 = k.paged_decode("fp8_e4m3", q, *args)
        o2, l2 = k.paged_decode("fp8_e4m3", q, *args, seq_lens_host=wl.seq_lens)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
