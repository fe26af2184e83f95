"""GPU parity of kvq_paged_decode_append: each sequence's new token stored,
then the decode, in one call.

Every case is checked twice:
  - against the library's two calls it stands for (kvq_store of the new rows
    at the slots the header defines, then kvq_paged_decode) on a copy of the
    same pools: output, lse and every pool byte identical;
  - against the oracle (its store of the new rows, then its decode):
    max |o_gpu - o_ref| / max |o_ref| <= 2e-2 over the whole output and lse
    within 1e-2, the decode's tolerance.

The cases cover the kernel that stores inside the decode launch (separate
K/V, fewer than 8 query heads per kv head: head_dim 32-256, several head
groups per kv head, head group 0 the only writer) and the shapes that store
first and decode after (the matrix-core kernel, the shared MLA slab, the
656-byte row); lengths at page edges, an empty sequence, a new token on a
masked page (not stored, not attended) and a length beyond the page table
(nothing stored).

Page keys: [PR126] "Add fp8 KV-cache quantization (--kv-dtype)" §How it works
(the new k/v rows are converted as they are written, attention dequantizes on
read); [PR103] "feat(kvcache): 8-bit KV cache (q8_0 / fp8_e4m3) behind
--kv-cache-dtype" §What (the store kernel; dequant inside attention).
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


def workload(D, Hq, Hkv, lens, width, seed, shared=False, masked_last=(), extra_pages=4):
    """Pages dealt from a permutation; lens beyond width * 16 fill the whole
    row; the sequences in masked_last lose their last page (-1)."""
    rng = np.random.default_rng(seed)
    lens = np.array(lens, np.int32)
    npg = [min((int(L) + W.PAGE - 1) // W.PAGE, width) for L in lens]
    n_pages = sum(npg) + extra_pages
    perm = rng.permutation(n_pages).astype(np.int32)
    pt = np.full((len(lens), width), -1, np.int32)
    o = 0
    for b, n in enumerate(npg):
        pt[b, :n] = perm[o:o + n]
        o += n
        if b in masked_last and n:
            pt[b, n - 1] = -1
    if shared:
        return W.Workload("append_mla_h%d" % Hq, len(lens), Hq, 1, 576, 512, n_pages, lens, pt,
                          seed, kind="mla", shared=True)
    return W.Workload("append_d%d_h%dx%d" % (D, Hq, Hkv), len(lens), Hq, Hkv, D, D, n_pages, lens,
                      pt, seed)


def new_slots(wl) -> np.ndarray:
    """The slot of each sequence's new token, as the header defines it."""
    slots = np.full(wl.batch, -1, np.int32)
    cap = wl.max_pages * W.PAGE
    for b in range(wl.batch):
        L = int(wl.seq_lens[b])
        if 1 <= L <= cap:
            P = int(wl.page_table[b, (L - 1) // W.PAGE])
            if 0 <= P < wl.num_pages:
                slots[b] = P * W.PAGE + (L - 1) % W.PAGE
    return slots


def new_rows(wl, seed, tensor) -> np.ndarray:
    """bf16 bits [batch][n_kv_heads][head_dim_qk]: N(0,1) with an all-zero
    block, a block of -0, a +-1e4 outlier and a constant block."""
    rng = np.random.Generator(np.random.PCG64([seed, 77, tensor]))
    x = rng.standard_normal((wl.batch, wl.n_kv_heads, wl.head_dim_qk), dtype=np.float32)
    b = wl.batch - 1
    x[b, 0, :32] = 0.0
    if wl.head_dim_qk >= 64:
        x[b, -1, 32:64] = -0.0
    x[0, -1, 5] = 1e4 if tensor == 0 else -1e4
    x[0, 0, -32:] = 0.75
    return W.to_bf16_bits(x)


def bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32) \
        if t.element_size() == 4 else t


def check_append(wl, qtype, seed=1):
    k = kvq()
    H, D = wl.n_kv_heads, wl.head_dim_qk
    pools = fill_both(wl, qtype)
    names = ("kp", "ks") if wl.shared else ("kp", "ks", "vp", "vs")
    copy = {n: (pools[n].clone() if pools[n] is not None else None) for n in names}
    if wl.shared:
        copy["vp"], copy["vs"] = copy["kp"], copy["ks"]
    nk = new_rows(wl, seed, 0)
    nv = None if wl.shared else new_rows(wl, seed, 1)
    d_nk, d_nv = dev_bf16(nk), (None if wl.shared else dev_bf16(nv))
    q = dev_bf16(wl.query())
    pt, sl = dev_i32(wl.page_table), dev_i32(wl.seq_lens)
    say("append", wl.name, qtype)
    out1, lse1 = k.paged_decode_append(qtype, q, d_nk, d_nv, pools["kp"], pools["ks"],
                                       pools["vp"], pools["vs"], pt, sl, wl.sm_scale,
                                       head_dim_v=wl.head_dim_v)
    slots = new_slots(wl)
    say("store then decode", wl.name, qtype)
    k.store(qtype, d_nk, d_nv, dev_i32(slots), copy["kp"], copy["ks"],
            None if wl.shared else copy["vp"], None if wl.shared else copy["vs"])
    out2, lse2 = k.paged_decode(qtype, q, copy["kp"], copy["ks"], copy["vp"], copy["vs"], pt, sl,
                                wl.sm_scale, head_dim_v=wl.head_dim_v)
    torch.cuda.synchronize()
    assert torch.equal(bits(out1), bits(out2))
    assert torch.equal(bits(lse1), bits(lse2))
    for n in names:
        if pools[n] is not None:
            assert torch.equal(bits(pools[n]), bits(copy[n])), n
    # the oracle: its own store of the new rows, then its decode
    oracle.store(qtype, nk, slots, H, D, W.PAGE, wl.num_pages, pools["okp"], pools["oks"])
    if not wl.shared:
        oracle.store(qtype, nv, slots, H, D, W.PAGE, wl.num_pages, pools["ovp"], pools["ovs"])
    vp = pools["okp"] if wl.shared else pools["ovp"]
    vs = pools["oks"] if wl.shared else pools["ovs"]
    o_out, o_lse = oracle.paged_decode(qtype, wl.query(), pools["okp"], pools["oks"], vp, vs,
                                       wl.page_table, wl.seq_lens, H, D, wl.head_dim_v, W.PAGE,
                                       wl.num_pages, wl.sm_scale)
    g = bf16_to_f64(host_u16(out1)).reshape(wl.batch * wl.n_q_heads, wl.head_dim_v)
    err = rel_err(g, o_out)
    say("  rel err %.3e" % err)
    assert err <= TOL, err
    g_lse = lse1.cpu().numpy().astype(np.float64).reshape(-1)
    fin = np.isfinite(o_lse)
    assert np.array_equal(np.isfinite(g_lse), fin)
    if fin.any():
        assert np.abs(g_lse[fin] - o_lse[fin]).max() < 1e-2
    return slots


LENS = [0, 1, 15, 16, 17, 300, 1111, 2000]   # the last one beyond a 100-page table


@pytest.mark.parametrize("qtype", ["fp8_e4m3", "q8_0", "bf16", "fp8_e4m3_cast", "fp8_e5m2_cast"])
@pytest.mark.parametrize("D,Hq,Hkv", [(128, 16, 8), (32, 16, 1), (128, 12, 2)])
def test_append_in_the_decode_launch_every_type(qtype, D, Hq, Hkv):
    wl = workload(D, Hq, Hkv, LENS, 100, seed=D + Hq, masked_last=(5,))
    slots = check_append(wl, qtype)
    # the cases the header names: empty, masked last page, beyond the table
    assert slots[0] == -1 and slots[5] == -1 and slots[7] == -1 and (slots[1:5] >= 0).all()


@pytest.mark.parametrize("qtype", ["fp8_e4m3", "q8_0"])
@pytest.mark.parametrize("D,Hq,Hkv", [(32, 4, 4), (64, 8, 2), (64, 6, 2), (256, 16, 4),
                                      (128, 4, 1), (256, 8, 2)])
def test_append_in_the_decode_launch_shapes(qtype, D, Hq, Hkv):
    wl = workload(D, Hq, Hkv, [3, 16, 33, 500, 4097], 300, seed=3 * D + Hq, masked_last=(2,))
    check_append(wl, qtype)


@pytest.mark.parametrize("qtype", ["fp8_e4m3", "q8_0", "bf16"])
@pytest.mark.parametrize("D,Hq,Hkv", [(128, 16, 2), (128, 8, 1), (256, 32, 2)])
def test_append_store_then_decode_on_the_matrix_cores(qtype, D, Hq, Hkv):
    wl = workload(D, Hq, Hkv, LENS, 100, seed=5 * D + Hq, masked_last=(4,))
    check_append(wl, qtype)


@pytest.mark.parametrize("qtype", ["fp8_e4m3", "fp8_ds_mla", "bf16"])
def test_append_mla_slab(qtype):
    wl = workload(576, 64, 1, [0, 1, 16, 33, 700], 50, seed=11, shared=True, masked_last=(3,))
    check_append(wl, qtype)


def test_append_large_batch():
    """More than 64 sequences: the work list is scanned in LDS."""
    rng = np.random.default_rng(17)
    lens = rng.integers(0, 400, 80).tolist()
    wl = workload(128, 16, 8, lens, 30, seed=17, masked_last=(7, 9))
    check_append(wl, "fp8_e4m3")


@pytest.mark.parametrize("qtype", ["fp8_e4m3", "q8_0"])
def test_append_qwen3_layer_all_rows(qtype):
    """8 x 16384 tokens, 16 q / 8 kv heads (the decode step's layer): the new
    token is the last position of each sequence."""
    check_append(W.qwen3(replicas=1), qtype)


def test_append_repeated_calls_are_stable():
    """The same append twice: the second call stores the same bytes again and
    returns the same bits (graph replays of a decode step do exactly this)."""
    k = kvq()
    wl = workload(128, 16, 8, [40, 1000, 17], 80, seed=23)
    pools = fill_both(wl, "fp8_e4m3")
    nk, nv = dev_bf16(new_rows(wl, 2, 0)), dev_bf16(new_rows(wl, 2, 1))
    q = dev_bf16(wl.query())
    pt, sl = dev_i32(wl.page_table), dev_i32(wl.seq_lens)
    args = (pools["kp"], pools["ks"], pools["vp"], pools["vs"], pt, sl, wl.sm_scale)
    say("append twice")
    o1, l1 = k.paged_decode_append("fp8_e4m3", q, nk, nv, *args)
    kp1 = pools["kp"].clone()
    o2, l2 = k.paged_decode_append("fp8_e4m3", q, nk, nv, *args, seq_lens_host=wl.seq_lens)
    torch.cuda.synchronize()
    assert torch.equal(bits(o1), bits(o2)) and torch.equal(bits(l1), bits(l2))
    assert torch.equal(kp1, pools["kp"])
