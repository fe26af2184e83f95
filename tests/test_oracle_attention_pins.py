"""Pins for the oracle's store placement, dequant and paged decode attention.

References: brute-force float64 attention in numpy over K/V dequantized with
library decoders (torch float8_e4m3fn, numpy float16), special cases with
closed-form answers (one valid token, identical keys), and invariances the
method must have (masked pages vs. the compacted sequence, physical page
permutation, split-and-merge of the softmax, the shared MLA slab vs. a
separate V pool holding the same leading columns).

Page keys used in citations:
  [PR103] "feat(kvcache): 8-bit KV cache (q8_0 / fp8_e4m3) behind --kv-cache-dtype"
  [PR113] "feat(kvcache): 8-bit DSV4 window/compressed KV behind --kv-cache-dtype"
"""
import numpy as np
import pytest
import torch

import oracle
from tests.test_oracle_pins import bf16_bits, bf16_to_f32, e4m3_lib_value, f16_value

PS = 16


def make_pool(qtype, n_pages, H, D, rng, scale=1.0):
    """Fill a pool through oracle.store from random bf16 rows; return pool, scales, src."""
    n_slots = n_pages * PS
    src = bf16_bits((rng.standard_normal((n_slots, H, D)) * scale).astype(np.float32))
    if qtype == "bf16":
        pool = np.zeros((n_pages, H, PS, D), np.uint16)
        scales = None
    else:
        pool = np.zeros((n_pages, H, PS, D), np.uint8)
        scales = np.zeros((n_pages, H, PS, D // 32), np.uint16)
    oracle.store(qtype, src, np.arange(n_slots, dtype=np.int32), H, D, PS, n_pages, pool, scales)
    return pool, scales, src


def lib_dequant_pool(qtype, pool, scales):
    """[pages][H][PS][D] float64 values via library decoders."""
    if qtype == "bf16":
        return bf16_to_f32(pool).astype(np.float64)
    D = pool.shape[-1]
    s = np.repeat(f16_value(scales), 32, axis=-1)[..., :D]
    if qtype == "fp8_e4m3":
        return e4m3_lib_value(pool) * s
    return pool.view(np.int8).astype(np.float64) * s


def brute_attention(qtype, q_bits, kpool, ks, vpool, vs, pt, seq_lens, Hkv, sm_scale, Dv,
                    shared=False):
    kv = lib_dequant_pool(qtype, kpool, ks)
    vv = kv[..., :Dv] if shared else lib_dequant_pool(qtype, vpool, vs)
    q = bf16_to_f32(q_bits).astype(np.float64)
    B, Hq, _ = q.shape
    G = Hq // Hkv
    n_pages = kpool.shape[0]
    out = np.zeros((B, Hq, Dv))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        L = min(int(seq_lens[b]), pt.shape[1] * PS)
        t = np.arange(L)
        pages = pt[b, t // PS]
        ok = (pages >= 0) & (pages < n_pages)
        t, pages = t[ok], pages[ok]
        if len(t) == 0:
            continue
        for h in range(Hq):
            g = h // G
            K = kv[pages, g, t % PS]
            V = vv[pages, g, t % PS]
            z = sm_scale * (K @ q[b, h])
            m = z.max()
            w = np.exp(z - m)
            out[b, h] = (w @ V) / w.sum()
            lse[b, h] = m + np.log(w.sum())
    return out, lse


def run_oracle(qtype, q_bits, kpool, ks, vpool, vs, pt, seq_lens, Hkv, sm_scale, Dqk, Dv,
               n_pages):
    o, l = oracle.paged_decode(qtype, q_bits, kpool, ks, vpool, vs, pt, seq_lens, Hkv, Dqk, Dv,
                               PS, n_pages, sm_scale)
    B, Hq = q_bits.shape[:2]
    return o.reshape(B, Hq, Dv), l.reshape(B, Hq)


@pytest.mark.parametrize("qtype", ["fp8_e4m3", "q8_0", "bf16"])
@pytest.mark.parametrize("D,Hq,Hkv", [(32, 2, 1), (64, 4, 2), (64, 2, 2)])
def test_decode_matches_brute_force(qtype, D, Hq, Hkv):
    rng = np.random.default_rng(hash((qtype, D, Hq, Hkv)) % 2**32)
    n_pages = 9
    kpool, ks, _ = make_pool(qtype, n_pages, Hkv, D, rng)
    vpool, vs, _ = make_pool(qtype, n_pages, Hkv, D, rng)
    B = 2
    pt = np.full((B, 3), -1, np.int32)
    perm = rng.permutation(n_pages)
    pt[0] = perm[:3]
    pt[1, :2] = perm[3:5]
    pt[1, 2] = -1  # masked column inside the sequence
    seq_lens = np.array([40, 37], np.int32)  # ragged tails
    q = bf16_bits(rng.standard_normal((B, Hq, D)).astype(np.float32))
    sm = 1 / np.sqrt(D)
    o, l = run_oracle(qtype, q, kpool, ks, vpool, vs, pt, seq_lens, Hkv, sm, D, D, n_pages)
    ro, rl = brute_attention(qtype, q, kpool, ks, vpool, vs, pt, seq_lens, Hkv, sm, D)
    np.testing.assert_allclose(o, ro, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l, rl, rtol=1e-12, atol=1e-12)


def test_single_valid_token_and_identical_keys():
    rng = np.random.default_rng(21)
    D, H = 64, 1
    kpool, ks, _ = make_pool("fp8_e4m3", 2, H, D, rng)
    vpool, vs, _ = make_pool("fp8_e4m3", 2, H, D, rng)
    q = bf16_bits(rng.standard_normal((1, 1, D)).astype(np.float32))
    pt = np.array([[1, 0]], np.int32)
    o, l = run_oracle("fp8_e4m3", q, kpool, ks, vpool, vs, pt, np.array([1], np.int32), 1, 0.125,
                      D, D, 2)
    V = lib_dequant_pool("fp8_e4m3", vpool, vs)
    K = lib_dequant_pool("fp8_e4m3", kpool, ks)
    np.testing.assert_allclose(o[0, 0], V[1, 0, 0], rtol=0, atol=1e-15)
    z = 0.125 * (K[1, 0, 0] @ bf16_to_f32(q[0, 0]).astype(np.float64))
    np.testing.assert_allclose(l[0, 0], z, rtol=1e-13)
    # identical keys: every token of page 0 gets the same K row -> o = mean of V rows
    kpool2 = kpool.copy()
    ks2 = ks.copy()
    kpool2[0, 0, :] = kpool[0, 0, 3]
    ks2[0, 0, :] = ks[0, 0, 3]
    o2, l2 = run_oracle("fp8_e4m3", q, kpool2, ks2, vpool, vs, np.array([[0, 1]], np.int32),
                        np.array([16], np.int32), 1, 0.125, D, D, 2)
    np.testing.assert_allclose(o2[0, 0], V[0, 0].mean(axis=0), rtol=1e-12, atol=1e-14)
    z = 0.125 * (K[0, 0, 3] @ bf16_to_f32(q[0, 0]).astype(np.float64))
    np.testing.assert_allclose(l2[0, 0], z + np.log(16), rtol=1e-12)


def test_masked_page_equals_compacted_sequence_and_empty_is_zero():
    """[PR113 §Testing]: a -1 page-table column removes that page."""
    rng = np.random.default_rng(22)
    D, Hkv, Hq, n_pages = 64, 2, 4, 6
    kpool, ks, _ = make_pool("q8_0", n_pages, Hkv, D, rng)
    vpool, vs, _ = make_pool("q8_0", n_pages, Hkv, D, rng)
    q = bf16_bits(rng.standard_normal((3, Hq, D)).astype(np.float32))
    pt = np.array([[4, -1, 2, 5], [4, 2, 5, -1], [-1, -1, -1, -1]], np.int32)
    seq = np.array([16 * 3 + 9, 16 * 2 + 9, 50], np.int32)
    o, l = run_oracle("q8_0", q, kpool, ks, vpool, vs, pt, seq, Hkv, 0.1, D, D, n_pages)
    # row 0 (page 2 of the walk masked) == row 1's compacted walk, same query
    q2 = q.copy()
    q2[1] = q[0]
    o2, l2 = run_oracle("q8_0", q2, kpool, ks, vpool, vs, pt, seq, Hkv, 0.1, D, D, n_pages)
    assert np.array_equal(o2[1], o[0]) and np.array_equal(l2[1], l[0])
    assert np.all(o[2] == 0) and np.all(np.isneginf(l[2]))


def test_page_permutation_invariance_and_out_of_range_pages():
    rng = np.random.default_rng(23)
    D, Hkv, Hq, n_pages = 32, 1, 2, 5
    kpool, ks, _ = make_pool("fp8_e4m3", n_pages, Hkv, D, rng)
    vpool, vs, _ = make_pool("fp8_e4m3", n_pages, Hkv, D, rng)
    q = bf16_bits(rng.standard_normal((1, Hq, D)).astype(np.float32))
    pt = np.array([[3, 0, 4, 1]], np.int32)
    seq = np.array([60], np.int32)
    o, l = run_oracle("fp8_e4m3", q, kpool, ks, vpool, vs, pt, seq, Hkv, 0.2, D, D, n_pages)
    perm = rng.permutation(n_pages)  # physical page p moves to perm[p]
    kp2, ks2, vp2, vs2 = (np.empty_like(a) for a in (kpool, ks, vpool, vs))
    kp2[perm], ks2[perm], vp2[perm], vs2[perm] = kpool, ks, vpool, vs
    o2, l2 = run_oracle("fp8_e4m3", q, kp2, ks2, vp2, vs2, perm[pt], seq, Hkv, 0.2, D, D, n_pages)
    assert np.array_equal(o, o2) and np.array_equal(l, l2)
    # an id >= num_pages behaves as -1
    pt3 = pt.copy()
    pt3[0, 2] = n_pages + 7
    pt4 = pt.copy()
    pt4[0, 2] = -1
    o3, _ = run_oracle("fp8_e4m3", q, kpool, ks, vpool, vs, pt3, seq, Hkv, 0.2, D, D, n_pages)
    o4, _ = run_oracle("fp8_e4m3", q, kpool, ks, vpool, vs, pt4, seq, Hkv, 0.2, D, D, n_pages)
    assert np.array_equal(o3, o4)


def test_split_and_merge_identity():
    """Softmax over a sequence equals the log-sum-exp merge of its two halves."""
    rng = np.random.default_rng(24)
    D, Hkv, Hq, n_pages = 64, 1, 2, 8
    kpool, ks, _ = make_pool("fp8_e4m3", n_pages, Hkv, D, rng)
    vpool, vs, _ = make_pool("fp8_e4m3", n_pages, Hkv, D, rng)
    q = bf16_bits(rng.standard_normal((1, Hq, D)).astype(np.float32))
    qq = np.concatenate([q, q, q])
    pt = np.array([[0, 1, 2, 3, 4, 5], [0, 1, 2, -1, -1, -1], [5, 4, 3, -1, -1, -1]], np.int32)
    # second half of row 0 is pages 3,4,5 with 16+16+7 tokens; reorder pages to express it
    pt[2] = [3, 4, 5, -1, -1, -1]
    seq = np.array([16 * 5 + 7, 48, 16 * 2 + 7], np.int32)
    o, l = run_oracle("fp8_e4m3", qq, kpool, ks, vpool, vs, pt, seq, Hkv, 0.125, D, D, n_pages)
    m = np.maximum(l[1], l[2])
    w1, w2 = np.exp(l[1] - m), np.exp(l[2] - m)
    merged = (w1[:, None] * o[1] + w2[:, None] * o[2]) / (w1 + w2)[:, None]
    np.testing.assert_allclose(o[0], merged, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l[0], m + np.log(w1 + w2), rtol=1e-13)


def test_shared_mla_slab_equals_separate_leading_columns():
    """[PR113 §What this adds]: K and V are one row; V is its first Dv columns."""
    rng = np.random.default_rng(25)
    Dqk, Dv, Hq, n_pages = 96, 64, 4, 4
    pool, sc, _ = make_pool("fp8_e4m3", n_pages, 1, Dqk, rng)
    vpool = np.ascontiguousarray(pool[..., :Dv])
    vsc = np.ascontiguousarray(sc[..., : Dv // 32])
    q = bf16_bits(rng.standard_normal((1, Hq, Dqk)).astype(np.float32))
    pt = np.array([[2, 0, 3]], np.int32)
    seq = np.array([41], np.int32)
    o1, l1 = oracle.paged_decode("fp8_e4m3", q, pool, sc, pool, sc, pt, seq, 1, Dqk, Dv, PS,
                                 n_pages, 1 / 24)
    o2, l2 = oracle.paged_decode("fp8_e4m3", q, pool, sc, vpool, vsc, pt, seq, 1, Dqk, Dv, PS,
                                 n_pages, 1 / 24)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    ro, rl = brute_attention("fp8_e4m3", q, pool, sc, None, None, pt, seq, 1, 1 / 24, Dv,
                             shared=True)
    np.testing.assert_allclose(o1.reshape(ro.shape), ro, rtol=1e-12, atol=1e-12)


def test_store_places_rows_and_skips_invalid_slots():
    rng = np.random.default_rng(26)
    H, D, n_pages = 3, 64, 4
    n = 10
    src = bf16_bits(rng.standard_normal((n, H, D)).astype(np.float32))
    slots = np.array([5, 63, 0, -1, 64, 17, 999, 31, 32, 48], np.int32)
    pool = np.full((n_pages, H, PS, D), 0xAA, np.uint8)
    sc = np.full((n_pages, H, PS, D // 32), 0x5555, np.uint16)
    oracle.store("fp8_e4m3", src, slots, H, D, PS, n_pages, pool, sc)
    touched = np.zeros((n_pages, PS), bool)
    for i, s in enumerate(slots):
        if 0 <= s < n_pages * PS:
            p, o = divmod(int(s), PS)
            touched[p, o] = True
            for h in range(H):
                for j in range(D // 32):
                    codes, sb = oracle.quantize_block("fp8_e4m3", src[i, h, 32 * j: 32 * j + 32])
                    assert np.array_equal(pool[p, h, o, 32 * j: 32 * j + 32], codes)
                    assert sc[p, h, o, j] == sb
    untouched = ~touched
    assert np.all(pool.transpose(0, 2, 1, 3)[untouched] == 0xAA)
    assert np.all(sc.transpose(0, 2, 1, 3)[untouched] == 0x5555)
    # bf16 store is a plain copy
    pb = np.zeros((n_pages, H, PS, D), np.uint16)
    oracle.store("bf16", src, slots, H, D, PS, n_pages, pb, None)
    assert np.array_equal(pb[0, :, 5], src[0])


def test_dequant_gather_matches_library_decode():
    rng = np.random.default_rng(27)
    H, D, n_pages = 2, 64, 3
    for qtype in ("fp8_e4m3", "q8_0"):
        pool, sc, _ = make_pool(qtype, n_pages, H, D, rng, scale=3.0)
        slots = np.array([0, 47, -1, 20, 48], np.int32)
        f64, b16 = oracle.dequant(qtype, pool, sc, slots, H, D, PS, n_pages)
        ref = lib_dequant_pool(qtype, pool, sc)
        for i, s in enumerate(slots):
            if 0 <= s < n_pages * PS:
                p, o = divmod(int(s), PS)
                assert np.array_equal(f64[i], ref[p, :, o])
            else:
                assert np.all(f64[i] == 0)
        assert np.array_equal(b16, bf16_bits(f64.astype(np.float32)))
