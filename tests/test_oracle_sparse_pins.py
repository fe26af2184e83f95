"""Pins for the oracle's sparse top-k decode over the shared MLA slab.

References: the dense slab decode (itself pinned in test_oracle_attention_pins)
for a list that names every position of the sequence, the invariances the
definition implies (entries that are skipped change nothing, the order of the
list changes only rounding), and a brute-force softmax in numpy over rows
dequantized by the oracle's own (pinned) dequant.

Page keys: [PR25] "Experimental FP8 KV Cache" (SPARSE_MLA_DECODE: D=576,
Hq=128, Hkv=1, Dv=512, K=256 tokens per query); [PR113] "feat(kvcache):
8-bit DSV4 window/compressed KV behind --kv-cache-dtype" (§What this adds: K
and V the same row; §Testing: masked (-1) columns).
"""
import numpy as np
import pytest

import oracle

PAGE, DQK, DV = 16, 576, 512


def slab_case(seed, lens, width, mask_frac=0.2, qtype="fp8_e4m3", Hq=16):
    rng = np.random.default_rng(seed)
    lens = np.array(lens, np.int32)
    need = sum((int(L) + PAGE - 1) // PAGE for L in lens)
    n_pages = need + 4
    perm = rng.permutation(n_pages).astype(np.int32)
    pt = np.full((len(lens), width), -1, np.int32)
    o = 0
    for b, L in enumerate(lens):
        n = (int(L) + PAGE - 1) // PAGE
        pt[b, :n] = perm[o:o + n]
        o += n
        pt[b, :n][rng.random(n) < mask_frac] = -1
    rows = rng.standard_normal((n_pages * PAGE, 1, DQK), dtype=np.float32) * 2
    bits = (rows.view(np.uint32) >> 16).astype(np.uint16)  # truncation to bf16: any bf16 will do
    pool = np.zeros((n_pages, 1, PAGE, DQK), np.uint8 if qtype != "bf16" else np.uint16)
    scales = (np.zeros((n_pages, 1, PAGE, DQK // 32), np.uint16) if qtype in oracle.SCALED
              else None)
    oracle.store(qtype, bits, np.arange(n_pages * PAGE, dtype=np.int32), 1, DQK, PAGE, n_pages,
                 pool, scales)
    q = (rng.standard_normal((len(lens), Hq, DQK), dtype=np.float32).view(np.uint32) >> 16
         ).astype(np.uint16)
    return dict(rng=rng, lens=lens, pt=pt, pool=pool, scales=scales, q=q, n_pages=n_pages,
                qtype=qtype)


def sparse(c, topk, sm=0.04):
    return oracle.sparse_mla_decode(c["qtype"], c["q"], c["pool"], c["scales"], c["pt"], c["lens"],
                                    np.asarray(topk, np.int32), DQK, DV, PAGE, c["n_pages"], sm)


def dense(c, sm=0.04):
    return oracle.paged_decode(c["qtype"], c["q"], c["pool"], c["scales"], c["pool"], c["scales"],
                               c["pt"], c["lens"], 1, DQK, DV, PAGE, c["n_pages"], sm)


@pytest.mark.parametrize("qtype", ["fp8_e4m3", "q8_0", "bf16", "fp8_e5m2_cast"])
def test_a_list_of_every_position_is_the_dense_decode(qtype):
    c = slab_case(1, [0, 5, 40, 333], 25, qtype=qtype)
    K = int(c["lens"].max())
    topk = np.full((len(c["lens"]), K), -1, np.int32)
    for b, L in enumerate(c["lens"]):
        topk[b, :L] = np.arange(L)
    o_s, l_s = sparse(c, topk)
    o_d, l_d = dense(c)
    assert np.array_equal(o_s, o_d)
    assert np.array_equal(l_s, l_d)


def test_skipped_entries_change_nothing():
    """-1, positions at or past the length, and positions on masked pages."""
    c = slab_case(2, [200, 77], 16)
    rng = c["rng"]
    base = np.stack([rng.choice(int(L), 60, replace=False) for L in c["lens"]]).astype(np.int32)
    o0, l0 = sparse(c, base)
    extra = []
    for b, L in enumerate(c["lens"]):
        masked = [t for t in range(int(L)) if c["pt"][b, t // PAGE] < 0][:5]
        junk = [-1, -7, int(L), int(L) + 3, 10 ** 6] + masked
        extra.append(junk + [-1] * (10 - len(junk)))
    padded = np.concatenate([base, np.array(extra, np.int32)], axis=1)
    o1, l1 = sparse(c, padded)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


def test_list_order_changes_only_rounding():
    c = slab_case(3, [500], 40)
    rng = c["rng"]
    topk = rng.choice(500, 256, replace=False).astype(np.int32)[None]
    o0, l0 = sparse(c, topk)
    o1, l1 = sparse(c, topk[:, rng.permutation(256)])
    assert np.allclose(o0, o1, rtol=1e-12, atol=1e-14)
    assert np.allclose(l0, l1, rtol=1e-13)


def test_brute_force_with_duplicates_and_no_taken_entry():
    """Softmax attention in numpy over the taken rows (a duplicate taken
    twice), from rows the oracle's dequant returns; a list with nothing to
    take gives zeros and -inf."""
    c = slab_case(4, [90, 30], 8, mask_frac=0.3, Hq=16)
    rng = c["rng"]
    lists = []
    for b, L in enumerate(c["lens"]):
        t = rng.choice(int(L), 12, replace=False)
        lists.append(np.concatenate([t, t[:3], [-1, int(L)]]).astype(np.int32))
    topk = np.stack(lists)
    topk[1, :] = -1  # sequence 1 lists nothing
    sm = 0.05
    out, lse = sparse(c, topk, sm)
    qv = (c["q"].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for b in range(2):
        slots = []
        for t in topk[b]:
            if 0 <= t < c["lens"][b] and c["pt"][b, t // PAGE] >= 0:
                slots.append(int(c["pt"][b, t // PAGE]) * PAGE + int(t) % PAGE)
        Hq = qv.shape[1]
        if not slots:
            assert np.all(out[b * Hq:(b + 1) * Hq] == 0)
            assert np.all(np.isneginf(lse[b * Hq:(b + 1) * Hq]))
            continue
        rows, _ = oracle.dequant(c["qtype"], c["pool"], c["scales"], np.array(slots, np.int32), 1,
                                 DQK, PAGE, c["n_pages"])
        K = rows[:, 0, :]                       # [n, 576]
        z = sm * qv[b] @ K.T                    # [Hq, n]
        zm = z.max(axis=1, keepdims=True)
        w = np.exp(z - zm)
        ref = (w @ K[:, :DV]) / w.sum(axis=1, keepdims=True)
        assert np.allclose(out[b * Hq:(b + 1) * Hq], ref, rtol=1e-10, atol=1e-12)
        assert np.allclose(lse[b * Hq:(b + 1) * Hq], (zm[:, 0] + np.log(w.sum(axis=1))),
                           rtol=1e-12)
