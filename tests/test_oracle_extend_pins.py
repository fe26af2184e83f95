"""Pins for the oracle's causal extend (prefill) attention over the pool.

References: a numpy brute-force causal softmax over rows the oracle's own
(pinned) dequant returns, the causality the definition implies (rows past a
token's position change nothing for it), and the decode (pinned in
test_oracle_attention_pins) for the last new token of each sequence.

Page keys: [PR103] "feat(kvcache): 8-bit KV cache (q8_0 / fp8_e4m3) behind
--kv-cache-dtype" (§What: the quantized pool feeds the prefill / extend
attention kernels as well as the decode); [PR113] "feat(kvcache): 8-bit
DSV4 window/compressed KV behind --kv-cache-dtype" (§Testing: prefill,
masked (-1) columns).
"""
import numpy as np
import pytest

import oracle

PAGE = 16


def case(seed, lens, news, Hq=8, Hkv=2, D=64, qtype="fp8_e4m3", mask_frac=0.15):
    """A pool holding every sequence's tokens (pages drawn from one
    permutation, some masked) and the queries of each sequence's new tokens."""
    rng = np.random.default_rng(seed)
    lens = np.array(lens, np.int32)
    width = max(1, max((int(L) + PAGE - 1) // PAGE for L in lens))
    need = sum((int(L) + PAGE - 1) // PAGE for L in lens)
    n_pages = need + 3
    perm = rng.permutation(n_pages).astype(np.int32)
    pt = np.full((len(lens), width), -1, np.int32)
    o = 0
    for b, L in enumerate(lens):
        n = (int(L) + PAGE - 1) // PAGE
        pt[b, :n] = perm[o:o + n]
        o += n
        pt[b, :n][rng.random(n) < mask_frac] = -1
    code_t = np.uint16 if qtype == "bf16" else np.uint8
    pools = []
    for _ in range(2):
        rows = rng.standard_normal((n_pages * PAGE, Hkv, D), dtype=np.float32) * 1.5
        bits = (rows.view(np.uint32) >> 16).astype(np.uint16)
        pool = np.zeros((n_pages, Hkv, PAGE, D), code_t)
        sc = (np.zeros((n_pages, Hkv, PAGE, D // 32), np.uint16) if qtype in oracle.SCALED
              else None)
        oracle.store(qtype, bits, np.arange(n_pages * PAGE, dtype=np.int32), Hkv, D, PAGE,
                     n_pages, pool, sc)
        pools.append((pool, sc))
    q_start = np.concatenate([[0], np.cumsum(news)]).astype(np.int32)
    T = int(q_start[-1])
    q = (rng.standard_normal((T, Hq, D), dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return dict(lens=lens, pt=pt, pools=pools, q=q, q_start=q_start, n_pages=n_pages, Hq=Hq,
                Hkv=Hkv, D=D, qtype=qtype)


def extend(c, sm=0.1):
    (kp, ks), (vp, vs) = c["pools"]
    return oracle.extend_attention(c["qtype"], c["q"], c["q_start"], kp, ks, vp, vs, c["pt"],
                                   c["lens"], c["Hkv"], c["D"], PAGE, c["n_pages"], sm)


def brute(c, sm=0.1):
    """Softmax attention in numpy over the positions each new token may see."""
    (kp, ks), (vp, vs) = c["pools"]
    Hq, Hkv, D = c["Hq"], c["Hkv"], c["D"]
    G = Hq // Hkv
    qv = (c["q"].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    T = qv.shape[0]
    out = np.zeros((T * Hq, D))
    lse = np.full(T * Hq, -np.inf)
    for b, L in enumerate(c["lens"]):
        s0, s1 = int(c["q_start"][b]), int(c["q_start"][b + 1])
        E = s1 - s0
        for i in range(E):
            pos = int(L) - E + i
            slots = [int(c["pt"][b, t // PAGE]) * PAGE + t % PAGE for t in range(max(pos + 1, 0))
                     if c["pt"][b, t // PAGE] >= 0]
            if not slots:
                continue
            K, _ = oracle.dequant(c["qtype"], kp, ks, np.array(slots, np.int32), Hkv, D, PAGE,
                                  c["n_pages"])
            V, _ = oracle.dequant(c["qtype"], vp, vs, np.array(slots, np.int32), Hkv, D, PAGE,
                                  c["n_pages"])
            for h in range(Hq):
                z = sm * (K[:, h // G, :] @ qv[s0 + i, h])
                zm = z.max()
                w = np.exp(z - zm)
                r = (s0 + i) * Hq + h
                out[r] = (w @ V[:, h // G, :]) / w.sum()
                lse[r] = zm + np.log(w.sum())
    return out, lse


@pytest.mark.parametrize("qtype", ["fp8_e4m3", "q8_0", "bf16", "fp8_e5m2_cast"])
def test_brute_force_causal_softmax(qtype):
    """Prefill (no prefix), extends after a prefix, a sequence whose new
    tokens outnumber its pool (the first ones see nothing), masked pages and
    an empty sequence."""
    c = case(1, [40, 70, 3, 0, 33], [40, 5, 5, 0, 1], qtype=qtype)
    o, l = extend(c)
    ro, rl = brute(c)
    assert np.allclose(o, ro, rtol=1e-10, atol=1e-12)
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(l), fin)
    assert np.allclose(l[fin], rl[fin], rtol=1e-12)
    # tokens at negative positions (sequence 2: 5 new tokens, 3 in the pool)
    s0 = int(c["q_start"][2])
    Hq = c["Hq"]
    assert np.all(o[s0 * Hq:(s0 + 2) * Hq] == 0)
    assert np.all(np.isneginf(l[s0 * Hq:(s0 + 2) * Hq]))


def test_rows_past_a_token_change_nothing_for_it():
    c = case(2, [50], [12], mask_frac=0.0)
    o0, l0 = extend(c)
    (kp, ks), (vp, vs) = c["pools"]
    L, E = 50, 12
    cut = L - E + 5  # positions > cut are invisible to new tokens 0..5
    for t in range(cut + 1, L):
        s = int(c["pt"][0, t // PAGE]) * PAGE + t % PAGE
        page, row = divmod(s, PAGE)
        kp[page, :, row, :] = kp[page, :, row, ::-1].copy()
        vp[page, :, row, :] = vp[page, :, row, ::-1].copy()
    o1, l1 = extend(c)
    Hq = c["Hq"]
    seen = 6 * Hq  # rows of tokens 0..5
    assert np.array_equal(o0[:seen], o1[:seen]) and np.array_equal(l0[:seen], l1[:seen])
    assert not np.array_equal(o0[seen:], o1[seen:])


def test_last_new_token_is_the_decode():
    """The last new token sits at position L - 1: it sees the whole sequence,
    as the decode's query does."""
    c = case(3, [90, 17, 64], [7, 17, 1], Hq=8, Hkv=1)
    o, l = extend(c)
    (kp, ks), (vp, vs) = c["pools"]
    last = c["q_start"][1:] - 1
    qd = c["q"][last]
    od, ld = oracle.paged_decode(c["qtype"], qd, kp, ks, vp, vs, c["pt"], c["lens"], c["Hkv"],
                                 c["D"], c["D"], PAGE, c["n_pages"], 0.1)
    Hq = c["Hq"]
    rows = np.concatenate([np.arange(j * Hq, (j + 1) * Hq) for j in last])
    assert np.array_equal(o[rows], od) and np.array_equal(l[rows], ld)


def test_mla_slab_extend_brute_force():
    """The shared 576/512 slab: each new token's causal softmax over the
    rows it may see, K the whole row, V its first 512 elements."""
    rng = np.random.default_rng(9)
    lens, news = np.array([70, 40], np.int32), [5, 40]
    n_pages = 8
    pt = np.array([[3, 0, 6, 1, 7], [2, 5, 4, -1, -1]], np.int32)
    rows = (rng.standard_normal((n_pages * PAGE, 1, 576), dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    pool = np.zeros((n_pages, 1, PAGE, 576), np.uint8)
    sc = np.zeros((n_pages, 1, PAGE, 18), np.uint16)
    oracle.store("fp8_e4m3", rows, np.arange(n_pages * PAGE, dtype=np.int32), 1, 576, PAGE, n_pages, pool, sc)
    q_start = np.array([0, 5, 45], np.int32)
    q = (rng.standard_normal((45, 16, 576), dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    sm = 0.05
    out, lse = oracle.extend_attention("fp8_e4m3", q, q_start, pool, sc, pool, sc, pt, lens, 1, 576,
                                       PAGE, n_pages, sm, head_dim_v=512)
    qv = (q.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for b in range(2):
        E = news[b]
        for i in range(E):
            pos = int(lens[b]) - E + i
            slots = [int(pt[b, t // PAGE]) * PAGE + t % PAGE for t in range(pos + 1)]
            K, _ = oracle.dequant("fp8_e4m3", pool, sc, np.array(slots, np.int32), 1, 576, PAGE, n_pages)
            j = int(q_start[b]) + i
            z = sm * (qv[j] @ K[:, 0, :].T)              # [16 heads, n]
            zm = z.max(axis=1, keepdims=True)
            w = np.exp(z - zm)
            ref = (w @ K[:, 0, :512]) / w.sum(axis=1, keepdims=True)
            assert np.allclose(out[j * 16:(j + 1) * 16], ref, rtol=1e-10, atol=1e-12)
            assert np.allclose(lse[j * 16:(j + 1) * 16], zm[:, 0] + np.log(w.sum(axis=1)), rtol=1e-12)
