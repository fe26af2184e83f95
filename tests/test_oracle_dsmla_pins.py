"""Pins for the oracle's 656-byte MLA row (fp8_ds_mla): 512 e4m3fn codes,
four fp32 scales (one per 128 latent elements, amax / 448), 64 bf16 rope
elements, one row per token.

References, none of which re-types the oracle's formulas: numpy fp32
arithmetic for the scales and quotients, torch's float8_e4m3fn cast and
decode for the codes, the bf16 bits for the rope, and a numpy brute-force
softmax over the rows numpy decodes from the stored bytes.

Page key: [PR25] "Experimental FP8 KV Cache" (a 656-byte fp8 row for the
576-wide latent, laid out as in vLLM; the fields are the reading above).
"""
import numpy as np
import torch

import oracle

PAGE, D, DV = 16, 576, 512


def store(rows_bf16, n_pages):
    pool = np.zeros((n_pages, 1, PAGE, oracle.DS_ROW), np.uint8)
    oracle.store("fp8_ds_mla", rows_bf16, np.arange(rows_bf16.shape[0], dtype=np.int32), 1, D,
                 PAGE, n_pages, pool, None)
    return pool


def bf16_rows(rng, n, scale=1.0):
    x = rng.standard_normal((n, 1, D), dtype=np.float32) * scale
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def numpy_row_values(row_bytes):
    """Decode one stored row with numpy / torch only."""
    codes = torch.from_numpy(row_bytes[:512].copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    sc = row_bytes[512:528].copy().view(np.float32).astype(np.float64)
    rope = (row_bytes[528:656].copy().view(np.uint16).astype(np.uint32) << 16).view(np.float32)
    return np.concatenate([codes * np.repeat(sc, 128), rope.astype(np.float64)])


def test_row_fields_match_numpy_and_torch():
    rng = np.random.default_rng(1)
    src = bf16_rows(rng, 48, 3.0)
    src[5, 0, 128:256] = 0  # a zero tile
    pool = store(src, 3)
    flat = pool.reshape(-1, oracle.DS_ROW)
    for t in range(48):
        x = (src[t, 0].astype(np.uint32) << 16).view(np.float32)
        for j in range(4):
            tile = x[128 * j:128 * (j + 1)]
            sc = np.float32(np.abs(tile).max()) / np.float32(448.0)
            assert flat[t, 512 + 4 * j:516 + 4 * j].view(np.float32)[0] == sc
            if sc == 0:
                assert np.all(flat[t, 128 * j:128 * (j + 1)] == 0)
                continue
            q = (tile / sc).astype(np.float32)
            want = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(flat[t, 128 * j:128 * (j + 1)], want), (t, j)
        assert np.array_equal(flat[t, 528:656].view(np.uint16), src[t, 0, 512:])


def test_dequant_is_code_times_scale_and_the_rope():
    rng = np.random.default_rng(2)
    src = bf16_rows(rng, 32, 0.7)
    pool = store(src, 2)
    got, _ = oracle.dequant("fp8_ds_mla", pool, None, np.arange(32, dtype=np.int32), 1, D, PAGE, 2)
    flat = pool.reshape(-1, oracle.DS_ROW)
    for t in range(32):
        assert np.array_equal(got[t, 0], numpy_row_values(flat[t]))
    # the tile maximum is on the grid: it decodes to itself up to the scale's rounding
    x = (src[:, 0].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    err = np.abs(got[:, 0, :512] - x[:, :512]).max(axis=1) / np.abs(x[:, :512]).max(axis=1)
    assert err.max() < 2.0 ** -4  # e4m3: 3 fraction bits


def test_decode_brute_force():
    rng = np.random.default_rng(3)
    n_pages, L = 6, 83
    src = bf16_rows(rng, n_pages * PAGE)
    pool = store(src, n_pages)
    pt = np.array([[4, 0, 5, -1, 2, 1]], np.int32)
    q = bf16_rows(rng, 16)[:, 0][None]  # [1][16][576]
    sm = 0.06
    out, lse = oracle.paged_decode("fp8_ds_mla", q, pool, None, pool, None, pt,
                                   np.array([L], np.int32), 1, D, DV, PAGE, n_pages, sm)
    flat = pool.reshape(-1, oracle.DS_ROW)
    rows = [numpy_row_values(flat[pt[0, t // PAGE] * PAGE + t % PAGE]) for t in range(L)
            if pt[0, t // PAGE] >= 0]
    K = np.stack(rows)
    qv = (q[0].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    z = sm * qv @ K.T
    zm = z.max(axis=1, keepdims=True)
    w = np.exp(z - zm)
    ref = (w @ K[:, :DV]) / w.sum(axis=1, keepdims=True)
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-13)
    assert np.allclose(lse, zm[:, 0] + np.log(w.sum(axis=1)), rtol=1e-12)
