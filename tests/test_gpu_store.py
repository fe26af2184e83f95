"""GPU parity of kvq_store and kvq_dequant against the oracle: bit-exact codes,
fp16 scales and bf16 rows.

Page keys: [PR103] "feat(kvcache): 8-bit KV cache (q8_0 / fp8_e4m3) behind
--kv-cache-dtype" (§What; review comment §"A bug on sm_89": the arch-specific
fp8 cast is exactly what must be checked on the target GPU); [PR113]
"feat(kvcache): 8-bit DSV4 window/compressed KV behind --kv-cache-dtype"
(§Testing: saturation, the already-on-grid regime).
"""
import numpy as np
import pytest
import torch

import oracle
from paged_decode_attention_amd import workloads as W
from tests.gpu_util import (dev_bf16, dev_i32, host_u16, host_u8, kvq, np_pool, requires_gpu,
                            say)

pytestmark = [pytest.mark.gpu, requires_gpu]

QT8 = ["fp8_e4m3", "q8_0"]
CASTS = ["fp8_e4m3_cast", "fp8_e5m2_cast"]


def tricky_rows(rng, n, H, D):
    """bf16 rows mixing magnitudes from fp16-subnormal scales to saturating
    ones, all-zero and constant blocks, +-1e4 outliers, +-inf elements and
    exact ties."""
    x = rng.standard_normal((n, H, D), dtype=np.float32)
    mag = np.exp2(rng.uniform(-30, 28, (n, H, 1))).astype(np.float32)
    x *= np.where(rng.random((n, H, 1)) < 0.5, 1.0, mag)
    blocks = x.reshape(n, H, D // 32, 32)
    pick = rng.random(blocks.shape[:-1])
    blocks[pick < 0.03] = 0.0
    const = (pick >= 0.03) & (pick < 0.06)
    blocks[const] = rng.standard_normal(int(const.sum()), dtype=np.float32)[:, None]
    out = rng.random(x.shape) < 0.002
    x[out] = np.where(rng.random(int(out.sum())) < 0.5, -1e4, 1e4)
    # infinities saturate: the block's scale is held at 65504, the element
    # stores +-M (a wrong sign here once came from inf - inf in the quotient)
    inf = rng.random(x.shape) < 0.0005
    x[inf] = np.where(rng.random(int(inf.sum())) < 0.5, -np.inf, np.inf)
    bits = W.to_bf16_bits(x)
    # exact ties: block max 448*s (resp. 127*s), others on code midpoints times s
    grid = np.array([oracle.e4m3_value(c) for c in range(0x7F)])
    mids8 = (grid[:-1] + grid[1:]) / 2
    tb = bits.reshape(n, H, D // 32, 32)
    sel = rng.random(tb.shape[:-1]) < 0.05
    for idx in zip(*np.nonzero(sel)):
        k = int(rng.integers(-10, 4))
        if rng.random() < 0.5:
            s = rng.choice([1.5, 1.75]) * 2.0 ** k
            v = np.concatenate([[448 * s], rng.choice(mids8, 31) * s * rng.choice([-1, 1], 31)])
        else:
            s = 2.0 ** k
            v = np.concatenate([[127 * s], (rng.integers(0, 127, 31) + 0.5) * s *
                                rng.choice([-1, 1], 31)])
        tb[idx] = W.to_bf16_bits(v.astype(np.float32))
    return bits


@pytest.mark.parametrize("qtype", ["fp8_e4m3", "q8_0", "bf16"] + CASTS)
@pytest.mark.parametrize("H,D", [(1, 32), (2, 64), (8, 128), (2, 256), (1, 576), (3, 96)])
def test_store_bitexact(qtype, H, D):
    rng = np.random.default_rng(1000 + D + H)
    n_pages, n = 23, 300
    cap = n_pages * W.PAGE
    slots = rng.permutation(cap)[:n].astype(np.int32)
    slots[rng.random(n) < 0.05] = -1
    slots[rng.random(n) < 0.03] = cap + 5  # beyond capacity: skipped
    src = tricky_rows(rng, n, H, D)
    k = kvq()
    kp, ks = k.alloc_pool(qtype, n_pages, H, D)
    okp, oks = np_pool(qtype, n_pages, H, D, fill_code=0xA5, fill_scale=0x5A5A)
    if qtype == "bf16":
        kp.view(torch.int16).fill_(0x5A5A)
    else:
        kp.fill_(0xA5)
        if ks is not None:
            ks.fill_(0x5A5A)
    say("store_bitexact", qtype, H, D)
    k.store(qtype, dev_bf16(src), None, dev_i32(slots), kp, ks)
    torch.cuda.synchronize()
    oracle.store(qtype, src, slots, H, D, W.PAGE, n_pages, okp, oks)
    if qtype == "bf16":
        assert np.array_equal(host_u16(kp), okp)
    else:
        got_c = host_u8(kp)
        got_s = host_u16(ks) if ks is not None else None
        bad = np.nonzero(got_c != okp)
        assert bad[0].size == 0, "first code mismatch at %s: gpu %#x oracle %#x" % (
            [int(b[0]) for b in bad], got_c[bad][0], okp[bad][0])
        if oks is not None:
            assert np.array_equal(got_s, oks)
        else:
            assert ks is None


def test_device_e4m3_encoder_over_every_fp32_in_range():
    """The device's fp32 -> e4m3 encoder (clamp, then the gfx950 packed RNE
    conversion; every stored e4m3 code goes through it, including the 656-byte
    row's quotients by an fp32 scale, which take arbitrary fp32 values) on
    every fp32 in [-448, 448], against the oracle's encoder.  The conversion
    is what differs per architecture [PR103 "feat(kvcache): 8-bit KV cache
    (q8_0 / fp8_e4m3) behind --kv-cache-dtype", review §"A bug on sm_89"]."""
    k = kvq()
    top = 0x43E00000  # 448.0f; patterns 0 .. top are the magnitudes in [0, 448]
    chunk = 1 << 28
    out = torch.empty(chunk, dtype=torch.uint8, device="cuda")
    for sign in (0, 0x80000000):
        for lo in range(0, top + 1, chunk):
            n = min(chunk, top + 1 - lo)
            n4 = (n + 3) // 4 * 4  # the last quad may run up to 3 patterns past 448
            say("e4m3 sweep", hex(sign + lo), n)
            k.debug_e4m3_encode_range(sign + lo, n4, out[:n4])
            got = out[:n].cpu().numpy()
            exp = oracle.e4m3_encode_bits(sign + lo, n)
            bad = np.nonzero(got != exp)[0]
            assert bad.size == 0, "bits %#010x: gpu %#04x oracle %#04x (%d mismatches)" % (
                sign + lo + int(bad[0]), got[bad[0]], exp[bad[0]], bad.size)


@pytest.mark.parametrize("qtype", QT8)
def test_store_fused_kv_with_token_stride(qtype):
    """K and V in one call, rows embedded in a wider [n, 3*H*D] tensor."""
    rng = np.random.default_rng(77)
    H, D, n_pages, n = 4, 128, 40, 500
    cap = n_pages * W.PAGE
    slots = rng.permutation(cap)[:n].astype(np.int32)
    wide = W.to_bf16_bits(rng.standard_normal((n, 3 * H * D), dtype=np.float32) * 3)
    d_wide = dev_bf16(wide)
    k = kvq()
    kp, ks = k.alloc_pool(qtype, n_pages, H, D)
    vp, vs = k.alloc_pool(qtype, n_pages, H, D)
    for t in (kp, ks, vp, vs):
        t.zero_()
    say("store_fused", qtype)
    k.store(qtype, d_wide[:, H * D:], d_wide[:, 2 * H * D:], dev_i32(slots), kp, ks, vp, vs)
    torch.cuda.synchronize()
    for part, (gp, gs) in ((1, (kp, ks)), (2, (vp, vs))):
        okp, oks = np_pool(qtype, n_pages, H, D)
        src = np.ascontiguousarray(wide[:, part * H * D:(part + 1) * H * D])
        oracle.store(qtype, src, slots, H, D, W.PAGE, n_pages, okp, oks)
        assert np.array_equal(host_u8(gp), okp)
        assert np.array_equal(host_u16(gs), oks)


@pytest.mark.parametrize("qtype", QT8)
def test_store_every_bf16_pair_over_the_scale_range(qtype):
    """Exhaustive over (block max a, element x): every bf16 a whose scale
    a/M spans the fp16 range (and past it, saturating), every bf16 x with
    a * 2^-22 <= |x| <= a of both signs, plus tiny x, against the oracle."""
    rows = []
    for A in range(0x3600, 0x4D80):  # bf16 exponents 2^-20 .. 2^27
        lo = max(1, A - 22 * 128)
        xs = np.arange(lo, A + 1, dtype=np.uint16)
        xs = np.concatenate([xs, xs | 0x8000, np.array([0, 0x8000, 1, 0x8001], np.uint16)])
        pad = (-len(xs)) % 31
        xs = np.concatenate([xs, np.zeros(pad, np.uint16)]).reshape(-1, 31)
        head = np.full((len(xs), 1), A, np.uint16)
        head[1::2] |= 0x8000
        rows.append(np.concatenate([head, xs], axis=1))
    src = np.concatenate(rows)[:, None, :]  # [n, 1 head, 32]
    n = src.shape[0]
    n_pages = (n + W.PAGE - 1) // W.PAGE
    slots = np.arange(n, dtype=np.int32)
    k = kvq()
    kp, ks = k.alloc_pool(qtype, n_pages, 1, 32)
    say("store_exhaustive", qtype, "blocks", n)
    k.store(qtype, dev_bf16(src), None, dev_i32(slots), kp, ks)
    torch.cuda.synchronize()
    okp, oks = np_pool(qtype, n_pages, 1, 32)
    oracle.store(qtype, src, slots, 1, 32, W.PAGE, n_pages, okp, oks)
    got_c = host_u8(kp).reshape(-1, 32)[:n]
    exp_c = okp.reshape(-1, 32)[:n]
    bad = np.nonzero(got_c != exp_c)
    if bad[0].size:
        r, c = bad[0][0], bad[1][0]
        pytest.fail("%d mismatches; first: block max %#06x x %#06x gpu %#04x oracle %#04x" % (
            bad[0].size, src[r, 0, 0], src[r, 0, c], got_c[r, c], exp_c[r, c]))
    assert np.array_equal(host_u16(ks).reshape(-1)[:n], oks.reshape(-1)[:n])


@pytest.mark.parametrize("qtype", ["fp8_e4m3", "q8_0", "bf16"] + CASTS)
def test_dequant_bitexact(qtype):
    rng = np.random.default_rng(88)
    H, D, n_pages = 2, 128, 30
    cap = n_pages * W.PAGE
    src = tricky_rows(rng, cap, H, D)
    slots = np.arange(cap, dtype=np.int32)
    k = kvq()
    kp, ks = k.alloc_pool(qtype, n_pages, H, D)
    say("dequant", qtype)
    k.store(qtype, dev_bf16(src), None, dev_i32(slots), kp, ks)
    q_slots = rng.integers(-3, cap + 3, 400).astype(np.int32)
    out = k.dequant(qtype, kp, ks, dev_i32(q_slots))
    torch.cuda.synchronize()
    okp, oks = np_pool(qtype, n_pages, H, D)
    oracle.store(qtype, src, slots, H, D, W.PAGE, n_pages, okp, oks)
    _, ob = oracle.dequant(qtype, okp, oks, q_slots, H, D, W.PAGE, n_pages)
    assert np.array_equal(host_u16(out), ob)


@pytest.mark.parametrize("qtype", QT8)
def test_store_mixed_workload_full_size(qtype):
    """The timed store of the mixed workload: 8192 new tokens x 8 heads x 128,
    K and V fused, into the 2^20-token pool; every written row bit-exact and
    a sample of untouched rows unchanged."""
    wl = W.mixed()
    H, D = wl.n_kv_heads, wl.head_dim_qk
    slots = wl.new_tokens["slots"]
    kv = wl.new_rows()
    k = kvq()
    kp, ks = k.alloc_pool(qtype, wl.num_pages, H, D)
    vp, vs = k.alloc_pool(qtype, wl.num_pages, H, D)
    for t in (kp, ks, vp, vs):
        t.view(torch.uint8).fill_(0x3C)
    say("store_mixed_full", qtype, "tokens", len(slots))
    k.store(qtype, dev_bf16(kv[0]), dev_bf16(kv[1]), dev_i32(slots), kp, ks, vp, vs)
    torch.cuda.synchronize()
    pages = np.unique(slots // W.PAGE)
    for t, (gp, gs) in enumerate(((kp, ks), (vp, vs))):
        okp, oks = np_pool(qtype, len(pages), H, D, fill_code=0x3C, fill_scale=0x3C3C)
        remap = {int(p): i for i, p in enumerate(pages)}
        local = np.array([remap[int(s) // W.PAGE] * W.PAGE + int(s) % W.PAGE for s in slots],
                         np.int32)
        oracle.store(qtype, kv[t], local, H, D, W.PAGE, len(pages), okp, oks)
        idx = torch.from_numpy(pages.astype(np.int64)).cuda()
        assert np.array_equal(host_u8(gp.index_select(0, idx)), okp)
        assert np.array_equal(host_u16(gs.index_select(0, idx)), oks)
        other = torch.from_numpy(np.setdiff1d(np.arange(0, wl.num_pages, 97), pages)).cuda()
        assert bool((gp.index_select(0, other) == 0x3C).all())


@pytest.mark.parametrize("qtype", CASTS)
def test_cast_store_of_every_bf16_value(qtype):
    """Every finite bf16 pattern (in range, saturating and both zeros), K and
    V in one call, against the oracle's cast: bit-exact codes, no scales
    [PR126 "Add fp8 KV-cache quantization (--kv-dtype)" §How it works]."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = (bits.astype(np.uint32) << 16).view(np.float32)
    bits = bits[np.isfinite(f)]
    bits = np.concatenate([bits, np.zeros((-len(bits)) % 32, np.uint16)])
    src = bits.reshape(-1, 1, 32)
    srcv = np.ascontiguousarray(src[::-1])
    n = src.shape[0]
    n_pages = (n + W.PAGE - 1) // W.PAGE
    slots = np.arange(n, dtype=np.int32)
    k = kvq()
    kp, ks = k.alloc_pool(qtype, n_pages, 1, 32)
    vp, vs = k.alloc_pool(qtype, n_pages, 1, 32)
    assert ks is None and vs is None
    say("cast_store_exhaustive", qtype, "rows", n)
    k.store(qtype, dev_bf16(src), dev_bf16(srcv), dev_i32(slots), kp, None, vp, None)
    torch.cuda.synchronize()
    for gp, s in ((kp, src), (vp, srcv)):
        okp, _ = np_pool(qtype, n_pages, 1, 32)
        oracle.store(qtype, s, slots, 1, 32, W.PAGE, n_pages, okp, None)
        got = host_u8(gp).reshape(-1, 32)[:n]
        exp = okp.reshape(-1, 32)[:n]
        bad = np.nonzero(got != exp)
        if bad[0].size:
            r, c = bad[0][0], bad[1][0]
            pytest.fail("%d mismatches; first: x %#06x gpu %#04x oracle %#04x" % (
                bad[0].size, s[r, 0, c], got[r, c], exp[r, c]))


@pytest.mark.parametrize("qtype", CASTS)
def test_cast_dequant_of_every_code(qtype):
    """All 256 codes in a pool (NaN codes of the format excluded) read back
    through kvq_dequant as the oracle's exact values in bf16."""
    codes = np.arange(256, dtype=np.uint8)
    vals = np.array([oracle.e5m2_value(int(c)) if qtype == "fp8_e5m2_cast" else
                     oracle.e4m3_value(int(c)) for c in codes])
    codes = codes[np.isfinite(vals)]
    codes = np.concatenate([codes, np.zeros((-len(codes)) % 32, np.uint8)])
    n = len(codes) // 32
    pool = np.zeros(((n + W.PAGE - 1) // W.PAGE, 1, W.PAGE, 32), np.uint8)
    pool.reshape(-1, 32)[:n] = codes.reshape(n, 32)
    n_pages = pool.shape[0]
    slots = np.arange(n, dtype=np.int32)
    k = kvq()
    say("cast_dequant_codes", qtype)
    out = k.dequant(qtype, torch.from_numpy(pool).cuda(), None, dev_i32(slots))
    torch.cuda.synchronize()
    _, ob = oracle.dequant(qtype, pool, None, slots, 1, 32, W.PAGE, n_pages)
    assert np.array_equal(host_u16(out), ob)
