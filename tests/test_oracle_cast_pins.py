"""Pins for the oracle's cast storage types: each element stored as an 8-bit
float itself (a per-tensor scale of 1.0, no scale buffer), e4m3fn or e5m2.

References, none of which re-types the oracle's formulas: the IEEE binary16
layout (an e5m2 code is the high byte of a binary16 with the same sign,
exponent and bias), torch's float8_e4m3fn / float8_e5m2 casts (round to
nearest even inside the format's range), exact rational midpoints, and the
token budgets the page prints (tests/golden).

Page key: [PR126] "Add fp8 KV-cache quantization (--kv-dtype)": §Summary
(fp8_e4m3 or fp8_e5m2), §How it works (the store casts with scale 1.0),
§Benchmark (the same bytes hold 2.00x the bf16 tokens).
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests.test_oracle_pins import FACTS, e4m3_lib_value

CASTS = {"fp8_e4m3_cast": (torch.float8_e4m3fn, 448.0), "fp8_e5m2_cast": (torch.float8_e5m2, 57344.0)}


def all_finite_bf16():
    """Every finite bf16 value as fp32 (both zeros included)."""
    bits = np.arange(1 << 16, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    return f[np.isfinite(f)]


def torch_cast(v: np.ndarray, tdtype) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(tdtype)
    return t.view(torch.uint8).numpy()


def code_values(qtype) -> np.ndarray:
    codes = np.arange(256, dtype=np.uint8)
    if qtype == "fp8_e5m2_cast":
        return np.array([oracle.e5m2_value(int(c)) for c in codes])
    return np.array([oracle.e4m3_value(int(c)) for c in codes])


def test_e5m2_decode_is_the_high_byte_of_binary16():
    """e5m2 shares binary16's sign, 5-bit exponent and bias 15: code c is the
    binary16 whose bits are c << 8 (infinities and NaNs included)."""
    codes = np.arange(256, dtype=np.uint16)
    ref = (codes << 8).astype(np.uint16).view(np.float16).astype(np.float64)
    got = np.array([oracle.e5m2_value(int(c)) for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    assert got[0x7B] == 57344.0 and got[0x7C] == np.inf and got[0x01] == 2.0 ** -16


def test_e5m2_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e5m2).to(torch.float64).numpy()
    got = np.array([oracle.e5m2_value(int(c)) for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


@pytest.mark.parametrize("qtype", sorted(CASTS))
def test_cast_of_every_in_range_bf16_matches_torch(qtype):
    """Every finite bf16 with |x| <= the format maximum: torch's cast."""
    tdtype, M = CASTS[qtype]
    v = all_finite_bf16()
    v = v[np.abs(v) <= M]
    assert np.array_equal(oracle.cast_encode(qtype, v), torch_cast(v, tdtype))


@pytest.mark.parametrize("qtype", sorted(CASTS))
def test_cast_saturates_beyond_the_format(qtype):
    """Beyond the largest finite magnitude (bf16 infinities included) the
    cast stores that magnitude with the element's sign."""
    _, M = CASTS[qtype]
    v = all_finite_bf16()
    v = np.concatenate([v[np.abs(v) > M], np.array([np.inf, -np.inf], np.float32)])
    vals = code_values(qtype)
    max_code = int(np.nonzero(vals == M)[0][0])
    got = oracle.cast_encode(qtype, v)
    want = np.where(v > 0, max_code, max_code | 0x80)
    assert np.array_equal(got, want.astype(np.uint8))


@pytest.mark.parametrize("qtype", sorted(CASTS))
def test_on_grid_values_round_trip_and_midpoints_tie_to_even(qtype):
    """Each finite code's value encodes to that code; the exact midpoint
    between two neighbouring positive codes goes to the even one, one fp32
    step to either side to the nearer one; negatives mirror with the sign."""
    vals = code_values(qtype)
    _, M = CASTS[qtype]
    pos = [c for c in range(0x80) if np.isfinite(vals[c]) and vals[c] <= M]
    got = oracle.cast_encode(qtype, vals[pos].astype(np.float32))
    assert list(got) == pos
    neg = oracle.cast_encode(qtype, (-vals[pos]).astype(np.float32))
    assert list(neg) == [0x80 | c for c in pos]
    for c in pos[:-1]:
        lo, hi = Fraction(float(vals[c])), Fraction(float(vals[c + 1]))
        mid = (lo + hi) / 2
        m32 = np.float32(float(mid))
        assert Fraction(float(m32)) == mid  # midpoints are exact in fp32
        even = c if c % 2 == 0 else c + 1
        trio = np.array([m32, np.nextafter(m32, np.float32(0)), np.nextafter(m32, np.float32(1e9))],
                        np.float32)
        assert list(oracle.cast_encode(qtype, trio)) == [even, c, c + 1]


def test_e4m3_cast_agrees_with_the_format_the_scaled_store_uses():
    """The e4m3 cast and the block-scaled store share the e4m3fn grid: the
    cast's code values are torch's float8_e4m3fn values."""
    codes = np.arange(256, dtype=np.uint8)
    ref = e4m3_lib_value(codes)
    got = code_values("fp8_e4m3_cast")
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])


def test_cast_pools_hold_twice_the_bf16_tokens():
    """One byte per element and no scale buffer: the same bytes hold 2.00x
    the bf16 tokens -- the page's 27,142 -> 54,284 [PR126 §Benchmark]."""
    from paged_decode_attention_amd import kvq
    for qtype in CASTS:
        total, codes, scales = kvq.pool_bytes(qtype, 1000, 16, 8, 128)
        bf, _, _ = kvq.pool_bytes("bf16", 1000, 16, 8, 128)
        assert scales == 0 and total == codes == 1000 * 16 * 8 * 128
        assert Fraction(bf, total) == 2
    assert FACTS["per_tensor_tokens_fp8"] == 2 * FACTS["per_tensor_tokens_bf16"]
