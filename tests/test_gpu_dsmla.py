"""GPU parity of the 656-byte MLA row (fp8_ds_mla) store and dequant against
the oracle: bytes identical (codes, fp32 tile scales, bf16 rope) for rows of
the mla recipe, for zero tiles, signed zeros, outliers and tiny tiles, with a
token stride and invalid slots; dequantized rows identical bf16 bits (the
product of code and fp32 scale rounded once).  The decode over this row is
covered with the other storage types in test_gpu_mla and test_gpu_sparse.

Page key: [PR25] "Experimental FP8 KV Cache" (a 656-byte fp8 row for the
576-wide latent, laid out as in vLLM).
"""
import numpy as np
import pytest
import torch

import oracle
from paged_decode_attention_amd import workloads as W
from tests.gpu_util import dev_bf16, dev_i32, host_u16, kvq, requires_gpu, say

pytestmark = [pytest.mark.gpu, requires_gpu]

D = 576


def rows(seed, n):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, D), dtype=np.float32)
    x[0, 128:256] = 0.0                      # a zero tile
    x[1, :128] = -0.0                        # a tile of negative zeros
    x[2, 300] = 3e4                          # an outlier
    x[3, 384:512] *= 1e-30                   # a tile of tiny values
    x[4] = np.where(rng.random(D) < 0.5, -x[4], x[4]) * 200.0
    return W.to_bf16_bits(x)


@pytest.mark.parametrize("stride", [D, D + 64])
def test_store_bytes_match_the_oracle(stride):
    k = kvq()
    n_pages, n = 12, 150
    src = rows(1, n)
    buf = np.zeros((n, stride), np.uint16)
    buf[:, :D] = src
    slots = np.random.default_rng(2).permutation(n_pages * 16)[:n].astype(np.int32)
    slots[7] = -1                            # skipped
    slots[9] = n_pages * 16                  # past the pool: skipped
    pool, sc = k.alloc_pool("fp8_ds_mla", n_pages, 1, D)
    assert sc is None and pool.shape[-1] == oracle.DS_ROW
    pool.zero_()
    say("dsm store stride", stride)
    k.store("fp8_ds_mla", dev_bf16(buf), None, dev_i32(slots), pool, None)
    torch.cuda.synchronize()
    want = np.zeros((n_pages, 1, 16, oracle.DS_ROW), np.uint8)
    oracle.store("fp8_ds_mla", buf, slots, 1, D, 16, n_pages, want, None, token_stride=stride)
    got = pool.cpu().numpy()
    assert np.array_equal(got, want)


def test_dequant_bits_match_the_oracle():
    k = kvq()
    n_pages, n = 8, 128
    src = rows(3, n)
    slots = np.arange(n, dtype=np.int32)
    pool, _ = k.alloc_pool("fp8_ds_mla", n_pages, 1, D)
    k.store("fp8_ds_mla", dev_bf16(src), None, dev_i32(slots), pool, None)
    q = np.concatenate([slots, [-1, n_pages * 16 + 5]]).astype(np.int32)
    out = k.dequant("fp8_ds_mla", pool, None, dev_i32(q))
    torch.cuda.synchronize()
    host = pool.cpu().numpy()
    _, want = oracle.dequant("fp8_ds_mla", host, None, q, 1, D, 16, n_pages)
    assert np.array_equal(host_u16(out), want)
