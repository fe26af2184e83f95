"""kvq_paged_decode_noalloc: the decode with the library's own scratch array
as its workspace (for callers that cannot allocate), against
kvq_paged_decode with a caller-owned workspace on the same inputs.

Two calls in a row on one GPU share the array; the second is smaller and
has another shape, so its arrival counters sit where the first call left
partial results.  Both must give kvq_paged_decode's bits.  A plan larger
than the array is refused before anything is launched.  The module's name
makes pytest collect it last.
"""
import ctypes

import numpy as np
import pytest
import torch

from paged_decode_attention_amd import workloads as W
from tests.gpu_util import dev_bf16, dev_i32, fill_both, kvq, requires_gpu, say
from tests.test_gpu_decode import small_workload

pytestmark = [pytest.mark.gpu, requires_gpu]

SCRATCH = 64 << 20  # the array's size


def _noalloc(qtype, q, pools, wl, head_dim_v, shared):
    k = kvq()
    B, Hq, Dqk = q.shape
    out = torch.empty((B, Hq, head_dim_v), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    pt, sl = dev_i32(wl.page_table), dev_i32(wl.seq_lens)
    vp, vs = (pools["kp"], pools["ks"]) if shared else (pools["vp"], pools["vs"])
    rc = k.LIB.kvq_paged_decode_noalloc(
        k.DTYPES[qtype], q.data_ptr(), pools["kp"].data_ptr(),
        pools["ks"].data_ptr() if pools["ks"] is not None else None, vp.data_ptr(),
        vs.data_ptr() if vs is not None else None, pt.data_ptr(), wl.max_pages, sl.data_ptr(),
        None, B, Hq, wl.n_kv_heads, Dqk, head_dim_v, W.PAGE, wl.max_pages, wl.num_pages,
        wl.sm_scale, out.data_ptr(), lse.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == k.OK, k.last_error()
    return out, lse


def _reference(qtype, q, pools, wl, head_dim_v, shared):
    k = kvq()
    vp, vs = (pools["kp"], pools["ks"]) if shared else (pools["vp"], pools["vs"])
    return k.paged_decode(qtype, q, pools["kp"], pools["ks"], vp, vs, dev_i32(wl.page_table),
                          dev_i32(wl.seq_lens), wl.sm_scale, head_dim_v=head_dim_v)


def test_noalloc_matches_the_workspace_entry_point_twice():
    from tests.test_gpu_mla import mla_workload
    cases = [
        # a batch whose long sequences split into many items (partials in the array)
        (small_workload(128, 16, 8, [20000, 9000, 17, 0, 3001], 1300, seed=41), "fp8_e4m3", 128,
         False),
        # then a smaller call of another shape: head_dim 64, 4 q heads per kv head
        (small_workload(64, 8, 2, [700, 33], 50, seed=42), "q8_0", 64, False),
    ]
    for wl, qtype, dv, shared in cases:
        pools = fill_both(wl, qtype)
        q = dev_bf16(wl.query())
        say("noalloc", wl.name, qtype)
        o1, l1 = _noalloc(qtype, q, pools, wl, dv, shared)
        o2, l2 = _reference(qtype, q, pools, wl, dv, shared)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # and the 576/512 slab (its own kernel and merge) after the two
    wl = mla_workload(64, [3000, 40], 200, seed=43)
    pools = fill_both(wl, "fp8_e4m3")
    q = dev_bf16(wl.query())
    say("noalloc slab")
    o1, l1 = _noalloc("fp8_e4m3", q, pools, wl, 512, True)
    o2, l2 = _reference("fp8_e4m3", q, pools, wl, 512, True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_noalloc_refuses_plans_beyond_the_array():
    k = kvq()
    # 16 sequences over the 576/512 slab, 10240 pages each: bf16 partial rows
    # of 128 heads for every item, far beyond 64 MiB
    plan = k.debug_plan("fp8_e4m3", 16, 128, 1, 576, 512, 10240)
    assert plan is not None and plan["bytes"] > SCRATCH
    # the call is refused on the host, before any launch (the pointers are
    # never dereferenced)
    rc = k.LIB.kvq_paged_decode_noalloc(k.DTYPES["fp8_e4m3"], 256, 256, 256, 256, 256, 256, 10240,
                                        256, None, 16, 128, 1, 576, 512, 16, 10240, 1 << 20, 0.1,
                                        256, None, None)
    assert rc == k.ERR_WORKSPACE and "scratch" in k.last_error()
