"""Host-side checks of the C ABI (CPU only, no kernel launches): the library
loads and exports every symbol the header declares, the cost model, and the
argument validation that runs before anything is enqueued.

Page keys: [PR103] "feat(kvcache): 8-bit KV cache (q8_0 / fp8_e4m3) behind
--kv-cache-dtype" (§What: effective bytes per element; review §"End-to-end
numbers": the pool grows by 2/1.0625); [PR113] "feat(kvcache): 8-bit DSV4
window/compressed KV behind --kv-cache-dtype" (§Gating: head_dim a multiple of
32, rejected up front with a clear message; §One ordering trap: the cost model
and the pool must agree).
"""
import ctypes
import os
import re
from fractions import Fraction

import pytest

from paged_decode_attention_amd import kvq
from tests.test_oracle_pins import FACTS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions(name="kvq.h"):
    src = open(os.path.join(ROOT, "include", name)).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    headers = sorted(f for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h"))
    assert "kvq.h" in headers and "kvq_debug.h" in headers
    names = header_functions("kvq.h")
    assert set(names) == set(kvq.EXPORTS)
    assert set(header_functions("kvq_debug.h")) == set(kvq.DEBUG_EXPORTS)
    for h in headers:
        for n in header_functions(h):
            assert ctypes.cast(getattr(kvq.LIB, n), ctypes.c_void_p).value, n


def test_pool_bytes_is_17_16_per_element_and_32_17_vs_bf16():
    for pages, H, D in [(1, 1, 32), (8192, 8, 128), (10240, 1, 576), (3, 2, 256)]:
        t8, c8, s8 = kvq.pool_bytes("fp8_e4m3", pages, 16, H, D)
        tq, cq, sq = kvq.pool_bytes("q8_0", pages, 16, H, D)
        tb, cb, sb = kvq.pool_bytes("bf16", pages, 16, H, D)
        elems = pages * 16 * H * D
        assert (t8, c8, s8) == (tq, cq, sq)
        assert Fraction(t8, elems) == Fraction(int(FACTS["bytes_per_elem_num"]),
                                               int(FACTS["bytes_per_elem_den"]))
        assert sb == 0 and Fraction(tb, t8) == Fraction(32, 17)
    # same byte budget: the measured pool growth on the page (+88%)
    budget = int(FACTS["pool_tokens_bf16"]) * kvq.pool_bytes("bf16", 1, 1, 1, 256)[0]
    per_tok = kvq.pool_bytes("fp8_e4m3", 1, 1, 1, 256)[0]
    assert abs(budget // per_tok - FACTS["pool_tokens_8bit"]) < 16


@pytest.mark.parametrize("dtype", ["fp8_e4m3", "q8_0", "fp8_e4m3_cast", "fp8_e5m2_cast"])
def test_head_dim_not_multiple_of_32_is_rejected_up_front(dtype):
    with pytest.raises(ValueError, match="multiple of"):
        kvq.pool_bytes(dtype, 4, 16, 1, 48)
    rc = kvq.LIB.kvq_store(kvq.DTYPES[dtype], 16, 16, 48, 16, 1, 1, 48, 16, 4, 16, 16, 16, 16,
                           None)
    assert rc == kvq.ERR_ARG and "multiple of the 32-element" in kvq.last_error()
    assert kvq.LIB.kvq_paged_decode_workspace_bytes(1, 2, 1, 48, 4, 16) == 0


def test_validation_errors_before_any_launch():
    L = kvq.LIB
    # null pointers, bad strides, bad dtype: rejected with messages, nothing launched
    assert L.kvq_store(1, None, None, 128, None, 4, 1, 128, 16, 4, None, None, None, None,
                       None) == kvq.ERR_ARG
    assert "null" in kvq.last_error()
    assert L.kvq_store(1, 16, None, 100, 16, 4, 1, 128, 16, 4, 16, 16, None, None,
                       None) == kvq.ERR_ARG
    assert "src_token_stride" in kvq.last_error()
    assert L.kvq_store(7, 16, None, 128, 16, 4, 1, 128, 16, 4, 16, 16, None, None,
                       None) == kvq.ERR_ARG
    assert L.kvq_store(1, 8, None, 128, 16, 4, 1, 128, 16, 4, 16, 16, None, None,
                       None) == kvq.ERR_ARG
    assert "aligned" in kvq.last_error()
    # zero tokens is a no-op success
    assert L.kvq_store(1, None, None, 128, None, 0, 1, 128, 16, 4, None, None, None, None,
                       None) == kvq.OK
    assert kvq.last_error() == ""


def test_decode_validation():
    L = kvq.LIB
    args = dict(q=256, kp=256, ks=256, vp=512, vs=512, pt=256, sl=256, sl_host=None, out=256,
                lse=None, wsp=256)

    def call(dtype=1, B=2, Hq=16, Hkv=8, D=128, Dv=128, ps=16, mp=8, pts=8, npg=64, ws=1 << 30,
             sm=0.1, **kw):
        a = dict(args, **kw)
        return L.kvq_paged_decode(dtype, a["q"], a["kp"], a["ks"], a["vp"], a["vs"], a["pt"], pts,
                                  a["sl"], a["sl_host"], B, Hq, Hkv, D, Dv, ps, mp, npg, sm,
                                  a["out"], a["lse"], a["wsp"], ws, None)

    assert call(Hq=12, Hkv=8) == kvq.ERR_ARG                 # not a multiple
    assert call(ps=32) == kvq.ERR_UNSUPPORTED and "page_size" in kvq.last_error()
    assert call(D=96, Dv=96) == kvq.ERR_UNSUPPORTED
    assert call(Dv=256) == kvq.ERR_ARG                       # Dv > Dqk
    assert call(pts=4) == kvq.ERR_ARG                        # stride < max_pages
    assert call(ws=16) == kvq.ERR_WORKSPACE
    assert call(wsp=None) == kvq.ERR_WORKSPACE
    assert call(kp=None) == kvq.ERR_ARG
    assert call(sm=float("nan")) == kvq.ERR_ARG
    assert call(B=0) == kvq.ERR_ARG
    assert call(B=5000) == kvq.ERR_UNSUPPORTED
    # k_pool == v_pool is the shared-slab form, only for 576/512
    assert call(vp=256, vs=256) == kvq.ERR_UNSUPPORTED
    need = kvq.workspace_bytes(2, 16, 8, 128, 8, 16)
    assert call(ws=need - 1) == kvq.ERR_WORKSPACE
    # the 656-byte row is the slab's format only
    assert call(dtype=5) == kvq.ERR_UNSUPPORTED and "656-byte" in kvq.last_error()


def test_append_validation():
    """kvq_paged_decode_append checks the new rows before anything is
    enqueued (every call here is refused on the host)."""
    L = kvq.LIB

    def call(nk=256, nv=512, stride=8 * 128, kp=256, vp=512, D=128, Dv=128, Hkv=8, ws=1 << 30,
             wsp=256):
        vs = 256 if vp == kp else 512
        return L.kvq_paged_decode_append(1, 256, nk, nv, stride, kp, 256, vp, vs, 256, 8, 256,
                                         None, 2, 16, Hkv, D, Dv, 16, 8, 64, 0.1, 256, None, wsp,
                                         ws, None)

    assert call(nk=None) == kvq.ERR_ARG and "new_k" in kvq.last_error()
    assert call(nv=None) == kvq.ERR_ARG and "new_v" in kvq.last_error()   # separate pools
    assert call(stride=100) == kvq.ERR_ARG and "stride" in kvq.last_error()
    assert call(stride=8 * 128 - 8) == kvq.ERR_ARG
    assert call(nk=264) == kvq.ERR_ARG and "aligned" in kvq.last_error()
    # the shared slab takes no new_v
    assert call(kp=256, vp=256, D=576, Dv=512, Hkv=1, stride=576) == kvq.ERR_ARG
    assert "new_v" in kvq.last_error()
    # the decode's own checks still apply (and come first)
    assert call(D=96, Dv=96) == kvq.ERR_UNSUPPORTED
    assert call(ws=16, nk=None) == kvq.ERR_ARG
    assert call(ws=16) == kvq.ERR_WORKSPACE


def test_workspace_query_covers_every_storage_type():
    """kvq_paged_decode_workspace_bytes takes no storage type: its answer is
    the largest workspace any type's plan needs for the shapes (the plans
    read through the library's test export)."""
    for B, Hq, Hkv, Dv, mp in [(8, 16, 8, 128, 1024), (3, 16, 2, 256, 2048), (64, 16, 8, 128, 8192),
                               (1, 128, 1, 512, 10240), (2, 32, 1, 64, 3), (5, 8, 8, 32, 100)]:
        need = kvq.workspace_bytes(B, Hq, Hkv, Dv, mp, 16)
        assert need > 0 and need % 256 == 0
        Dqk = 576 if (Hkv == 1 and Dv == 512) else Dv
        plans = [kvq.debug_plan(dt, B, Hq, Hkv, Dqk, Dv, mp) for dt in kvq.DTYPES]
        sizes = [p["bytes"] for p in plans if p is not None]
        assert sizes and need == max(sizes)


def test_python_errors_are_typed():
    with pytest.raises(ValueError):
        kvq.pool_bytes("fp8_e4m3", -1, 16, 1, 32)
    with pytest.raises(ValueError):
        kvq.pool_bytes("int4", 1, 16, 1, 32)
    with pytest.raises(NotImplementedError):
        kvq.workspace_bytes(1, 8, 1, 64, 4, 8)


def test_only_block_scaled_types_carry_scales():
    """Scale bytes: 2 per 32 elements for the block-scaled types, none for
    bf16 and the cast types [PR126 "Add fp8 KV-cache quantization
    (--kv-dtype)" §How it works: scale 1.0]; a block-scaled store without a
    scale buffer is rejected before any launch."""
    for dtype, code_b, scale_b in (("fp8_e4m3", 1, 2 / 32), ("q8_0", 1, 2 / 32), ("bf16", 2, 0),
                                   ("fp8_e4m3_cast", 1, 0), ("fp8_e5m2_cast", 1, 0)):
        total, codes, scales = kvq.pool_bytes(dtype, 10, 16, 4, 128)
        n = 10 * 16 * 4 * 128
        assert codes == code_b * n and scales == scale_b * n and total == codes + scales
    for dtype in ("fp8_e4m3", "q8_0"):
        rc = kvq.LIB.kvq_store(kvq.DTYPES[dtype], 16, None, 128, 16, 4, 1, 128, 16, 4, 16, None,
                               None, None, None)
        assert rc == kvq.ERR_ARG and "k_scales" in kvq.last_error()


def test_extend_validation():
    """kvq_extend_attention rejects bad shapes and arguments before any launch."""
    L = kvq.LIB
    args = dict(q=256, qs=256, kp=256, ks=256, vp=512, vs=512, pt=256, sl=256, out=256, lse=None,
                wsp=256)

    def call(dtype=1, mn=64, B=2, Hq=16, Hkv=8, D=128, ps=16, mp=8, pts=8, npg=64, ws=1 << 30,
             sm=0.1, **kw):
        a = dict(args, **kw)
        return L.kvq_extend_attention(dtype, a["q"], a["qs"], mn, a["kp"], a["ks"], a["vp"],
                                      a["vs"], a["pt"], pts, a["sl"], B, Hq, Hkv, D, ps, mp, npg,
                                      sm, a["out"], a["lse"], a["wsp"], ws, None)

    assert call(mn=0) == kvq.ERR_ARG
    assert call(mn=70000) == kvq.ERR_UNSUPPORTED and "max_new_tokens" in kvq.last_error()
    assert call(qs=None) == kvq.ERR_ARG
    assert call(Hq=12) == kvq.ERR_ARG
    assert call(D=96) == kvq.ERR_UNSUPPORTED                  # only 64, 128, 256
    assert call(D=48, dtype=0) == kvq.ERR_UNSUPPORTED
    assert call(vp=256, vs=256) == kvq.ERR_UNSUPPORTED        # shared slab: decode only
    assert call(ps=32) == kvq.ERR_UNSUPPORTED
    assert call(pts=4) == kvq.ERR_ARG
    assert call(sm=float("inf")) == kvq.ERR_ARG
    need = kvq.extend_workspace_bytes("fp8_e4m3", 2, 16, 8, 128, 16, 8, 64)
    assert need > kvq.workspace_bytes(2, 16, 8, 128, 8, 16)  # 8 tiles per kv head
    assert call(ws=need - 1) == kvq.ERR_WORKSPACE
    # the shared 576/512 slab: work numbered by new token, at most 1024 of them
    assert L.kvq_extend_attention_workspace_bytes(1, 1, 128, 1, 576, 16, 8, 4) > 0
    assert L.kvq_extend_attention_workspace_bytes(1, 8, 128, 1, 576, 16, 8, 200) == 0
    assert call(Hq=128, Hkv=1, D=576, vp=256, vs=256, mn=200, B=8) == kvq.ERR_UNSUPPORTED
    assert call(Hq=128, Hkv=1, D=576) == kvq.ERR_UNSUPPORTED  # separate pools at 576


def test_656_byte_row_shape_and_validation():
    """fp8_ds_mla: 656 bytes per token row, one head of 576 elements, no scale
    buffer; other shapes, a separate V source and the separate-K/V kernels
    are rejected before any launch."""
    L = kvq.LIB
    total, codes, scales = kvq.pool_bytes("fp8_ds_mla", 10, 16, 1, 576)
    assert total == codes == 10 * 16 * 656 and scales == 0
    assert L.kvq_pool_bytes(5, 10, 16, 1, 512, None) == -1
    assert L.kvq_pool_bytes(5, 10, 16, 2, 576, None) == -1
    # store: wrong shape, and a V source (the row is K and V at once)
    assert L.kvq_store(5, 16, None, 576, 16, 4, 1, 512, 16, 4, 16, None, None, None, None) == kvq.ERR_UNSUPPORTED
    assert L.kvq_store(5, 16, 16, 576, 16, 4, 1, 576, 16, 4, 16, None, 16, None, None) == kvq.ERR_ARG
    # decode: the slab shape only
    assert kvq.workspace_bytes(1, 128, 1, 512, 64, 16) > 0
    assert L.kvq_paged_decode(5, 256, 256, None, 512, None, 256, 8, 256, None, 2, 16, 8, 128, 128,
                              16, 8, 64, 0.1, 256, None, 256, 1 << 30, None) == kvq.ERR_UNSUPPORTED
    assert "656-byte" in kvq.last_error()
    assert L.kvq_extend_attention_workspace_bytes(5, 2, 16, 8, 128, 16, 8, 4) == 0
    assert kvq.sparse_workspace_bytes("fp8_ds_mla", 1, 128, 256) > 0


def test_in_kernel_merge_weights_fit_in_lds():
    """The last workgroup of a split sequence merges its chunks with one LDS
    weight per (chunk, query column), 4096 at most.  A sequence splits into at
    most ceil(max_pages / item pages) chunks, and the kernels never size items
    below the plan's fewest pages (their rule clamps to it), so the plan must
    keep ceil(max_pages / min_pages) x columns within 4096 whenever the merge
    runs inside the decode kernel: every G, new-token count, head_dim and
    table width."""
    checked = 0
    for D in (32, 64, 128, 256):
        for G in (1, 2, 3, 4, 5, 6, 8, 12, 16, 32):
            for ext in (0, 1, 2, 3, 5, 7, 11, 64):
                if ext and D == 32:
                    continue
                for mp in (1, 7, 100, 1000, 1365, 2048, 4095, 16384, 32768):
                    for dt in ("fp8_e4m3", "bf16"):
                        p = kvq.debug_plan(dt, 2, 2 * G, 2, D, D, mp, ext)
                        if p is None or not p["fused_merge"]:
                            continue
                        checked += 1
                        chunks = -(-mp // p["min_pages"])
                        assert chunks * p["gt"] * p["tn"] <= 4096, (D, G, ext, mp, dt, p)
                        assert p["min_pages"] % p["step"] == 0
                        assert p["min_pages"] <= p["cap_pages"]
    assert checked > 1000



def test_extend_long_prefill_plans_whole_sequences():
    """Extend attention with many query-row tiles (long prefill): once the
    (sequence, kv head, tile group) units reach four per resident workgroup
    (2048) and the split plan's partials would pass 1 GiB, each unit is one
    work item over its whole sequence, so nothing is split and the workspace
    holds no partials; otherwise sequences split (faster where both fit) and
    the workspace holds a partial row per item and column."""
    # 8 sequences x 8 kv heads x ceil(new x 2 / 32) tile groups (head_dim 128, G = 2)
    for new, whole in ((64, False), (512, False), (2048, False), (4096, True)):
        p = kvq.debug_plan("fp8_e4m3", 8, 16, 8, 128, 128, 1024, new)
        units = 8 * 8 * -(-new * 2 // 32)
        assert units >= 2048 or not p["whole"]
        assert bool(p["whole"]) == whole, (new, p)
        ws = kvq.extend_workspace_bytes("fp8_e4m3", 8, 16, 8, 128, 16, 1024, new)
        assert ws == p["bytes"]
        if whole:
            assert p["max_items"] == units and p["min_pages"] >= 1024
            assert ws < 128 * 1024, ws
        else:
            assert ws > 1 << 20, ws
    # the decode never plans whole sequences
    assert not kvq.debug_plan("fp8_e4m3", 64, 16, 2, 256, 256, 4096)["whole"]
