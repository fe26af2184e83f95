"""Python binding of libkvq.so (the HIP library for gfx950).

Argument marshalling only: every step of the store, dequant and decode runs in
the library's HIP kernels.  PyTorch supplies device memory and the current
stream.  Importing this module loads ``libkvq.so`` and fails loudly if it has
not been built (``python -m paged_decode_attention_amd.build``); there is no
fallback path.

Tensor conventions (device tensors unless noted):
  pool    uint8 [num_pages, n_heads, page_size, head_dim] (8-bit codes) or
          bfloat16 of the same shape for dtype "bf16"
  scales  any 2-byte dtype [num_pages, n_heads, page_size, head_dim // 32]
          holding IEEE fp16 bit patterns (None for "bf16" and the cast types
          "fp8_e4m3_cast" / "fp8_e5m2_cast", which store each element itself)
  q       bfloat16 [batch, n_q_heads, head_dim_qk]
  page_table int32 [batch, max_pages] (-1 = masked), seq_lens int32 [batch]
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# KVQ_LIB may name another build of the same sources (A/B timing of variants)
LIB_PATH = os.environ.get("KVQ_LIB") or os.path.join(HERE, "libkvq.so")

DTYPES = {"bf16": 0, "fp8_e4m3": 1, "q8_0": 2, "fp8_e4m3_cast": 3, "fp8_e5m2_cast": 4, "fp8_ds_mla": 5}
SCALED = ("fp8_e4m3", "q8_0")  # storage types with a scale buffer
OK, ERR_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, -1, -2, -3, -4


class KvqError(RuntimeError):
    """A non-OK status from libkvq.so; ``status`` holds the code."""

    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError("libkvq.so is not built at %s; run "
                          "`python -m paged_decode_attention_amd.build`" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    c = ctypes
    P, I, I64 = c.c_void_p, c.c_int, c.c_int64
    lib.kvq_pool_bytes.argtypes = [I, I64, I, I, I, c.POINTER(I64)]
    lib.kvq_pool_bytes.restype = I64
    lib.kvq_store.argtypes = [I, P, P, I64, P, I64, I, I, I, I64, P, P, P, P, P]
    lib.kvq_store.restype = I
    lib.kvq_dequant.argtypes = [I, P, P, P, I64, I, I, I, I64, P, P]
    lib.kvq_dequant.restype = I
    lib.kvq_paged_decode_workspace_bytes.argtypes = [I, I, I, I, I, I]
    lib.kvq_paged_decode_workspace_bytes.restype = c.c_size_t
    lib.kvq_paged_decode.argtypes = [I, P, P, P, P, P, P, I64, P, P, I, I, I, I, I, I, I, I64,
                                     c.c_float, P, P, P, c.c_size_t, P]
    lib.kvq_paged_decode.restype = I
    lib.kvq_paged_decode_append.argtypes = [I, P, P, P, I64, P, P, P, P, P, I64, P, P, I, I, I, I,
                                            I, I, I, I64, c.c_float, P, P, P, c.c_size_t, P]
    lib.kvq_paged_decode_append.restype = I
    lib.kvq_sparse_mla_decode_workspace_bytes.argtypes = [I, I, I, I]
    lib.kvq_sparse_mla_decode_workspace_bytes.restype = c.c_size_t
    lib.kvq_sparse_mla_decode.argtypes = [I, P, P, P, P, I64, P, P, I64, I, I, I, I, I, I64,
                                          c.c_float, P, P, P, c.c_size_t, P]
    lib.kvq_sparse_mla_decode.restype = I
    lib.kvq_extend_attention_workspace_bytes.argtypes = [I, I, I, I, I, I, I, I]
    lib.kvq_extend_attention_workspace_bytes.restype = c.c_size_t
    lib.kvq_extend_attention.argtypes = [I, P, P, I, P, P, P, P, P, I64, P, I, I, I, I, I, I, I64,
                                         c.c_float, P, P, P, c.c_size_t, P]
    lib.kvq_extend_attention.restype = I
    lib.kvq_paged_decode_noalloc.argtypes = [I, P, P, P, P, P, P, I64, P, P, I, I, I, I, I, I, I,
                                             I64, c.c_float, P, P, P]
    lib.kvq_paged_decode_noalloc.restype = I
    lib.kvq_debug_e4m3_encode_range.argtypes = [c.c_uint32, I64, P, P]
    lib.kvq_debug_e4m3_encode_range.restype = I
    lib.kvq_debug_decode_plan.argtypes = [I, I, I, I, I, I, I, I, c.POINTER(I64), I]
    lib.kvq_debug_decode_plan.restype = I
    lib.kvq_last_error.argtypes = []
    lib.kvq_last_error.restype = c.c_char_p
    return lib


LIB = _load()

# every symbol the public header declares
EXPORTS = ("kvq_pool_bytes", "kvq_store", "kvq_dequant", "kvq_paged_decode_workspace_bytes",
           "kvq_paged_decode", "kvq_paged_decode_append", "kvq_paged_decode_noalloc", "kvq_sparse_mla_decode_workspace_bytes",
           "kvq_sparse_mla_decode", "kvq_extend_attention_workspace_bytes", "kvq_extend_attention",
           "kvq_last_error")
# the test exports (kvq_debug.h)
DEBUG_EXPORTS = ("kvq_debug_e4m3_encode_range", "kvq_debug_decode_plan")
PLAN_FIELDS = ("kind", "gt", "tn", "n_hg", "step", "min_pages", "cap_pages", "target",
               "max_items", "bytes", "item_pages", "fused_merge", "mfma", "whole")


def last_error() -> str:
    return LIB.kvq_last_error().decode()


def _dt(dtype) -> int:
    if isinstance(dtype, str):
        if dtype not in DTYPES:
            raise ValueError("unknown KV dtype %r (expected one of %s)" % (dtype, list(DTYPES)))
        return DTYPES[dtype]
    return int(dtype)


def _check(rc: int):
    if rc != OK:
        msg = last_error()
        if rc == ERR_UNSUPPORTED:
            raise NotImplementedError(msg)
        if rc in (ERR_ARG, ERR_WORKSPACE):
            raise ValueError(msg)
        raise KvqError(rc, msg)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(device, stream) -> int | None:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    return torch.cuda.current_stream(device).cuda_stream


# ---- host-only -------------------------------------------------------------------

def pool_bytes(dtype, num_pages: int, page_size: int, n_heads: int, head_dim: int):
    """(total, code_bytes, scale_bytes) of one K or V pool; the cost model
    (kvq_pool_bytes returns the total and the scale part)."""
    sb = ctypes.c_int64(0)
    total = LIB.kvq_pool_bytes(_dt(dtype), num_pages, page_size, n_heads, head_dim,
                               ctypes.byref(sb))
    if total < 0:
        raise ValueError(last_error())
    return total, total - sb.value, sb.value


def workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim_v, max_pages, page_size) -> int:
    """kvq_paged_decode_workspace_bytes: enough for every storage type."""
    n = LIB.kvq_paged_decode_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim_v,
                                             max_pages, page_size)
    if n == 0:
        raise NotImplementedError(last_error())
    return n


def _host_lens(seq_lens_host):
    """An int32 numpy copy of the lengths for the host argument (None: absent)."""
    if seq_lens_host is None:
        return None, None
    import numpy as np
    arr = np.ascontiguousarray(seq_lens_host, dtype=np.int32)
    return arr, arr.ctypes.data


def debug_plan(dtype, batch, n_q_heads, n_kv_heads, head_dim_qk, head_dim_v, max_pages,
               max_new_tokens=0):
    """The decode planner's fields (PLAN_FIELDS) for these shapes, or None
    when it refuses them (kvq_debug_decode_plan)."""
    out = (ctypes.c_int64 * len(PLAN_FIELDS))()
    n = LIB.kvq_debug_decode_plan(_dt(dtype), batch, n_q_heads, n_kv_heads, head_dim_qk,
                                  head_dim_v, max_pages, max_new_tokens, out, len(PLAN_FIELDS))
    if n < 0:
        return None
    return dict(zip(PLAN_FIELDS, list(out)[:n]))


def debug_e4m3_encode_range(first_bits: int, count: int, out, stream=None) -> None:
    """The device e4m3 encoder over fp32 bit patterns first_bits .. + count - 1
    into the uint8 device tensor out (kvq_debug_e4m3_encode_range)."""
    _check(LIB.kvq_debug_e4m3_encode_range(first_bits, count, _ptr(out),
                                           _stream(out.device, stream)))


DS_ROW = 656  # bytes of one row of the fp8_ds_mla slab (576 elements)


def _row_dim(dtype, pool) -> int:
    """Elements per head row of a pool tensor (its last dimension is bytes for
    the 656-byte row)."""
    return 576 if _dt(dtype) == DTYPES["fp8_ds_mla"] else pool.shape[3]


def alloc_pool(dtype, num_pages: int, n_heads: int, head_dim: int, page_size: int = 16,
               device="cuda"):
    """Allocate (pool, scales) tensors of the layout above, sized by kvq_pool_bytes."""
    total, cb, sb = pool_bytes(dtype, num_pages, page_size, n_heads, head_dim)
    if _dt(dtype) == DTYPES["bf16"]:
        pool = torch.empty((num_pages, n_heads, page_size, head_dim), dtype=torch.bfloat16,
                           device=device)
        return pool, None
    if _dt(dtype) == DTYPES["fp8_ds_mla"]:  # 656-byte rows: codes, scales and rope together
        pool = torch.empty((num_pages, n_heads, page_size, DS_ROW), dtype=torch.uint8,
                           device=device)
        assert pool.numel() == cb
        return pool, None
    pool = torch.empty((num_pages, n_heads, page_size, head_dim), dtype=torch.uint8,
                       device=device)
    if sb == 0:  # the cast types: no scale buffer
        assert pool.numel() == cb
        return pool, None
    scales = torch.empty((num_pages, n_heads, page_size, head_dim // 32), dtype=torch.int16,
                         device=device)
    assert pool.numel() == cb and scales.numel() * 2 == sb
    return pool, scales


# ---- device calls -----------------------------------------------------------------

def store(dtype, k, v, slot_mapping, k_pool, k_scales, v_pool=None, v_scales=None,
          stream=None) -> None:
    """Quantize-on-store of k (and v) bf16 [n_tokens, n_heads, head_dim] (or
    [n_tokens, stride] rows whose first n_heads*head_dim elements are the heads)."""
    num_pages, n_heads, page_size, _ = k_pool.shape
    head_dim = _row_dim(dtype, k_pool)
    n_tokens = slot_mapping.numel()
    # a single token's leading stride is irrelevant (and may be anything)
    stride = k.stride(0) if n_tokens > 1 else n_heads * head_dim
    if v is not None and n_tokens > 1 and v.stride(0) != stride:
        raise ValueError("k and v must share the token stride")
    rc = LIB.kvq_store(_dt(dtype), _ptr(k), _ptr(v), stride, _ptr(slot_mapping), n_tokens,
                       n_heads, head_dim, page_size, num_pages, _ptr(k_pool), _ptr(k_scales),
                       _ptr(v_pool) if v is not None else None,
                       _ptr(v_scales) if v is not None else None,
                       _stream(k_pool.device, stream))
    _check(rc)


def dequant(dtype, pool, scales, slot_mapping, out=None, stream=None):
    """Rows at slot_mapping, dequantized to bf16 [n_tokens, n_heads, head_dim]."""
    num_pages, n_heads, page_size, _ = pool.shape
    head_dim = _row_dim(dtype, pool)
    n = slot_mapping.numel()
    if out is None:
        out = torch.empty((n, n_heads, head_dim), dtype=torch.bfloat16, device=pool.device)
    rc = LIB.kvq_dequant(_dt(dtype), _ptr(pool), _ptr(scales), _ptr(slot_mapping), n, n_heads,
                         head_dim, page_size, num_pages, _ptr(out),
                         _stream(pool.device, stream))
    _check(rc)
    return out


def paged_decode(dtype, q, k_pool, k_scales, v_pool, v_scales, page_table, seq_lens,
                 sm_scale: float, head_dim_v: int | None = None, out=None, lse=None,
                 workspace=None, stream=None, seq_lens_host=None):
    """One-token decode attention over the paged pool; returns (out, lse).

    Pass v_pool=k_pool (and v_scales=k_scales) for the shared MLA slab, with
    head_dim_v the V width taken from the front of each row.  seq_lens_host
    (optional, the same lengths on the host) sizes the launch exactly."""
    batch, n_q_heads, head_dim_qk = q.shape
    num_pages, n_kv_heads, page_size, _ = k_pool.shape
    if head_dim_v is None:
        head_dim_v = v_pool.shape[3]
    max_pages = page_table.shape[1]
    if page_table.stride(1) != 1:
        raise ValueError("page_table rows must be contiguous")
    # a size-1 leading dimension may carry any stride; the row length is then exact
    pt_stride = page_table.stride(0) if batch > 1 else max_pages
    if out is None:
        out = torch.empty((batch, n_q_heads, head_dim_v), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((batch, n_q_heads), dtype=torch.float32, device=q.device)
    need = workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim_v, max_pages, page_size)
    if workspace is None:  # zero-filled once; each call leaves it zeroed
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    _lens, lens_ptr = _host_lens(seq_lens_host)
    rc = LIB.kvq_paged_decode(_dt(dtype), _ptr(q), _ptr(k_pool), _ptr(k_scales), _ptr(v_pool),
                              _ptr(v_scales), _ptr(page_table), pt_stride,
                              _ptr(seq_lens), lens_ptr, batch, n_q_heads, n_kv_heads, head_dim_qk,
                              head_dim_v, page_size, max_pages, num_pages, float(sm_scale),
                              _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes,
                              _stream(q.device, stream))
    _check(rc)
    return out, lse


def _new_stride(new_k, batch, n_kv_heads, head_dim_qk) -> int:
    if new_k.stride(-1) != 1 or (new_k.dim() == 3 and new_k.stride(1) != head_dim_qk):
        raise ValueError("new_k rows must be contiguous [batch][n_kv_heads][head_dim]")
    return new_k.stride(0) if batch > 1 else n_kv_heads * head_dim_qk


def paged_decode_append(dtype, q, new_k, new_v, k_pool, k_scales, v_pool, v_scales, page_table,
                        seq_lens, sm_scale: float, head_dim_v: int | None = None, out=None,
                        lse=None, workspace=None, stream=None, seq_lens_host=None):
    """Store each sequence's new token (bf16 new_k / new_v [batch][n_kv_heads]
    [head_dim], position seq_lens[b] - 1), then decode; returns (out, lse).
    new_v is None for the shared MLA slab."""
    batch, n_q_heads, head_dim_qk = q.shape
    num_pages, n_kv_heads, page_size, _ = k_pool.shape
    if head_dim_v is None:
        head_dim_v = v_pool.shape[3]
    max_pages = page_table.shape[1]
    if page_table.stride(1) != 1:
        raise ValueError("page_table rows must be contiguous")
    pt_stride = page_table.stride(0) if batch > 1 else max_pages
    if out is None:
        out = torch.empty((batch, n_q_heads, head_dim_v), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((batch, n_q_heads), dtype=torch.float32, device=q.device)
    need = workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim_v, max_pages, page_size)
    if workspace is None:
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    _lens, lens_ptr = _host_lens(seq_lens_host)
    rc = LIB.kvq_paged_decode_append(
        _dt(dtype), _ptr(q), _ptr(new_k), _ptr(new_v),
        _new_stride(new_k, batch, n_kv_heads, head_dim_qk), _ptr(k_pool), _ptr(k_scales),
        _ptr(v_pool), _ptr(v_scales), _ptr(page_table), pt_stride, _ptr(seq_lens), lens_ptr,
        batch, n_q_heads, n_kv_heads, head_dim_qk, head_dim_v, page_size, max_pages, num_pages,
        float(sm_scale), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes,
        _stream(q.device, stream))
    _check(rc)
    return out, lse


def paged_decode_noalloc(dtype, q, k_pool, k_scales, v_pool, v_scales, page_table, seq_lens,
                         sm_scale: float, head_dim_v: int | None = None, out=None, lse=None,
                         stream=None, seq_lens_host=None):
    """paged_decode with the library's own scratch array as the workspace
    (kvq_paged_decode_noalloc); out and lse may be passed in so that the
    call allocates nothing."""
    batch, n_q_heads, head_dim_qk = q.shape
    num_pages, n_kv_heads, page_size, _ = k_pool.shape
    if head_dim_v is None:
        head_dim_v = v_pool.shape[3]
    max_pages = page_table.shape[1]
    pt_stride = page_table.stride(0) if batch > 1 else max_pages
    if out is None:
        out = torch.empty((batch, n_q_heads, head_dim_v), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((batch, n_q_heads), dtype=torch.float32, device=q.device)
    _lens, lens_ptr = _host_lens(seq_lens_host)
    rc = LIB.kvq_paged_decode_noalloc(_dt(dtype), _ptr(q), _ptr(k_pool), _ptr(k_scales),
                                      _ptr(v_pool), _ptr(v_scales), _ptr(page_table), pt_stride,
                                      _ptr(seq_lens), lens_ptr, batch, n_q_heads, n_kv_heads,
                                      head_dim_qk, head_dim_v, page_size, max_pages, num_pages,
                                      float(sm_scale), _ptr(out), _ptr(lse),
                                      _stream(q.device, stream))
    _check(rc)
    return out, lse


def sparse_workspace_bytes(dtype, batch, n_q_heads, topk) -> int:
    n = LIB.kvq_sparse_mla_decode_workspace_bytes(_dt(dtype), batch, n_q_heads, topk)
    if n == 0:
        raise NotImplementedError(last_error())
    return n


def sparse_mla_decode(dtype, q, slab, scales, page_table, seq_lens, topk_idx, sm_scale,
                      out=None, lse=None, workspace=None, stream=None):
    """Sparse top-k decode over the shared 576/512 slab: sequence b attends to
    the token positions listed in topk_idx[b] (int32 [batch, k], -1 = none)."""
    batch, n_q_heads, head_dim_qk = q.shape
    num_pages, _, page_size, _ = slab.shape
    max_pages = page_table.shape[1]
    topk = topk_idx.shape[1]
    if out is None:
        out = torch.empty((batch, n_q_heads, 512), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((batch, n_q_heads), dtype=torch.float32, device=q.device)
    need = sparse_workspace_bytes(dtype, batch, n_q_heads, topk)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    pt_stride = page_table.stride(0) if batch > 1 else max_pages
    tk_stride = topk_idx.stride(0) if batch > 1 else topk
    rc = LIB.kvq_sparse_mla_decode(_dt(dtype), _ptr(q), _ptr(slab), _ptr(scales),
                                   _ptr(page_table), pt_stride, _ptr(seq_lens), _ptr(topk_idx),
                                   tk_stride, topk, batch, n_q_heads, page_size, max_pages,
                                   num_pages, float(sm_scale), _ptr(out), _ptr(lse),
                                   _ptr(workspace), workspace.numel(),
                                   _stream(q.device, stream))
    _check(rc)
    return out, lse


def extend_workspace_bytes(dtype, batch, n_q_heads, n_kv_heads, head_dim, page_size, max_pages,
                           max_new_tokens) -> int:
    n = LIB.kvq_extend_attention_workspace_bytes(_dt(dtype), batch, n_q_heads, n_kv_heads,
                                                 head_dim, page_size, max_pages, max_new_tokens)
    if n == 0:
        raise NotImplementedError(last_error())
    return n


def extend_attention(dtype, q, q_start, max_new_tokens, k_pool, k_scales, v_pool, v_scales,
                     page_table, seq_lens, sm_scale, out=None, lse=None, workspace=None,
                     stream=None):
    """Causal extend (prefill) attention: q bf16 [T, Hq, D] holds the new
    tokens of every sequence back to back (q_start int32 [batch + 1]); each
    attends to its sequence's pool up to its own position.  Pass v_pool=k_pool
    for the shared 576/512 slab (out [T, Hq, 512]).  Returns (out, lse)."""
    T, n_q_heads, head_dim = q.shape
    head_dim_v = 512 if v_pool is k_pool else head_dim
    num_pages, n_kv_heads, page_size, _ = k_pool.shape
    batch = seq_lens.numel()
    max_pages = page_table.shape[1]
    if page_table.stride(1) != 1:
        raise ValueError("page_table rows must be contiguous")
    pt_stride = page_table.stride(0) if batch > 1 else max_pages
    if out is None:
        out = torch.empty((T, n_q_heads, head_dim_v), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((T, n_q_heads), dtype=torch.float32, device=q.device)
    need = extend_workspace_bytes(dtype, batch, n_q_heads, n_kv_heads, head_dim, page_size,
                                  max_pages, max_new_tokens)
    if workspace is None:  # zero-filled once; each call leaves it zeroed
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    rc = LIB.kvq_extend_attention(_dt(dtype), _ptr(q), _ptr(q_start), max_new_tokens,
                                  _ptr(k_pool), _ptr(k_scales), _ptr(v_pool), _ptr(v_scales),
                                  _ptr(page_table), pt_stride, _ptr(seq_lens), batch, n_q_heads,
                                  n_kv_heads, head_dim, page_size, max_pages, num_pages,
                                  float(sm_scale), _ptr(out), _ptr(lse), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(),
                                  _stream(q.device, stream))
    _check(rc)
    return out, lse


class PreparedExtend:
    """kvq_extend_attention with every argument resolved once."""

    def __init__(self, dtype, q, q_start, max_new_tokens, k_pool, k_scales, v_pool, v_scales,
                 page_table, seq_lens, sm_scale, workspace=None, stream=None):
        T, n_q_heads, head_dim = q.shape
        num_pages, n_kv_heads, page_size, _ = k_pool.shape
        batch = seq_lens.numel()
        max_pages = page_table.shape[1]
        head_dim_v = 512 if v_pool is k_pool else head_dim
        self.out = torch.empty((T, n_q_heads, head_dim_v), dtype=torch.bfloat16, device=q.device)
        self.lse = torch.empty((T, n_q_heads), dtype=torch.float32, device=q.device)
        need = extend_workspace_bytes(dtype, batch, n_q_heads, n_kv_heads, head_dim, page_size,
                                      max_pages, max_new_tokens)
        self.workspace = workspace if workspace is not None else torch.zeros(
            need, dtype=torch.uint8, device=q.device)
        pt_stride = page_table.stride(0) if batch > 1 else max_pages
        self._keep = (q, q_start, k_pool, k_scales, v_pool, v_scales, page_table, seq_lens)
        self.args = (_dt(dtype), _ptr(q), _ptr(q_start), max_new_tokens, _ptr(k_pool),
                     _ptr(k_scales), _ptr(v_pool), _ptr(v_scales), _ptr(page_table), pt_stride,
                     _ptr(seq_lens), batch, n_q_heads, n_kv_heads, head_dim, page_size, max_pages,
                     num_pages, float(sm_scale), _ptr(self.out), _ptr(self.lse),
                     _ptr(self.workspace), self.workspace.numel(), _stream(q.device, stream))

    def __call__(self):
        _check(LIB.kvq_extend_attention(*self.args))


class PreparedDecode:
    """kvq_paged_decode with every argument resolved once (for timed loops and
    graph capture): calling it only crosses into the library."""

    def __init__(self, dtype, q, k_pool, k_scales, v_pool, v_scales, page_table, seq_lens,
                 sm_scale, head_dim_v=None, out=None, lse=None, workspace=None, stream=None,
                 seq_lens_host=None, new_k=None, new_v=None):
        """With new_k (and new_v, unless the pool is the shared slab) the call
        is kvq_paged_decode_append: each sequence's new token is stored first."""
        batch, n_q_heads, head_dim_qk = q.shape
        num_pages, n_kv_heads, page_size, _ = k_pool.shape
        head_dim_v = head_dim_v or v_pool.shape[3]
        max_pages = page_table.shape[1]
        self.out = out if out is not None else torch.empty(
            (batch, n_q_heads, head_dim_v), dtype=torch.bfloat16, device=q.device)
        self.lse = lse if lse is not None else torch.empty(
            (batch, n_q_heads), dtype=torch.float32, device=q.device)
        need = workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim_v, max_pages, page_size)
        self.workspace = workspace if workspace is not None else torch.zeros(
            need, dtype=torch.uint8, device=q.device)
        pt_stride = page_table.stride(0) if batch > 1 else max_pages
        lens, lens_ptr = _host_lens(seq_lens_host)
        self._keep = (q, k_pool, k_scales, v_pool, v_scales, page_table, seq_lens, lens, new_k,
                      new_v)
        head = (_dt(dtype), _ptr(q))
        if new_k is not None:
            head += (_ptr(new_k), _ptr(new_v), _new_stride(new_k, batch, n_kv_heads, head_dim_qk))
        self.fn = LIB.kvq_paged_decode_append if new_k is not None else LIB.kvq_paged_decode
        self.args = head + (_ptr(k_pool), _ptr(k_scales), _ptr(v_pool),
                            _ptr(v_scales), _ptr(page_table), pt_stride, _ptr(seq_lens), lens_ptr,
                            batch, n_q_heads, n_kv_heads, head_dim_qk, head_dim_v, page_size,
                            max_pages, num_pages, float(sm_scale), _ptr(self.out), _ptr(self.lse),
                            _ptr(self.workspace), self.workspace.numel(),
                            _stream(q.device, stream))

    def __call__(self):
        _check(self.fn(*self.args))


class PreparedSparse:
    """kvq_sparse_mla_decode with every argument resolved once."""

    def __init__(self, dtype, q, slab, scales, page_table, seq_lens, topk_idx, sm_scale,
                 out=None, lse=None, workspace=None, stream=None):
        batch, n_q_heads, _ = q.shape
        num_pages, _, page_size, _ = slab.shape
        max_pages, topk = page_table.shape[1], topk_idx.shape[1]
        self.out = out if out is not None else torch.empty(
            (batch, n_q_heads, 512), dtype=torch.bfloat16, device=q.device)
        self.lse = lse if lse is not None else torch.empty(
            (batch, n_q_heads), dtype=torch.float32, device=q.device)
        need = sparse_workspace_bytes(dtype, batch, n_q_heads, topk)
        self.workspace = workspace if workspace is not None else torch.empty(
            need, dtype=torch.uint8, device=q.device)
        pt_stride = page_table.stride(0) if batch > 1 else max_pages
        tk_stride = topk_idx.stride(0) if batch > 1 else topk
        self._keep = (q, slab, scales, page_table, seq_lens, topk_idx)
        self.args = (_dt(dtype), _ptr(q), _ptr(slab), _ptr(scales), _ptr(page_table), pt_stride,
                     _ptr(seq_lens), _ptr(topk_idx), tk_stride, topk, batch, n_q_heads,
                     page_size, max_pages, num_pages, float(sm_scale), _ptr(self.out),
                     _ptr(self.lse), _ptr(self.workspace), self.workspace.numel(),
                     _stream(q.device, stream))

    def __call__(self):
        _check(LIB.kvq_sparse_mla_decode(*self.args))


class PreparedStore:
    """kvq_store with every argument resolved once."""

    def __init__(self, dtype, k, v, slot_mapping, k_pool, k_scales, v_pool=None, v_scales=None,
                 stream=None):
        num_pages, n_heads, page_size, _ = k_pool.shape
        head_dim = _row_dim(dtype, k_pool)
        n_tokens = slot_mapping.numel()
        stride = k.stride(0) if n_tokens > 1 else n_heads * head_dim
        self._keep = (k, v, slot_mapping, k_pool, k_scales, v_pool, v_scales)
        self.args = (_dt(dtype), _ptr(k), _ptr(v), stride, _ptr(slot_mapping), n_tokens, n_heads,
                     head_dim, page_size, num_pages, _ptr(k_pool), _ptr(k_scales),
                     _ptr(v_pool) if v is not None else None,
                     _ptr(v_scales) if v is not None else None, _stream(k_pool.device, stream))

    def __call__(self):
        _check(LIB.kvq_store(*self.args))
