"""CPU oracle for the block-scaled 8-bit paged KV cache (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this package.  The product path (the HIP library and its Python
binding) never imports, links or calls it.

The arithmetic lives in ``kvq_oracle.c`` (plain scalar C, compiled with gcc,
no fast-math, no FMA contraction); this module only builds it and marshals
numpy arrays through ctypes.  See the C file's header for the sources and the
readings taken where the pages leave a step open.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kvq_oracle.c")
LIB = os.path.join(HERE, "libkvq_oracle.so")

BF16, FP8_E4M3, Q8_0, FP8_E4M3_CAST, FP8_E5M2_CAST, FP8_DS_MLA = 0, 1, 2, 3, 4, 5
QTYPES = {"bf16": BF16, "fp8_e4m3": FP8_E4M3, "q8_0": Q8_0, "fp8_e4m3_cast": FP8_E4M3_CAST,
          "fp8_e5m2_cast": FP8_E5M2_CAST, "fp8_ds_mla": FP8_DS_MLA}
# the 656-byte MLA row: 512 e4m3 codes, 4 fp32 scales (one per 128), 64 bf16 rope
DS_ROW = 656
# storage types with a scale buffer beside the pool
SCALED = ("fp8_e4m3", "q8_0")

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/libkvq_oracle.so``."""
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
           "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
           "-o", tmp, SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def lib() -> ctypes.CDLL:
    """The oracle library.  KVQ_ORACLE_LIB may name another build of the same
    source (the mutation tests load deliberately broken copies this way)."""
    global _lib
    if _lib is None:
        path = os.environ.get("KVQ_ORACLE_LIB")
        if not path:
            build(force=False)
            path = LIB
        _lib = ctypes.CDLL(path)
        _declare(_lib)
    return _lib


def _declare(L):
    c = ctypes
    P = c.c_void_p
    L.kvo_f16_value.argtypes = [c.c_uint16]
    L.kvo_f16_value.restype = c.c_double
    L.kvo_f16_from_double.argtypes = [c.c_double]
    L.kvo_f16_from_double.restype = c.c_uint16
    L.kvo_bf16_value.argtypes = [c.c_uint16]
    L.kvo_bf16_value.restype = c.c_double
    L.kvo_bf16_from_double.argtypes = [c.c_double]
    L.kvo_bf16_from_double.restype = c.c_uint16
    L.kvo_e4m3_value.argtypes = [c.c_uint8]
    L.kvo_e4m3_value.restype = c.c_double
    L.kvo_e4m3_encode.argtypes = [c.c_float]
    L.kvo_e4m3_encode.restype = c.c_uint8
    L.kvo_q8_encode.argtypes = [c.c_float]
    L.kvo_q8_encode.restype = c.c_int8
    L.kvo_block_scale.argtypes = [c.c_int, c.c_float]
    L.kvo_block_scale.restype = c.c_uint16
    L.kvo_quantize_block.argtypes = [c.c_int, P, c.c_int, P, P]
    L.kvo_quantize_block.restype = None
    L.kvo_element_value.argtypes = [c.c_int, c.c_uint8, c.c_uint16]
    L.kvo_element_value.restype = c.c_double
    L.kvo_store.argtypes = [c.c_int, P, c.c_int64, P, c.c_int64, c.c_int, c.c_int, c.c_int,
                            c.c_int64, P, P, c.c_int]
    L.kvo_store.restype = None
    L.kvo_dequant.argtypes = [c.c_int, P, P, P, c.c_int64, c.c_int, c.c_int, c.c_int,
                              c.c_int64, P, P, c.c_int]
    L.kvo_dequant.restype = None
    L.kvo_paged_decode.argtypes = [c.c_int, P, P, P, P, P, P, c.c_int64, P,
                                   c.c_int, c.c_int, c.c_int, c.c_int, c.c_int, c.c_int,
                                   c.c_int, c.c_int64, c.c_double, P, c.c_int64, P, P, c.c_int]
    L.kvo_paged_decode.restype = None
    L.kvo_e4m3_encode_array.argtypes = [P, c.c_int64, P]
    L.kvo_e4m3_encode_array.restype = None
    L.kvo_e4m3_encode_bits.argtypes = [c.c_uint32, c.c_int64, P]
    L.kvo_e4m3_encode_bits.restype = None
    L.kvo_q8_encode_array.argtypes = [P, c.c_int64, P]
    L.kvo_q8_encode_array.restype = None
    L.kvo_sparse_mla_decode.argtypes = [c.c_int, P, P, P, P, c.c_int64, P, P, c.c_int64, c.c_int,
                                        c.c_int, c.c_int, c.c_int, c.c_int, c.c_int, c.c_int,
                                        c.c_int64, c.c_double, P, P, c.c_int]
    L.kvo_sparse_mla_decode.restype = None
    L.kvo_extend_attention.argtypes = [c.c_int, P, P, P, P, P, P, P, c.c_int64, P, c.c_int, c.c_int,
                                       c.c_int, c.c_int, c.c_int, c.c_int, c.c_int, c.c_int64,
                                       c.c_double, P, P, c.c_int]
    L.kvo_extend_attention.restype = None
    L.kvo_e5m2_value.argtypes = [c.c_uint8]
    L.kvo_e5m2_value.restype = c.c_double
    L.kvo_e5m2_encode.argtypes = [c.c_float]
    L.kvo_e5m2_encode.restype = c.c_uint8
    L.kvo_cast_encode.argtypes = [c.c_int, c.c_float]
    L.kvo_cast_encode.restype = c.c_uint8
    L.kvo_cast_encode_array.argtypes = [c.c_int, P, c.c_int64, P]
    L.kvo_cast_encode_array.restype = None


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _qt(qtype) -> int:
    return QTYPES[qtype] if isinstance(qtype, str) else int(qtype)


# ---- scalar / elementwise helpers -------------------------------------------------

def e4m3_encode(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    lib().kvo_e4m3_encode_array(_ptr(v), v.size, _ptr(out))
    return out


def e4m3_encode_bits(first: int, count: int, threads: int | None = None) -> np.ndarray:
    """e4m3 codes of the fp32 values whose bit patterns are first .. first +
    count - 1 (the encoder over a range, split across threads)."""
    from concurrent.futures import ThreadPoolExecutor
    out = np.empty(count, dtype=np.uint8)
    threads = threads or default_threads()
    per = -(-count // threads) if count else 0
    L = lib()
    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(lambda k: L.kvo_e4m3_encode_bits(first + k * per, min(per, count - k * per),
                                                       out.ctypes.data + k * per),
                    [k for k in range(threads) if k * per < count]))
    return out


def q8_encode(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.int8)
    lib().kvo_q8_encode_array(_ptr(v), v.size, _ptr(out))
    return out


def cast_encode(qtype, v: np.ndarray) -> np.ndarray:
    """The cast store of each element (per-tensor scale 1.0): clamp, round."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    lib().kvo_cast_encode_array(_qt(qtype), _ptr(v), v.size, _ptr(out))
    return out


def e5m2_value(code: int) -> float:
    return lib().kvo_e5m2_value(code)


def e4m3_value(code: int) -> float:
    return lib().kvo_e4m3_value(code)


def f16_value(bits: int) -> float:
    return lib().kvo_f16_value(bits)


def block_scale(qtype, amax: float) -> int:
    return lib().kvo_block_scale(_qt(qtype), amax)


def quantize_block(qtype, x_bf16: np.ndarray):
    """x_bf16: uint16 bf16 bit patterns, length 32.  Returns (codes uint8[32], scale bits)."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    codes = np.empty(x.size, dtype=np.uint8)
    scale = np.zeros(1, dtype=np.uint16)
    lib().kvo_quantize_block(_qt(qtype), _ptr(x), x.size, _ptr(codes), _ptr(scale))
    return codes, int(scale[0])


# ---- pool-level operations --------------------------------------------------------

def store(qtype, src_bf16: np.ndarray, slots: np.ndarray, n_heads: int, head_dim: int,
          page_size: int, num_pages: int, pool: np.ndarray, scales: np.ndarray | None,
          token_stride: int | None = None, threads: int | None = None) -> None:
    """Quantize ``src_bf16`` (uint16 [n_tokens][..]) into ``pool``/``scales`` in place."""
    qt = _qt(qtype)
    src = np.ascontiguousarray(src_bf16, dtype=np.uint16)
    slots = np.ascontiguousarray(slots, dtype=np.int32)
    n_tokens = slots.size
    if token_stride is None:
        token_stride = n_heads * head_dim
    lib().kvo_store(qt, _ptr(src), token_stride, _ptr(slots), n_tokens, n_heads, head_dim,
                    page_size, num_pages, _ptr(pool), _ptr(scales),
                    threads or default_threads())


def dequant(qtype, pool: np.ndarray, scales: np.ndarray | None, slots: np.ndarray,
            n_heads: int, head_dim: int, page_size: int, num_pages: int,
            threads: int | None = None):
    """Returns (exact float64 [n][H][D], bf16 bits uint16 [n][H][D])."""
    slots = np.ascontiguousarray(slots, dtype=np.int32)
    n = slots.size
    f64 = np.empty((n, n_heads, head_dim), dtype=np.float64)
    b16 = np.empty((n, n_heads, head_dim), dtype=np.uint16)
    lib().kvo_dequant(_qt(qtype), _ptr(pool), _ptr(scales), _ptr(slots), n, n_heads, head_dim,
                      page_size, num_pages, _ptr(f64), _ptr(b16), threads or default_threads())
    return f64, b16


def paged_decode(qtype, q_bf16: np.ndarray, k_pool: np.ndarray, k_scales, v_pool: np.ndarray,
                 v_scales, page_table: np.ndarray, seq_lens: np.ndarray, n_kv_heads: int,
                 head_dim_qk: int, head_dim_v: int, page_size: int, num_pages: int,
                 sm_scale: float, rows: np.ndarray | None = None,
                 threads: int | None = None):
    """Attention in double.  q_bf16: uint16 [B][Hq][Dqk].  page_table: int32 [B][W].

    Pass ``v_pool is k_pool`` for the shared MLA slab.  Returns (out float64
    [n_rows][Dv], lse float64 [n_rows]); rows = b*Hq+h, all rows when None.
    """
    q = np.ascontiguousarray(q_bf16, dtype=np.uint16)
    B, Hq = q.shape[0], q.shape[1]
    pt = np.ascontiguousarray(page_table, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    n_rows = B * Hq if rows is None else len(rows)
    rows_a = None if rows is None else np.ascontiguousarray(rows, dtype=np.int32)
    out = np.empty((n_rows, head_dim_v), dtype=np.float64)
    lse = np.empty(n_rows, dtype=np.float64)
    kp = _ptr(k_pool)
    vp = kp if v_pool is k_pool else _ptr(v_pool)
    ks = _ptr(k_scales)
    vs = ks if v_pool is k_pool else _ptr(v_scales)
    lib().kvo_paged_decode(_qt(qtype), _ptr(q), kp, ks, vp, vs, _ptr(pt), pt.shape[1], _ptr(sl),
                           B, Hq, n_kv_heads, head_dim_qk, head_dim_v, page_size, pt.shape[1],
                           num_pages, float(sm_scale), _ptr(rows_a), n_rows, _ptr(out),
                           _ptr(lse), threads or default_threads())
    return out, lse


def extend_attention(qtype, q_bf16: np.ndarray, q_start: np.ndarray, k_pool: np.ndarray,
                     k_scales, v_pool: np.ndarray, v_scales, page_table: np.ndarray,
                     seq_lens: np.ndarray, n_kv_heads: int, head_dim: int, page_size: int,
                     num_pages: int, sm_scale: float, threads: int | None = None,
                     head_dim_v: int | None = None):
    """Causal extend attention in double.  q_bf16: uint16 [T][Hq][D], the new
    tokens of every sequence back to back; q_start: int32 [B+1] (q_start[0] =
    0).  Pass ``v_pool is k_pool`` and head_dim_v for the shared MLA slab.
    Returns (out float64 [T*Hq][Dv], lse float64 [T*Hq])."""
    head_dim_v = head_dim_v or head_dim
    q = np.ascontiguousarray(q_bf16, dtype=np.uint16)
    T, Hq = q.shape[0], q.shape[1]
    qs = np.ascontiguousarray(q_start, dtype=np.int32)
    assert qs[0] == 0 and qs[-1] == T and np.all(np.diff(qs) >= 0)
    pt = np.ascontiguousarray(page_table, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    B = len(sl)
    out = np.empty((T * Hq, head_dim_v), dtype=np.float64)
    lse = np.empty(T * Hq, dtype=np.float64)
    kp = _ptr(k_pool)
    vp = kp if v_pool is k_pool else _ptr(v_pool)
    lib().kvo_extend_attention(_qt(qtype), _ptr(q), _ptr(qs), kp, _ptr(k_scales),
                               vp, _ptr(v_scales), _ptr(pt), pt.shape[1], _ptr(sl), B,
                               Hq, n_kv_heads, head_dim, head_dim_v, page_size, pt.shape[1],
                               num_pages,
                               float(sm_scale), _ptr(out), _ptr(lse),
                               threads or default_threads())
    return out, lse


def sparse_mla_decode(qtype, q_bf16: np.ndarray, slab: np.ndarray, scales, page_table: np.ndarray,
                      seq_lens: np.ndarray, topk: np.ndarray, head_dim_qk: int, head_dim_v: int,
                      page_size: int, num_pages: int, sm_scale: float,
                      threads: int | None = None):
    """Sparse top-k decode over the shared slab, in double.  topk: int32
    [B][k] token positions (-1 = padding).  Returns (out float64 [B*Hq][Dv],
    lse float64 [B*Hq])."""
    q = np.ascontiguousarray(q_bf16, dtype=np.uint16)
    B, Hq = q.shape[0], q.shape[1]
    pt = np.ascontiguousarray(page_table, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    tk = np.ascontiguousarray(topk, dtype=np.int32)
    out = np.empty((B * Hq, head_dim_v), dtype=np.float64)
    lse = np.empty(B * Hq, dtype=np.float64)
    lib().kvo_sparse_mla_decode(_qt(qtype), _ptr(q), _ptr(slab), _ptr(scales), _ptr(pt),
                                pt.shape[1], _ptr(sl), _ptr(tk), tk.shape[1], tk.shape[1], B, Hq,
                                head_dim_qk, head_dim_v, page_size, pt.shape[1], num_pages,
                                float(sm_scale), _ptr(out), _ptr(lse),
                                threads or default_threads())
    return out, lse
