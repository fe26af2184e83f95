"""Helpers shared by the GPU parity tests: move seeded inputs to the device,
run the library through its binding, and run the oracle on the same inputs.

Inputs come from ``paged_decode_attention_amd.workloads`` or are built here
from numpy; expected values come only from ``oracle``.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
from paged_decode_attention_amd import workloads as W

requires_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


def say(*a):
    """Name the case on stdout before a GPU step (a fault ends the process)."""
    print(*a, flush=True)
    sys.stdout.flush()


def kvq():
    from paged_decode_attention_amd import kvq as k
    return k


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def dev_i32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def host_u8(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint8) if t.dtype == torch.uint8 else t.cpu().view(torch.uint8).numpy()


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def np_pool(qtype, num_pages, H, D, fill_code=0, fill_scale=0):
    if qtype == "bf16":
        return np.full((num_pages, H, W.PAGE, D), fill_scale, np.uint16), None
    if qtype == "fp8_ds_mla":  # 656-byte rows
        return np.full((num_pages, H, W.PAGE, oracle.DS_ROW), fill_code, np.uint8), None
    codes = np.full((num_pages, H, W.PAGE, D), fill_code, np.uint8)
    if qtype not in oracle.SCALED:  # the cast types: no scale buffer
        return codes, None
    return codes, np.full((num_pages, H, W.PAGE, D // 32), fill_scale, np.uint16)


def gpu_pool_from(np_pool_arr, np_scales):
    """Upload oracle-layout pool arrays (used for poison fills)."""
    if np_pool_arr.dtype == np.uint16:
        return dev_bf16(np_pool_arr), None
    if np_scales is None:
        return torch.from_numpy(np_pool_arr).cuda(), None
    return (torch.from_numpy(np_pool_arr).cuda(),
            torch.from_numpy(np_scales.view(np.int16)).cuda())


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / max |ref| over the whole output (0 when both are 0)."""
    den = np.abs(ref).max()
    num = np.abs(got - ref).max()
    return float(num / den) if den > 0 else float(num)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return W.bf16_bits_to_f32(bits).astype(np.float64)


def fill_both(wl: W.Workload, qtype: str):
    """Fill the pool with every slot's source rows on the GPU (kvq_store) and on
    the CPU (oracle.store).  Returns dict with device and host pools."""
    k = kvq()
    n = wl.n_slots
    H, D = wl.n_kv_heads, wl.head_dim_qk
    slots = np.arange(n, dtype=np.int32)
    ksrc = wl.kv_rows(0, 0, n)
    vsrc = None if wl.shared else wl.kv_rows(1, 0, n)
    kp, ks = k.alloc_pool(qtype, wl.num_pages, H, D)
    vp, vs = (kp, ks) if wl.shared else k.alloc_pool(qtype, wl.num_pages, H, D)
    d_slots = dev_i32(slots)
    say("store", wl.name, qtype, "slots", n)
    k.store(qtype, dev_bf16(ksrc), None if wl.shared else dev_bf16(vsrc), d_slots, kp, ks,
            None if wl.shared else vp, None if wl.shared else vs)
    torch.cuda.synchronize()
    okp, oks = np_pool(qtype, wl.num_pages, H, D)
    oracle.store(qtype, ksrc, slots, H, D, W.PAGE, wl.num_pages, okp, oks)
    if wl.shared:
        ovp, ovs = okp, oks
    else:
        ovp, ovs = np_pool(qtype, wl.num_pages, H, D)
        oracle.store(qtype, vsrc, slots, H, D, W.PAGE, wl.num_pages, ovp, ovs)
    return dict(kp=kp, ks=ks, vp=vp, vs=vs, okp=okp, oks=oks, ovp=ovp, ovs=ovs)


def decode_both(wl: W.Workload, qtype: str, pools: dict, rows=None, threads=None):
    """GPU decode of the whole batch and oracle decode of `rows` (all if None).
    Returns (gpu_out f64 [B*Hq][Dv], gpu_lse f64 [B*Hq], ora_out, ora_lse, rows)."""
    k = kvq()
    q = wl.query()
    say("decode", wl.name, qtype)
    out, lse = k.paged_decode(qtype, dev_bf16(q), pools["kp"], pools["ks"], pools["vp"],
                              pools["vs"], dev_i32(wl.page_table), dev_i32(wl.seq_lens),
                              wl.sm_scale, head_dim_v=wl.head_dim_v)
    torch.cuda.synchronize()
    g_out = bf16_to_f64(host_u16(out)).reshape(wl.batch * wl.n_q_heads, wl.head_dim_v)
    g_lse = lse.cpu().numpy().astype(np.float64).reshape(-1)
    if rows is None:
        rows = np.arange(wl.batch * wl.n_q_heads, dtype=np.int32)
    vp = pools["okp"] if wl.shared else pools["ovp"]
    vs = pools["oks"] if wl.shared else pools["ovs"]
    o_out, o_lse = oracle.paged_decode(qtype, q, pools["okp"], pools["oks"], vp, vs,
                                       wl.page_table, wl.seq_lens, wl.n_kv_heads,
                                       wl.head_dim_qk, wl.head_dim_v, W.PAGE, wl.num_pages,
                                       wl.sm_scale, rows=rows, threads=threads)
    return g_out, g_lse, o_out, o_lse, rows
