"""Seeded synthetic inputs for the store and paged-decode workloads.

This module only draws numbers and lays out page tables; it holds none of the
quantization or attention arithmetic, and both the HIP path (tests, bench) and
the CPU oracle take their inputs from it.  Everything is numpy PCG64 with a
fixed seed; K/V rows are generated in chunks of 4096 slots from independent
sub-streams, so any slot range can be regenerated without the rest.  Values
are rounded to bf16 with torch's conversion (round to nearest even).

Workloads (all with page size 16):
  tiny     1 seq x 1024 tokens, 16 q / 8 kv heads, head_dim 128, identity
           page table; K, V ~ N(0,1) * per-channel LogNormal(0, 0.5).
  qwen3    batch 8 x 16384 tokens, 16 q / 8 kv heads, head_dim 128 (the
           Qwen3-1.7B attention shape), random-permutation page tables;
           K, V ~ N(0,1) with 0.1% of elements x30.
  ragged256  batch 8, contexts uniform in [4096, 32768], 16 q / 2 kv heads,
           head_dim 256 (the Qwen3.6-35B-A3B attention shape); N(0,1).
  single256  batch 1 x 262144 tokens, same heads; N(0,1).
  mla      batch 1 x 163840 tokens, one shared 576-wide row per token (512
           latent + 64 rope), 128 q heads, V = first 512; the latent part is
           already on the e4m3 grid under power-of-two block-64 scales, the
           rope tail is plain bf16 N(0,1).
  mixed    a 2^20-token pool (65536 pages) of N(0,1) background (page-seeded,
           see Workload.page_rows), batch 64
           with contexts log-uniform in [1024, 131072], 8192 new tokens (the
           last 128 of each sequence) to store, with 1% all-zero 32-blocks,
           1% constant blocks and 0.1% +-1e4 outliers; 1% of the older page-
           table columns masked with -1.
"""
from __future__ import annotations

import math
import os
from dataclasses import dataclass, field

import numpy as np
import torch

PAGE = 16
CHUNK = 4096  # slots per independent random sub-stream


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclass
class Workload:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim_qk: int
    head_dim_v: int
    num_pages: int
    seq_lens: np.ndarray          # int32 [batch]
    page_table: np.ndarray        # int32 [batch, max_pages]
    seed: int
    kind: str = "normal"          # value recipe for pool rows
    shared: bool = False          # single slab, K == V
    layer_replicas: int = 1       # bench: distinct copies of the pool swept per step
    new_tokens: dict = field(default_factory=dict)  # "slots": int32 [n] (mixed only)

    @property
    def max_pages(self) -> int:
        return self.page_table.shape[1]

    @property
    def n_slots(self) -> int:
        return self.num_pages * PAGE

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim_qk)

    # ---- value generation ----------------------------------------------------
    def _chunk_rows(self, tensor: int, c: int) -> np.ndarray:
        """float32 [CHUNK, n_kv_heads, head_dim_qk] for slot chunk c of tensor 0 (K) / 1 (V)."""
        H, D = self.n_kv_heads, self.head_dim_qk
        rng = np.random.Generator(np.random.PCG64([self.seed, tensor, c]))
        if self.kind == "mla":
            return _mla_rows(rng, CHUNK)[:, None, :]
        x = rng.standard_normal((CHUNK, H, D), dtype=np.float32)
        if self.kind == "outlier30":
            hit = rng.random((CHUNK, H, D)) < 0.001
            x[hit] *= 30.0
        elif self.kind == "channel":
            ch = np.random.Generator(np.random.PCG64([self.seed, tensor, 1 << 30]))
            m = np.exp(ch.normal(0.0, 0.5, (H, D))).astype(np.float32)
            x *= m[None]
        return x

    def kv_rows(self, tensor: int, lo: int, hi: int) -> np.ndarray:
        """bf16 bits uint16 [hi-lo, n_kv_heads, head_dim] of the pool's source rows."""
        out = []
        for c in range(lo // CHUNK, (hi + CHUNK - 1) // CHUNK):
            rows = self._chunk_rows(tensor, c)
            a, b = max(lo, c * CHUNK) - c * CHUNK, min(hi, (c + 1) * CHUNK) - c * CHUNK
            out.append(rows[a:b])
        if not out:
            return np.zeros((0, self.n_kv_heads, self.head_dim_qk), np.uint16)
        return to_bf16_bits(np.concatenate(out))

    def page_rows(self, tensor: int, pages) -> np.ndarray:
        """bf16 bits uint16 [len(pages) * 16, n_kv_heads, head_dim] for the slots
        of `pages`, each page drawn from its own sub-stream (N(0,1)).  The mixed
        workload's pool background is defined this way, so that any subset of
        its 65536 pages can be generated on its own."""
        from concurrent.futures import ThreadPoolExecutor
        H, D = self.n_kv_heads, self.head_dim_qk
        pages = np.asarray(pages, dtype=np.int64)
        out = np.empty((len(pages), PAGE, H, D), np.float32)

        def fill(i):  # numpy draws without holding the GIL
            rng = np.random.Generator(np.random.PCG64([self.seed, tensor, 1 << 24, int(pages[i])]))
            out[i] = rng.standard_normal((PAGE, H, D), dtype=np.float32)

        with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
            list(ex.map(fill, range(len(pages))))
        return to_bf16_bits(out.reshape(-1, H, D))

    def query(self) -> np.ndarray:
        rng = np.random.Generator(np.random.PCG64([self.seed, 7, 0]))
        q = rng.standard_normal((self.batch, self.n_q_heads, self.head_dim_qk), dtype=np.float32)
        return to_bf16_bits(q)

    def new_rows(self) -> np.ndarray:
        """Rows of the tokens stored in the timed step (mixed): bf16 bits
        [2, n_new, n_kv_heads, head_dim] for K and V."""
        n = len(self.new_tokens["slots"])
        H, D = self.n_kv_heads, self.head_dim_qk
        rng = np.random.Generator(np.random.PCG64([self.seed, 9, 0]))
        x = rng.standard_normal((2, n, H, D), dtype=np.float32)
        blocks = x.reshape(2, n, H, D // 32, 32)
        pick = rng.random(blocks.shape[:-1])
        blocks[pick < 0.01] = 0.0                                  # all-zero blocks
        const = (pick >= 0.01) & (pick < 0.02)                     # constant blocks
        c = rng.standard_normal(blocks.shape[:-1], dtype=np.float32)
        blocks[const] = c[const][:, None]
        out = rng.random(x.shape) < 0.001                          # +-1e4 outliers
        x[out] = np.where(rng.random(out.sum()) < 0.5, -1e4, 1e4).astype(np.float32)
        return to_bf16_bits(x)

    def algorithmic_bytes(self, qtype: str) -> int:
        """Bytes the decode must move: codes + scales of every valid token of
        every kv head (K and V, or the one shared row), Q, O, the page-table
        entries walked and seq_lens.  Masked pages are not counted."""
        D, Dv = self.head_dim_qk, self.head_dim_v
        per = {"bf16": 2.0, "fp8_e4m3": 17 / 16, "q8_0": 17 / 16, "fp8_e4m3_cast": 1.0,
               "fp8_e5m2_cast": 1.0, "fp8_ds_mla": 656 / 576}[qtype]  # 656-byte row: whole row
        n_valid = 0
        for b in range(self.batch):
            L = min(int(self.seq_lens[b]), self.max_pages * PAGE)
            cols = self.page_table[b, : (L + PAGE - 1) // PAGE]
            ok = (cols >= 0) & (cols < self.num_pages)
            full = ok.copy()
            valid_tokens = int(ok.sum()) * PAGE
            if L % PAGE and len(cols) and ok[-1]:
                valid_tokens -= PAGE - L % PAGE
            n_valid += valid_tokens
        row = (D if self.shared else D + Dv) * per
        kv = n_valid * self.n_kv_heads * row
        qo = self.batch * self.n_q_heads * (D + Dv) * 2
        pt = sum((min(int(L), self.max_pages * PAGE) + PAGE - 1) // PAGE for L in self.seq_lens) * 4
        return int(round(kv)) + qo + pt + 4 * self.batch


# ---- MLA latent rows: already on the e4m3 grid under block-64 power-of-two scales

def _mla_rows(rng: np.random.Generator, n: int) -> np.ndarray:
    lat = rng.standard_normal((n, 8, 64), dtype=np.float32)
    amax = np.abs(lat).max(axis=-1, keepdims=True)
    s64 = np.exp2(np.ceil(np.log2(amax / 448.0))).astype(np.float32)
    g = torch.from_numpy(np.ascontiguousarray(lat / s64)).to(torch.float8_e4m3fn)
    lat = g.to(torch.float32).numpy() * s64          # exact: 4 significant bits x 2^k
    rope = rng.standard_normal((n, 64), dtype=np.float32)
    return np.concatenate([lat.reshape(n, 512), rope], axis=1)


# ---- page tables --------------------------------------------------------------------

def _perm_table(rng, seq_lens, width, num_pages):
    need = [(int(L) + PAGE - 1) // PAGE for L in seq_lens]
    perm = rng.permutation(num_pages).astype(np.int32)
    pt = np.full((len(seq_lens), width), -1, np.int32)
    o = 0
    for b, n in enumerate(need):
        pt[b, :n] = perm[o:o + n]
        o += n
    return pt


def tiny(seed: int = 1) -> Workload:
    L, n_pages = 1024, 64
    pt = np.arange(n_pages, dtype=np.int32)[None]
    return Workload("tiny_b1_ctx1024_h16x8_d128", 1, 16, 8, 128, 128, n_pages,
                    np.array([L], np.int32), pt, seed, kind="channel")


def qwen3(seed: int = 2, batch: int = 8, ctx: int = 16384, replicas: int = 28) -> Workload:
    rng = np.random.Generator(np.random.PCG64([seed, 100]))
    n_pages = batch * ctx // PAGE
    pt = rng.permutation(n_pages).astype(np.int32).reshape(batch, ctx // PAGE)
    return Workload("qwen3_b%d_ctx%d_h16x8_d128" % (batch, ctx), batch, 16, 8, 128, 128,
                    n_pages, np.full(batch, ctx, np.int32), pt, seed, kind="outlier30",
                    layer_replicas=replicas)


def ragged256(seed: int = 3, batch: int = 8, lo: int = 4096, hi: int = 32768) -> Workload:
    rng = np.random.Generator(np.random.PCG64([seed, 100]))
    L = rng.integers(lo, hi + 1, batch).astype(np.int32)
    width = hi // PAGE
    n_pages = int(sum((int(x) + PAGE - 1) // PAGE for x in L))
    pt = _perm_table(rng, L, width, n_pages)
    return Workload("ragged_b%d_ctx%d-%d_h16x2_d256" % (batch, lo, hi), batch, 16, 2, 256, 256,
                    n_pages, L, pt, seed)


def single256(seed: int = 3, ctx: int = 262144) -> Workload:
    rng = np.random.Generator(np.random.PCG64([seed, 101]))
    n_pages = ctx // PAGE
    pt = rng.permutation(n_pages).astype(np.int32)[None]
    return Workload("single_b1_ctx%d_h16x2_d256" % ctx, 1, 16, 2, 256, 256, n_pages,
                    np.array([ctx], np.int32), pt, seed)


def extend(seed: int = 6, batch: int = 8, ctx: int = 16384, new: int = 64) -> Workload:
    """The qwen3 decode shape with the last `new` positions of every sequence
    new: their K/V in the pool, their queries (`extend_queries`) attending
    causally.  new_tokens["q_start"]: int32 [batch + 1]."""
    wl = qwen3(seed=seed, batch=batch, ctx=ctx, replicas=1)
    wl.name = "extend_b%d_ctx%d_new%d_h16x8_d128" % (batch, ctx, new)
    wl.new_tokens = {"q_start": (np.arange(batch + 1) * new).astype(np.int32)}
    return wl


def mla_extend(seed: int = 4, ctx: int = 163840, new: int = 4) -> Workload:
    """The mla slab with its last `new` positions new (extend over the slab)."""
    wl = mla(seed=seed, ctx=ctx)
    wl.name = "mla_extend_b1_ctx%d_new%d_h128x1_d576_dv512" % (ctx, new)
    wl.new_tokens = {"q_start": np.array([0, new], np.int32)}
    return wl


def extend_queries(wl: Workload, n_tokens: int) -> np.ndarray:
    """bf16 bits uint16 [n_tokens, n_q_heads, head_dim_qk]: the new tokens'
    queries, N(0,1), from their own sub-stream."""
    rng = np.random.Generator(np.random.PCG64([wl.seed, 7]))
    return to_bf16_bits(rng.standard_normal((n_tokens, wl.n_q_heads, wl.head_dim_qk),
                                            dtype=np.float32))


def mla(seed: int = 4, ctx: int = 163840, n_q_heads: int = 128) -> Workload:
    rng = np.random.Generator(np.random.PCG64([seed, 100]))
    n_pages = (ctx + PAGE - 1) // PAGE
    pt = rng.permutation(n_pages).astype(np.int32)[None]
    return Workload("mla_b1_ctx%d_h%dx1_d576_dv512" % (ctx, n_q_heads), 1, n_q_heads, 1, 576,
                    512, n_pages, np.array([ctx], np.int32), pt, seed, kind="mla", shared=True)


def mixed(seed: int = 5, batch: int = 64, pool_pages: int = 65536, lo: int = 1024,
          hi: int = 131072, new_per_seq: int = 128, mask_frac: float = 0.01) -> Workload:
    """Mixed store + decode over a shared pool (pages reused across sequences)."""
    rng = np.random.Generator(np.random.PCG64([seed, 100]))
    L = np.floor(np.exp(rng.uniform(np.log(lo), np.log(hi), batch))).astype(np.int64)
    L = np.maximum(L, new_per_seq).astype(np.int32)
    width = hi // PAGE
    pt = np.full((batch, width), -1, np.int32)
    perm = rng.permutation(pool_pages).astype(np.int32)
    # pages holding each sequence's new tail tokens: disjoint across sequences
    tail_first = [(int(x) - new_per_seq) // PAGE for x in L]
    n_tail = [(int(x) + PAGE - 1) // PAGE - f for f, x in zip(tail_first, L)]
    reserved = perm[: sum(n_tail)]
    rest = perm[sum(n_tail):]
    o = 0
    slots = []
    for b in range(batch):
        f, n = tail_first[b], n_tail[b]
        pt[b, f:f + n] = reserved[o:o + n]
        o += n
        older = rng.choice(rest, size=f, replace=False) if f > 0 else np.zeros(0, np.int32)
        if f > 0:
            drop = rng.random(f) < mask_frac
            older = np.where(drop, -1, older)
            pt[b, :f] = older
        t = np.arange(int(L[b]) - new_per_seq, int(L[b]))
        slots.append(pt[b, t // PAGE].astype(np.int64) * PAGE + t % PAGE)
    w = Workload("mixed_b%d_ctx%d-%d_pool%d_h16x8_d128" % (batch, lo, hi, pool_pages * PAGE),
                 batch, 16, 8, 128, 128, pool_pages, L, pt, seed)
    w.new_tokens = {"slots": np.concatenate(slots).astype(np.int32)}
    return w


BY_NAME = {"tiny": tiny, "qwen3": qwen3, "ragged256": ragged256, "single256": single256,
           "mla": mla, "mixed": mixed, "extend": extend}
