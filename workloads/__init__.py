"""Seeded synthetic inputs for sink attention.

This module only draws and packs inputs: lengths, page permutations, bf16 Q/K/V bit
patterns and fp32 sink vectors. It contains none of the attention arithmetic, so both
the CPU oracle and the GPU path can consume the same inputs without sharing any of
the method's code.

Shapes and distributions follow the workloads of the source pages: GPT-OSS-style GQA
decode and prefill ("GPT-OSS on Day 0", section "Attention sinks"), the ragged
embedding batches of "Fast Embeddings on GPUs" (section on ragged attention), and
multi-token verification of "Accelerating Sonar through speculation" (MTP section).

Recipe (fixed, documented in the design notes):
  * ``numpy.random.default_rng(seed)``; draw order: lengths -> page permutation ->
    Q -> K -> V -> sinks (chunked prefill draws chunk lengths, then cached lengths).
  * Q/K/V are fp32 N(0, 1) rounded to bf16 with round-to-nearest-even.
  * Sinks are fp32 ``sink_std * N(0, 1)``; ``sink_std=None`` means the sink is
    disabled (-inf for every head).
  * Uniform integer lengths are inclusive: ``rng.integers(lo, hi + 1)``.
  * The paged KV pool holds exactly the pages the batch needs, in a seeded random
    physical order; page-table entries past a sequence's last page are 0 and are
    never dereferenced.
  * KV cache layout is [num_pages, num_kv_heads, page_size, head_dim] ("HND").
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np

__all__ = [
    "VarlenSpec", "PagedSpec", "PagedPrefillSpec", "CONFIGS", "bf16_round_bits", "bf16_bits_to_f32",
    "make_varlen", "make_paged", "make_paged_prefill", "make_tree_masks", "scaled",
]


# ---------------------------------------------------------------------------------
# bf16 bit handling (representation only)
# ---------------------------------------------------------------------------------
def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 with round-to-nearest-even; return uint16 bit patterns.

    Inputs here are finite normals, so NaN handling is not needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return bf16_round_bits(x)


def _sinks(rng: np.random.Generator, hq: int, std: Optional[float]) -> np.ndarray:
    if std is None:
        return np.full(hq, -np.inf, dtype=np.float32)
    return (np.float32(std) * rng.standard_normal(size=hq, dtype=np.float32)).astype(np.float32)


# ---------------------------------------------------------------------------------
# Workload descriptions
# ---------------------------------------------------------------------------------
@dataclass(frozen=True)
class VarlenSpec:
    """Packed variable-length self-attention (prefill / embedding), no KV cache."""
    name: str
    batch: int
    seqlen: Tuple[int, int]          # inclusive uniform range; (n, n) for fixed length
    hq: int
    hkv: int
    head_dim: int = 64
    causal: bool = True
    window: int = 0                  # <= 0: no window; else W keys including self
    sink_std: Optional[float] = 1.0  # None: sinks disabled (-inf)
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))


@dataclass(frozen=True)
class PagedSpec:
    """Decode / verify against a paged KV cache (q_len new tokens per sequence)."""
    name: str
    batch: int
    q_len: int
    kv_len: Tuple[int, int]          # inclusive uniform range; includes the q_len new tokens
    hq: int
    hkv: int
    head_dim: int = 64
    page_size: int = 16
    kv_chunk: int = 512
    causal: bool = True
    window: int = 0
    sink_std: Optional[float] = 2.0
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))


@dataclass(frozen=True)
class PagedPrefillSpec:
    """Chunked prefill against a paged KV cache: every sequence appends a chunk of new tokens
    (its queries) to a cache that already holds ctx_len tokens; kv_len = ctx_len + q_len."""
    name: str
    batch: int
    q_len: Tuple[int, int]           # inclusive uniform range of the chunk length
    ctx_len: Tuple[int, int]         # inclusive uniform range of the tokens already cached
    hq: int
    hkv: int
    head_dim: int = 64
    page_size: int = 16
    causal: bool = True
    window: int = 0
    sink_std: Optional[float] = 2.0
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))


CONFIGS = {
    # Tiny causal GQA 4:1, single sequence of 16 tokens, single KV chunk.
    "tiny_causal": VarlenSpec("tiny_causal", batch=1, seqlen=(16, 16), hq=4, hkv=1,
                              causal=True, sink_std=1.0, seed=0),
    # Paged single-token decode, 64 sequences, KV 1024..8192, 64/8 heads, 512-token chunks.
    "paged_decode": PagedSpec("paged_decode", batch=64, q_len=1, kv_len=(1024, 8192), hq=64, hkv=8,
                              page_size=16, kv_chunk=512, sink_std=2.0, seed=1),
    # Causal prefill 8 x 4096 packed; the same inputs also run with a 128-key window.
    "causal_prefill": VarlenSpec("causal_prefill", batch=8, seqlen=(4096, 4096), hq=64, hkv=8,
                                 causal=True, window=0, sink_std=2.0, seed=2),
    "window_prefill": VarlenSpec("window_prefill", batch=8, seqlen=(4096, 4096), hq=64, hkv=8,
                                 causal=True, window=128, sink_std=2.0, seed=2),
    # Speculative verify: 5 query tokens per sequence, causal inside the block. The chunk length
    # is an implementation choice here (the workload fixes none): 2048-token chunks keep the
    # partials (5 rows x 64 heads per chunk) and their merge small next to the KV stream.
    "verify": PagedSpec("verify", batch=32, q_len=5, kv_len=(2048, 16384), hq=64, hkv=8,
                        page_size=16, kv_chunk=2048, sink_std=2.0, seed=3),
    # Bidirectional MHA embedding batch; pass A with sinks disabled, pass B with N(0,1) sinks.
    "embed_nosink": VarlenSpec("embed_nosink", batch=512, seqlen=(16, 512), hq=16, hkv=16,
                               causal=False, sink_std=None, seed=4),
    "embed_sink": VarlenSpec("embed_sink", batch=512, seqlen=(16, 512), hq=16, hkv=16,
                             causal=False, sink_std=1.0, seed=4),
    # Chunked prefill on the paged cache (the LLM prefill path of "Fast Embeddings on GPUs"):
    # 8 sequences each append a 2048-token chunk to 0..6144 cached tokens; 64/8 heads as
    # the prefill workload, 16-token pages.
    # Verification of an 8-node draft tree per sequence (EAGLE-style drafts of "Accelerating Sonar
    # through speculation"), on the verify workload's cache shape; one random tree per sequence.
    "tree_verify": PagedSpec("tree_verify", batch=32, q_len=8, kv_len=(2048, 16384), hq=64, hkv=8,
                             page_size=16, kv_chunk=2048, sink_std=2.0, seed=6),
    "chunked_prefill": PagedPrefillSpec("chunked_prefill", batch=8, q_len=(2048, 2048), ctx_len=(0, 6144),
                                        hq=64, hkv=8, page_size=16, sink_std=2.0, seed=5),
    # One GPU's share of the decode and causal prefill workloads under 4-way head sharding
    # (tensor parallel): each GPU holds 2 of the 8 KV heads and their 16 query heads, with the
    # same sequences, lengths, pages and chunking.
    "paged_decode_tp4": PagedSpec("paged_decode_tp4", batch=64, q_len=1, kv_len=(1024, 8192), hq=16, hkv=2,
                                  page_size=16, kv_chunk=512, sink_std=2.0, seed=1),
    "causal_prefill_tp4": VarlenSpec("causal_prefill_tp4", batch=8, seqlen=(4096, 4096), hq=16, hkv=2,
                                     causal=True, window=0, sink_std=2.0, seed=2),
}


def scaled(spec, **changes):
    """A copy of ``spec`` with some fields replaced (smaller parity-test variants)."""
    return dataclasses.replace(spec, **changes)


# ---------------------------------------------------------------------------------
# Generators
# ---------------------------------------------------------------------------------
def _draw_lengths(rng: np.random.Generator, batch: int, lo_hi: Tuple[int, int]) -> np.ndarray:
    lo, hi = lo_hi
    if lo == hi:
        return np.full(batch, lo, dtype=np.int32)
    return rng.integers(lo, hi + 1, size=batch).astype(np.int32)


def make_varlen(spec: VarlenSpec, seqlens: Optional[np.ndarray] = None) -> dict:
    """Inputs for packed varlen attention.

    Returns q [T, hq, d], k/v [T, hkv, d] as uint16 bf16 bits, sinks fp32 [hq],
    cu_seqlens int32 [batch + 1] (the same array serves Q and KV) and max_seqlen.
    ``seqlens`` overrides the drawn lengths (edge-case tests); the draw order of the
    remaining tensors is unchanged.
    """
    rng = np.random.default_rng(spec.seed)
    lens = _draw_lengths(rng, spec.batch, spec.seqlen)
    if seqlens is not None:
        lens = np.asarray(seqlens, dtype=np.int32)
    cu = np.zeros(len(lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens, dtype=np.int64).astype(np.int32)
    total = int(cu[-1])
    q = _normal_bf16(rng, (total, spec.hq, spec.head_dim))
    k = _normal_bf16(rng, (total, spec.hkv, spec.head_dim))
    v = _normal_bf16(rng, (total, spec.hkv, spec.head_dim))
    sinks = _sinks(rng, spec.hq, spec.sink_std)
    return dict(q=q, k=k, v=v, sinks=sinks, cu_seqlens=cu, seqlens=lens,
                max_seqlen=int(lens.max()) if len(lens) else 0)


def make_paged(spec: PagedSpec, kv_lens: Optional[np.ndarray] = None,
               max_pages_per_seq: Optional[int] = None) -> dict:
    """Inputs for paged decode / verify.

    Returns q [batch * q_len, hq, d] bits, k_cache / v_cache [num_pages, hkv, page, d]
    bits, page_table int32 [batch, max_pages_per_seq], kv_lens int32 [batch] and sinks
    fp32 [hq]. Row ``b * q_len + t`` of q is query token t of sequence b; its absolute
    position is ``kv_lens[b] - q_len + t``.
    """
    rng = np.random.default_rng(spec.seed)
    lens = _draw_lengths(rng, spec.batch, spec.kv_len)
    if kv_lens is not None:
        lens = np.asarray(kv_lens, dtype=np.int32)
    P = spec.page_size
    npages_b = (lens.astype(np.int64) + P - 1) // P
    num_pages = int(npages_b.sum())
    perm = rng.permutation(num_pages).astype(np.int32)
    if max_pages_per_seq is None:
        max_pages_per_seq = max(1, -(-max(spec.kv_len[1], int(lens.max()) if len(lens) else 0) // P))
    table = np.zeros((len(lens), max_pages_per_seq), dtype=np.int32)
    off = 0
    for b, n in enumerate(npages_b):
        table[b, :n] = perm[off:off + n]
        off += int(n)
    q = _normal_bf16(rng, (len(lens) * spec.q_len, spec.hq, spec.head_dim))
    pool = max(num_pages, 1)
    k_cache = _normal_bf16(rng, (pool, spec.hkv, P, spec.head_dim))
    v_cache = _normal_bf16(rng, (pool, spec.hkv, P, spec.head_dim))
    sinks = _sinks(rng, spec.hq, spec.sink_std)
    return dict(q=q, k_cache=k_cache, v_cache=v_cache, page_table=table, kv_lens=lens.astype(np.int32),
                sinks=sinks, num_pages=pool, max_kv_len=int(lens.max()) if len(lens) else 0)


def make_paged_prefill(spec: PagedPrefillSpec, q_lens: Optional[np.ndarray] = None,
                       ctx_lens: Optional[np.ndarray] = None, max_pages_per_seq: Optional[int] = None) -> dict:
    """Inputs for chunked prefill against a paged cache.

    Returns q [T, hq, d] bits with cu_seqlens_q int32 [batch + 1] (sequence b owns rows
    cu[b]:cu[b+1], its q_lens[b] newest tokens), kv_lens int32 [batch] (= ctx + q_len),
    k_cache / v_cache [num_pages, hkv, page, d] bits, page_table int32
    [batch, max_pages_per_seq] and sinks fp32 [hq]. Draw order: chunk lengths -> cached
    lengths -> page permutation -> Q -> K -> V -> sinks. ``q_lens`` / ``ctx_lens`` override
    the drawn lengths (edge-case tests).
    """
    rng = np.random.default_rng(spec.seed)
    ql = _draw_lengths(rng, spec.batch, spec.q_len)
    cl = _draw_lengths(rng, spec.batch, spec.ctx_len)
    if q_lens is not None:
        ql = np.asarray(q_lens, dtype=np.int32)
    if ctx_lens is not None:
        cl = np.asarray(ctx_lens, dtype=np.int32)
    lens = (ql.astype(np.int64) + cl).astype(np.int32)
    P = spec.page_size
    npages_b = (lens.astype(np.int64) + P - 1) // P
    num_pages = int(npages_b.sum())
    perm = rng.permutation(num_pages).astype(np.int32)
    if max_pages_per_seq is None:
        cap = spec.q_len[1] + spec.ctx_len[1]
        max_pages_per_seq = max(1, -(-max(cap, int(lens.max()) if len(lens) else 0) // P))
    table = np.zeros((len(lens), max_pages_per_seq), dtype=np.int32)
    off = 0
    for b, n in enumerate(npages_b):
        table[b, :n] = perm[off:off + n]
        off += int(n)
    cu = np.zeros(len(ql) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(ql, dtype=np.int64).astype(np.int32)
    q = _normal_bf16(rng, (int(cu[-1]), spec.hq, spec.head_dim))
    pool = max(num_pages, 1)
    k_cache = _normal_bf16(rng, (pool, spec.hkv, P, spec.head_dim))
    v_cache = _normal_bf16(rng, (pool, spec.hkv, P, spec.head_dim))
    sinks = _sinks(rng, spec.hq, spec.sink_std)
    return dict(q=q, cu_seqlens_q=cu, q_lens=ql, kv_lens=lens, k_cache=k_cache, v_cache=v_cache,
                page_table=table, sinks=sinks, num_pages=pool,
                max_q=int(ql.max()) if len(ql) else 0, max_kv_len=int(lens.max()) if len(lens) else 0)


def make_tree_masks(spec: PagedSpec, batch: Optional[int] = None) -> np.ndarray:
    """Random draft trees, one per sequence, as int32 bitmaps [batch * q_len]: node 0 is the
    root, node i > 0 hangs under a parent drawn uniformly from nodes 0..i-1, and row i has the
    bits of node i and of all its ancestors. Drawn from ``default_rng([seed, 1])``, a stream
    apart from the paged inputs'."""
    rng = np.random.default_rng([spec.seed, 1])
    n = spec.batch if batch is None else batch
    out = np.zeros(n * spec.q_len, dtype=np.int32)
    for b in range(n):
        for i in range(spec.q_len):
            parent = int(rng.integers(0, i)) if i > 0 else -1
            out[b * spec.q_len + i] = (1 << i) | (out[b * spec.q_len + parent] if parent >= 0 else 0)
    return out
