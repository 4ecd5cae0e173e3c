"""Plain fp64 attention with a per-head sink logit (test infrastructure only).

Source pages: "GPT-OSS on Day 0" (section "Attention sinks": the sink is an extra
per-head term added before the softmax alongside the Q.K products; the streaming form
keeps a running maximum m and a scale d, seeds m with the head's sink, and includes
that seed only in the first chunk when the KV sequence is split), "Fast Embeddings on
GPUs" (section on ragged and paged attention) and "Accelerating Sonar through
speculation" (verification of several query tokens per sequence).

Readings of points the pages leave open (all stated in the design notes):
  * the sink is in the units of the scaled score (it is not multiplied by the softmax
    scale) and contributes exp(sink) to the denominator with a zero value vector;
  * query head h reads KV head h // (Hq / Hkv);
  * with q_len query tokens and kv_len keys, query token t sits at absolute position
    p = kv_len - q_len + t (the new tokens are the last ones in the cache);
  * causal: key j is visible iff j <= p; window W > 0: also p - j < W (W keys
    including the query's own position);
  * the returned log-sum-exp includes the sink: lse = ln(sum_j e^{s_j} + e^{sink});
  * a row with no visible key returns out = 0 and lse = sink (-inf if the sink is
    disabled).
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

import numpy as np



def _positions(lq: int, lk: int) -> np.ndarray:
    """Absolute positions of lq query tokens that are the last lq of lk tokens."""
    return (lk - lq) + np.arange(lq)


def _visible(q_pos: np.ndarray, lk: int, causal: bool, window: int) -> np.ndarray:
    """Boolean [lq, lk]: key j visible to the query at absolute position q_pos[t]."""
    p = np.asarray(q_pos, dtype=np.int64)[:, None]
    j = np.arange(lk)[None, :]
    lq = p.shape[0]
    vis = np.ones((lq, lk), dtype=bool)
    if causal:
        vis &= j <= p
    if window > 0:
        vis &= (p - j) < window
    return vis


def attention_weights(q: np.ndarray, k: np.ndarray, sink: float, scale: float,
                      causal: bool, window: int,
                      q_pos: Optional[np.ndarray] = None,
                      visible: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Softmax over [scores, sink] for ONE head of ONE sequence.

    q [lq, d], k [lk, d] (fp64). Returns (w [lq, lk], w_sink [lq], lse [lq]) with
    w[t, j] = e^{s_tj - M_t} / D_t for visible keys (0 otherwise), w_sink = e^{sink - M_t} / D_t,
    M_t = max(max_j s_tj, sink), D_t = sum_j e^{s_tj - M_t} + e^{sink - M_t}, lse = M_t + ln D_t.
    ``q_pos`` gives the absolute query positions (default: the last lq of lk positions);
    ``visible`` (bool [lq, lk]), when given, is the mask itself and replaces causal/window.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    lq, lk = q.shape[0], k.shape[0]
    s = scale * (q @ k.T) if lk else np.zeros((lq, 0))
    if visible is not None:
        vis = np.asarray(visible, dtype=bool)
    else:
        vis = _visible(_positions(lq, lk) if q_pos is None else q_pos, lk, causal, window)
    s_vis = np.where(vis, s, -np.inf)
    sink = float(sink)
    row_max = s_vis.max(axis=1) if lk else np.full(lq, -np.inf)
    m = np.maximum(row_max, sink)
    w = np.zeros((lq, lk))
    w_sink = np.zeros(lq)
    lse = np.full(lq, -np.inf)
    live = m > -np.inf                      # rows with at least one visible key or a finite sink
    if live.any():
        ml = m[live][:, None]
        e = np.where(vis[live], np.exp(s_vis[live] - ml), 0.0)
        es = np.exp(sink - m[live]) if sink > -np.inf else np.zeros(int(live.sum()))
        den = e.sum(axis=1) + es
        w[live] = e / den[:, None]
        w_sink[live] = es / den
        lse[live] = m[live] + np.log(den)
    return w, w_sink, lse


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, sinks: np.ndarray, scale: float,
           causal: bool, window: int = 0, heads: Optional[Sequence[int]] = None,
           q_pos: Optional[np.ndarray] = None, visible: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Sink attention for ONE sequence.

    q [lq, hq, d], k/v [lk, hkv, d], sinks [hq] (fp32 or fp64, -inf disables a head's sink).
    ``q_pos``: absolute positions of the query rows (default: the last lq of lk positions).
    Returns out [lq, hq, d] and lse [lq, hq] in fp64 (columns of heads not in ``heads`` are NaN).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    lq, hq, d = q.shape
    hkv = k.shape[1]
    assert hq % hkv == 0, "query heads must be a multiple of KV heads"
    group = hq // hkv
    out = np.full((lq, hq, d), np.nan)
    lse = np.full((lq, hq), np.nan)
    for h in (range(hq) if heads is None else heads):
        g = h // group
        w, _, l = attention_weights(q[:, h, :], k[:, g, :], float(sinks[h]), scale, causal, window, q_pos, visible)
        out[:, h, :] = w @ v[:, g, :] if k.shape[0] else 0.0
        lse[:, h] = l
    return out, lse


def prefill_varlen(q, k, v, cu_seqlens_q, cu_seqlens_kv, sinks, scale, causal, window=0,
                   seqs: Optional[Sequence[int]] = None, rows: Optional[dict] = None):
    """Packed varlen attention: sequence b owns Q rows cu_q[b]:cu_q[b+1] and KV rows
    cu_kv[b]:cu_kv[b+1]. ``seqs`` limits the sequences computed; ``rows[b]`` (optional)
    limits the query tokens of sequence b (local indices). Uncomputed rows are NaN.
    """
    cu_q = np.asarray(cu_seqlens_q, dtype=np.int64)
    cu_k = np.asarray(cu_seqlens_kv, dtype=np.int64)
    total_q, hq, d = q.shape
    out = np.full((total_q, hq, d), np.nan)
    lse = np.full((total_q, hq), np.nan)
    for b in (range(len(cu_q) - 1) if seqs is None else seqs):
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        k0, k1 = int(cu_k[b]), int(cu_k[b + 1])
        qb = np.asarray(q[q0:q1], dtype=np.float64)
        kb = np.asarray(k[k0:k1], dtype=np.float64)
        vb = np.asarray(v[k0:k1], dtype=np.float64)
        if rows is not None and b in rows:
            sel = np.asarray(rows[b], dtype=np.int64)
            pos = _positions(q1 - q0, k1 - k0)[sel]
            o, l = attend(qb[sel], kb, vb, sinks, scale, causal, window, q_pos=pos)
            out[q0 + sel], lse[q0 + sel] = o, l
        else:
            o, l = attend(qb, kb, vb, sinks, scale, causal, window)
            out[q0:q1], lse[q0:q1] = o, l
    return out, lse


def gather_pages(cache: np.ndarray, page_row: np.ndarray, length: int) -> np.ndarray:
    """Contiguous [length, hkv, d] view of one sequence in a paged cache.

    cache [num_pages, hkv, page_size, d]; token j lives in physical page
    page_row[j // page_size], slot j % page_size.
    """
    page_size = cache.shape[2]
    out = np.empty((length, cache.shape[1], cache.shape[3]), dtype=cache.dtype)
    for j in range(0, length, page_size):
        n = min(page_size, length - j)
        out[j:j + n] = np.transpose(cache[int(page_row[j // page_size]), :, :n, :], (1, 0, 2))
    return out


def decode_paged(q, k_cache, v_cache, page_table, kv_lens, sinks, q_len, scale, causal=True, window=0,
                 seqs: Optional[Sequence[int]] = None):
    """Decode / verify against a paged cache. q [batch * q_len, hq, d]; returns out, lse
    (rows of sequences not in ``seqs`` are NaN)."""
    batch = len(kv_lens)
    rows, hq, d = q.shape
    out = np.full((rows, hq, d), np.nan)
    lse = np.full((rows, hq), np.nan)
    for b in (range(batch) if seqs is None else seqs):
        L = int(kv_lens[b])
        kb = gather_pages(k_cache, page_table[b], L)
        vb = gather_pages(v_cache, page_table[b], L)
        o, l = attend(q[b * q_len:(b + 1) * q_len], kb, vb, sinks, scale, causal, window)
        out[b * q_len:(b + 1) * q_len], lse[b * q_len:(b + 1) * q_len] = o, l
    return out, lse


def tree_visible(tree_mask_rows: np.ndarray, q_len: int, lk: int, window: int = 0) -> np.ndarray:
    """Visibility [q_len, lk] of a draft tree verified in one step ("Accelerating Sonar through
    speculation", EAGLE section: tree-shaped drafts need a custom attention mask). The q_len
    draft tokens are the last q_len of lk tokens; row t sees every earlier (prefix) token and
    the draft tokens i whose bit i is set in tree_mask_rows[t]; a window W > 0 also bounds
    every key by position (p - j < W)."""
    p = (lk - q_len) + np.arange(q_len)
    j = np.arange(lk)
    vis = np.zeros((q_len, lk), dtype=bool)
    vis[:, :lk - q_len] = True
    bits = np.asarray(tree_mask_rows, dtype=np.int64)
    for t in range(q_len):
        for i in range(q_len):
            vis[t, lk - q_len + i] = bool((bits[t] >> i) & 1)
    if window > 0:
        vis &= (p[:, None] - j[None, :]) < window
    return vis


def decode_paged_tree(q, k_cache, v_cache, page_table, kv_lens, tree_mask, sinks, q_len, scale, window=0,
                      seqs: Optional[Sequence[int]] = None):
    """Verification of a draft tree against a paged cache. q [batch * q_len, hq, d]; tree_mask
    int [batch * q_len] bitmaps (bit i of row b * q_len + t: draft token i visible to token t).
    Returns out, lse (rows of sequences not in ``seqs`` are NaN)."""
    batch = len(kv_lens)
    rows, hq, d = q.shape
    out = np.full((rows, hq, d), np.nan)
    lse = np.full((rows, hq), np.nan)
    for b in (range(batch) if seqs is None else seqs):
        L = int(kv_lens[b])
        kb = gather_pages(k_cache, page_table[b], L)
        vb = gather_pages(v_cache, page_table[b], L)
        vis = tree_visible(tree_mask[b * q_len:(b + 1) * q_len], q_len, L, window)
        o, l = attend(q[b * q_len:(b + 1) * q_len], kb, vb, sinks, scale, True, window, visible=vis)
        out[b * q_len:(b + 1) * q_len], lse[b * q_len:(b + 1) * q_len] = o, l
    return out, lse

def prefill_paged(q, k_cache, v_cache, page_table, cu_seqlens_q, kv_lens, sinks, scale, causal, window=0,
                  seqs: Optional[Sequence[int]] = None, rows: Optional[dict] = None):
    """Chunked prefill against a paged cache ("Fast Embeddings on GPUs": the LLM path runs
    prefill as well as decode on paged KV). Sequence b owns Q rows cu_q[b]:cu_q[b+1], the
    last Lq_b = cu_q[b+1] - cu_q[b] of its kv_lens[b] tokens, so query token t sits at
    position kv_lens[b] - Lq_b + t; its K/V come through page_table[b]. ``seqs`` limits the
    sequences computed, ``rows[b]`` (optional) the query tokens of sequence b (local
    indices). Uncomputed rows are NaN.
    """
    cu_q = np.asarray(cu_seqlens_q, dtype=np.int64)
    total_q, hq, d = q.shape
    out = np.full((total_q, hq, d), np.nan)
    lse = np.full((total_q, hq), np.nan)
    for b in (range(len(kv_lens)) if seqs is None else seqs):
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        L = int(kv_lens[b])
        kb = gather_pages(k_cache, page_table[b], L).astype(np.float64)
        vb = gather_pages(v_cache, page_table[b], L).astype(np.float64)
        qb = np.asarray(q[q0:q1], dtype=np.float64)
        sel = np.arange(q1 - q0) if rows is None or b not in rows else np.asarray(rows[b], dtype=np.int64)
        o, l = attend(qb[sel], kb, vb, sinks, scale, causal, window, q_pos=_positions(q1 - q0, L)[sel])
        out[q0 + sel], lse[q0 + sel] = o, l
    return out, lse

# ----------------------------------------------------------------------------------
# Streaming form, as the "Attention sinks" section describes it
# ----------------------------------------------------------------------------------
def online_partials(q, k, v, sinks, scale, causal, window, chunk: int, tile: int = 16,
                    sink_chunk: int = 0):
    """Split-KV partials for ONE sequence, each chunk folded in with an online softmax.

    For chunk c covering keys [c*chunk, (c+1)*chunk) the state (m, d, o) per query row and
    head starts at (sink, 1, 0) if c == sink_chunk, else (-inf, 1, 0). Visible keys are
    folded in ``tile`` at a time: m' = max(m, max s); d = d*e^(m-m') + sum e^(s-m');
    o = o*e^(m-m') + sum e^(s-m') v; m = m'. Each chunk emits o/d and m + ln d
    (o = 0, lse = -inf when nothing at all entered the chunk).

    Returns (o_parts [n_chunks, lq, hq, d], lse_parts [n_chunks, lq, hq]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    lq, hq, dim = q.shape
    lk, hkv = k.shape[0], k.shape[1]
    group = hq // hkv
    n_chunks = max(1, -(-lk // chunk))
    vis = _visible(_positions(lq, lk), lk, causal, window)
    o_parts = np.zeros((n_chunks, lq, hq, dim))
    lse_parts = np.full((n_chunks, lq, hq), -np.inf)
    for h in range(hq):
        g = h // group
        s_all = scale * (q[:, h, :] @ k[:, g, :].T)
        for c in range(n_chunks):
            m = np.full(lq, float(sinks[h]) if c == sink_chunk else -np.inf)
            d = np.ones(lq)
            o = np.zeros((lq, dim))
            for j0 in range(c * chunk, min((c + 1) * chunk, lk), tile):
                j1 = min(j0 + tile, (c + 1) * chunk, lk)
                s = np.where(vis[:, j0:j1], s_all[:, j0:j1], -np.inf)
                m_new = np.maximum(m, s.max(axis=1))
                upd = m_new > -np.inf            # rows that have seen something finite
                m_ref = np.where(upd, m_new, 0.0)
                alpha = np.where(upd, np.exp(np.where(upd, m, 0.0) - m_ref), 1.0)
                p = np.where(upd[:, None] & np.isfinite(s), np.exp(s - m_ref[:, None]), 0.0)
                d = d * alpha + p.sum(axis=1)
                o = o * alpha[:, None] + p @ v[j0:j1, g, :]
                m = np.where(upd, m_new, m)
            live = m > -np.inf
            o_parts[c, live, h, :] = o[live] / d[live, None]
            lse_parts[c, live, h] = m[live] + np.log(d[live])
    return o_parts, lse_parts


def merge(o_parts: np.ndarray, lse_parts: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Log-sum-exp merge over axis 0: LSE = ln sum_c e^{lse_c}; out = sum_c e^{lse_c - LSE} o_c.

    Partials with lse = -inf carry weight 0; if all are -inf the result is out = 0, lse = -inf.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    M = lse_parts.max(axis=0)
    live = M > -np.inf
    Ms = np.where(live, M, 0.0)
    w = np.where(lse_parts > -np.inf, np.exp(lse_parts - Ms[None]), 0.0)
    W = w.sum(axis=0)
    Wsafe = np.where(live, W, 1.0)
    out = np.where(live[..., None], (w[..., None] * o_parts).sum(axis=0) / Wsafe[..., None], 0.0)
    lse = np.where(live, Ms + np.log(Wsafe), -np.inf)
    return out, lse


def plan_chunks(kv_lens: Sequence[int], q_len: int, chunk: int) -> Tuple[List[int], List[int]]:
    """Integer split plan, one entry per query row r = b*q_len + t.

    Chunk count n_b = max(1, ceil(L_b / chunk)) (chunk <= 0: one chunk; an empty sequence
    still has chunk 0, which carries the sink); partial_indptr is the exclusive prefix sum
    of the per-row counts (length rows + 1). Plain Python ints.
    """
    counts: List[int] = []
    for L in kv_lens:
        L = int(L)
        n = 1 if chunk <= 0 else max(1, -(-L // chunk))
        counts.extend([n] * q_len)
    indptr = [0]
    for n in counts:
        indptr.append(indptr[-1] + n)
    return counts, indptr


def split_decode(q, k_cache, v_cache, page_table, kv_lens, sinks, q_len, scale, chunk, causal=True,
                 window=0, seqs: Optional[Sequence[int]] = None):
    """Split-KV partials of a paged decode/verify batch in the plan's compact layout.

    Returns (o_parts [n_partials, hq, d], lse_parts [n_partials, hq], counts, indptr); partial
    indptr[r] + c holds chunk c of query row r (rows of skipped sequences stay NaN).
    """
    counts, indptr = plan_chunks(kv_lens, q_len, chunk)
    hq, d = q.shape[1], q.shape[2]
    o_all = np.full((indptr[-1], hq, d), np.nan)
    l_all = np.full((indptr[-1], hq), np.nan)
    for b in (range(len(kv_lens)) if seqs is None else seqs):
        L = int(kv_lens[b])
        kb = gather_pages(k_cache, page_table[b], L)
        vb = gather_pages(v_cache, page_table[b], L)
        c_eff = chunk if chunk > 0 else max(L, 1)
        o, l = online_partials(q[b * q_len:(b + 1) * q_len], kb, vb, sinks, scale, causal, window, c_eff)
        for t in range(q_len):
            r = b * q_len + t
            o_all[indptr[r]:indptr[r + 1]] = o[:, t]
            l_all[indptr[r]:indptr[r + 1]] = l[:, t]
    return o_all, l_all, counts, indptr
