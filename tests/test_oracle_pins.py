"""Pins for the fp64 oracle, each independent of the oracle's own formulas.

The method ("GPT-OSS on Day 0", section "Attention sinks") adds a per-head sink logit to
the softmax over the scaled Q.K scores; the streaming form seeds the running max with the
sink in the first KV chunk only. The pages print no worked example, so the oracle is
pinned by: library attention with the sink disabled, closed forms, invariants, a 50-digit
brute force on tiny inputs and hand-derived cases (tests/golden/hand_derived.json).
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import mpmath

import oracle
from workloads import (CONFIGS, bf16_bits_to_f32, make_paged, make_paged_prefill, make_tree_masks, make_varlen,
                       scaled)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_derived.json")


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _sdpa_plain(q, k, v, scale, causal, window, q_pos=None):
    """Ordinary attention (no sink) from torch's library routine, fp64 on the CPU.

    q [lq, hq, d], k/v [lk, hkv, d] -> out [lq, hq, d], lse [lq, hq]. GQA by repeating each KV
    head over its consecutive group of query heads; masks built explicitly.
    """
    lq, hq, d = q.shape
    lk, hkv = k.shape[0], k.shape[1]
    G = hq // hkv
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))             # [hq, lq, d]
    kt = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2))).repeat_interleave(G, 0)
    vt = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2))).repeat_interleave(G, 0)
    pos = torch.arange(lk - lq, lk) if q_pos is None else torch.as_tensor(q_pos)
    j = torch.arange(lk)
    mask = torch.ones(lq, lk, dtype=torch.bool)
    if causal:
        mask &= j[None, :] <= pos[:, None]
    if window > 0:
        mask &= (pos[:, None] - j[None, :]) < window
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    scores = (qt @ kt.transpose(1, 2)) * scale
    lse = torch.logsumexp(scores.masked_fill(~mask, float("-inf")), dim=-1)
    return out.permute(1, 0, 2).numpy(), lse.T.numpy()


# ---------------------------------------------------------------------------------------
# c-P1: sink disabled reduces to ordinary attention (torch SDPA, fp64)
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("lq,lk,hq,hkv,causal,window", [
    (16, 16, 4, 1, True, 0), (1, 37, 8, 2, True, 0), (5, 40, 8, 8, True, 0),
    (13, 13, 6, 3, False, 0), (24, 24, 4, 2, True, 7), (3, 50, 4, 4, True, 16),
])
def test_no_sink_equals_library_attention(lq, lk, hq, hkv, causal, window):
    rng = np.random.default_rng(100 + lq + lk)
    q, k, v = _rand(rng, lq, hq, 64), _rand(rng, lk, hkv, 64), _rand(rng, lk, hkv, 64)
    sinks = np.full(hq, -np.inf)
    out, lse = oracle.attend(q, k, v, sinks, 0.125, causal, window)
    ref_o, ref_l = _sdpa_plain(q, k, v, 0.125, causal, window)
    np.testing.assert_allclose(out, ref_o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_l, rtol=0, atol=1e-12)


def test_no_sink_equals_textbook_softmax():
    """Second library route: scipy's softmax over explicitly masked rows."""
    from scipy.special import softmax
    rng = np.random.default_rng(7)
    q, k, v = _rand(rng, 9, 2, 16), _rand(rng, 9, 2, 16), _rand(rng, 9, 2, 16)
    out, _ = oracle.attend(q, k, v, np.full(2, -np.inf), 0.25, True, 0)
    for h in range(2):
        s = 0.25 * q[:, h] @ k[:, h].T
        s[np.triu_indices(9, 1)] = -np.inf
        np.testing.assert_allclose(out[:, h], softmax(s, axis=1) @ v[:, h], atol=1e-13, rtol=0)


# ---------------------------------------------------------------------------------------
# c-P2: single key closed form
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("sink", [-3.0, 0.0, 0.7, 4.0])
def test_single_key_closed_form(sink):
    rng = np.random.default_rng(11)
    q, k, v = _rand(rng, 1, 1, 64), _rand(rng, 1, 1, 64), _rand(rng, 1, 1, 64)
    scale = 0.125
    s = scale * math.fsum(float(a) * float(b) for a, b in zip(q[0, 0], k[0, 0]))
    out, lse = oracle.attend(q, k, v, np.array([sink]), scale, True, 0)
    expect = v[0, 0] * (math.exp(s) / (math.exp(s) + math.exp(sink)))
    np.testing.assert_allclose(out[0, 0], expect, rtol=1e-14, atol=1e-15)
    assert abs(lse[0, 0] - math.log(math.exp(s) + math.exp(sink))) < 1e-14 * max(1.0, abs(lse[0, 0]))


# ---------------------------------------------------------------------------------------
# c-P3: attention weights plus the sink weight sum to one
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("causal,window", [(True, 0), (False, 0), (True, 5)])
def test_weights_and_sink_weight_sum_to_one(causal, window):
    rng = np.random.default_rng(3)
    for lq, lk in [(1, 1), (4, 19), (12, 12)]:
        q, k = _rand(rng, lq, 32), _rand(rng, lk, 32)
        for sink in (-np.inf, -2.0, 0.0, 3.5):
            w, ws, _ = oracle.attention_weights(q, k, sink, 0.3, causal, window)
            assert np.all(w >= 0) and np.all(ws >= 0)
            np.testing.assert_allclose(w.sum(axis=1) + ws, 1.0, atol=1e-12, rtol=0)
            if sink > -np.inf:
                assert np.all(ws > 0)


# ---------------------------------------------------------------------------------------
# c-P4: chunk count invariance; the sink may sit in any single chunk
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("chunk", [1, 3, 16, 512, 45])
def test_split_merge_equals_direct(chunk):
    rng = np.random.default_rng(21)
    lq, lk, hq, hkv = 3, 45, 4, 2
    q, k, v = _rand(rng, lq, hq, 64), _rand(rng, lk, hkv, 64), _rand(rng, lk, hkv, 64)
    sinks = 2.0 * rng.standard_normal(hq)
    out, lse = oracle.attend(q, k, v, sinks, 0.125, True, 0)
    o_p, l_p = oracle.online_partials(q, k, v, sinks, 0.125, True, 0, chunk, tile=4)
    mo, ml = oracle.merge(o_p, l_p)
    np.testing.assert_allclose(mo, out, atol=1e-12, rtol=0)
    np.testing.assert_allclose(ml, lse, atol=1e-12, rtol=0)


def test_sink_in_any_single_chunk():
    rng = np.random.default_rng(22)
    lq, lk, hq, hkv = 2, 40, 2, 1
    q, k, v = _rand(rng, lq, hq, 16), _rand(rng, lk, hkv, 16), _rand(rng, lk, hkv, 16)
    sinks = np.array([1.5, -0.5])
    out, lse = oracle.attend(q, k, v, sinks, 0.25, True, 6)
    for sc in range(4):
        o_p, l_p = oracle.online_partials(q, k, v, sinks, 0.25, True, 6, 10, tile=3, sink_chunk=sc)
        mo, ml = oracle.merge(o_p, l_p)
        np.testing.assert_allclose(mo, out, atol=1e-12, rtol=0)
        np.testing.assert_allclose(ml, lse, atol=1e-12, rtol=0)


def test_sink_in_every_chunk_is_wrong():
    """Seeding every chunk with the sink counts it once per chunk: the merge must differ."""
    rng = np.random.default_rng(23)
    q, k, v = _rand(rng, 1, 1, 16), _rand(rng, 32, 1, 16), _rand(rng, 32, 1, 16)
    sinks = np.array([3.0])
    out, _ = oracle.attend(q, k, v, sinks, 0.25, True, 0)
    parts = [oracle.online_partials(q, k, v, sinks, 0.25, True, 0, 8, sink_chunk=c) for c in range(4)]
    o_bad = np.stack([p[0][c] for c, p in enumerate(parts)])
    l_bad = np.stack([p[1][c] for c, p in enumerate(parts)])
    mo, _ = oracle.merge(o_bad, l_bad)
    assert np.abs(mo - out).max() > 1e-3


def test_merge_edge_cases():
    o = np.ones((3, 2, 4))
    l = np.full((3, 2), -np.inf)
    mo, ml = oracle.merge(o, l)
    assert np.all(mo == 0) and np.all(ml == -np.inf)
    l[1, 0] = 0.3                          # a single live partial passes through unchanged
    mo, ml = oracle.merge(o * np.arange(3)[:, None, None], l)
    np.testing.assert_allclose(mo[0], 1.0)
    assert ml[0] == 0.3 and ml[1] == -np.inf and np.all(mo[1] == 0)


# ---------------------------------------------------------------------------------------
# c-P5: brute force, 50 digits, explicit loops
# ---------------------------------------------------------------------------------------
def _brute(q, k, v, sinks, scale, causal, window):
    mpmath.mp.dps = 50
    lq, hq, d = q.shape
    lk, hkv = k.shape[0], k.shape[1]
    G = hq // hkv
    out = np.zeros((lq, hq, d))
    lse = np.zeros((lq, hq))
    for t in range(lq):
        p = lk - lq + t
        for h in range(hq):
            g = h // G
            terms = []
            for j in range(lk):
                if causal and j > p:
                    continue
                if window > 0 and p - j >= window:
                    continue
                s = mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(float(q[t, h, e])) * mpmath.mpf(float(k[j, g, e]))
                                                    for e in range(d))
                terms.append((mpmath.exp(s), j))
            den = mpmath.fsum(x for x, _ in terms)
            if sinks[h] > -np.inf:
                den += mpmath.exp(mpmath.mpf(float(sinks[h])))
            for e in range(d):
                out[t, h, e] = float(mpmath.fsum(x * mpmath.mpf(float(v[j, g, e])) for x, j in terms) / den)
            lse[t, h] = float(mpmath.log(den))
    return out, lse


@pytest.mark.parametrize("lq,lk,hq,hkv,causal,window", [
    (1, 1, 1, 1, True, 0), (2, 8, 4, 2, True, 0), (4, 4, 4, 1, True, 2), (3, 7, 2, 2, False, 0), (5, 8, 4, 4, True, 3),
])
def test_brute_force_50_digits(lq, lk, hq, hkv, causal, window):
    rng = np.random.default_rng(lq * 31 + lk)
    q, k, v = _rand(rng, lq, hq, 8), _rand(rng, lk, hkv, 8), _rand(rng, lk, hkv, 8)
    sinks = rng.standard_normal(hq) * 2
    sinks[0] = -np.inf if hq > 1 else sinks[0]
    out, lse = oracle.attend(q, k, v, sinks, 0.35, causal, window)
    bo, bl = _brute(q, k, v, sinks, 0.35, causal, window)
    np.testing.assert_allclose(out, bo, atol=1e-13, rtol=0)
    np.testing.assert_allclose(lse, bl, atol=1e-13, rtol=0)


# ---------------------------------------------------------------------------------------
# c-P6: sigmoid identity against the library
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["tiny_causal", "paged_decode", "causal_prefill", "window_prefill", "verify",
                                  "embed_sink"])
def test_sigmoid_identity(name):
    spec = CONFIGS[name]
    rng = np.random.default_rng(5)
    lq = 1 if name == "paged_decode" else (5 if name == "verify" else 24)
    lk = 60 if name in ("paged_decode", "verify") else lq
    hq, hkv = min(spec.hq, 16), min(spec.hkv, 16 if spec.hq == spec.hkv else 2)
    q, k, v = _rand(rng, lq, hq, 64), _rand(rng, lk, hkv, 64), _rand(rng, lk, hkv, 64)
    sinks = 2.0 * rng.standard_normal(hq)
    out, lse = oracle.attend(q, k, v, sinks, spec.scale, spec.causal, spec.window if spec.window <= 8 else 8)
    po, pl = _sdpa_plain(q, k, v, spec.scale, spec.causal, spec.window if spec.window <= 8 else 8)
    sig = 1.0 / (1.0 + np.exp(sinks[None, :] - pl))
    np.testing.assert_allclose(out, po * sig[..., None], atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse, np.logaddexp(pl, sinks[None, :]), atol=1e-12, rtol=0)


# ---------------------------------------------------------------------------------------
# c-P7: GQA equals MHA with repeated KV heads
# ---------------------------------------------------------------------------------------
def test_gqa_equals_repeated_mha():
    rng = np.random.default_rng(8)
    q, k, v = _rand(rng, 6, 8, 64), _rand(rng, 20, 2, 64), _rand(rng, 20, 2, 64)
    sinks = rng.standard_normal(8)
    a = oracle.attend(q, k, v, sinks, 0.125, True, 0)
    b = oracle.attend(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), sinks, 0.125, True, 0)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ---------------------------------------------------------------------------------------
# c-P8: paged gather equals contiguous; page-pool permutation changes nothing
# ---------------------------------------------------------------------------------------
def test_paged_equals_contiguous_and_permutation_invariant():
    spec = scaled(CONFIGS["verify"], batch=3, kv_len=(20, 70), hq=8, hkv=2, seed=9)
    inp = make_paged(spec)
    f = lambda x: bf16_bits_to_f32(x).astype(np.float64)
    q, kc, vc = f(inp["q"]), f(inp["k_cache"]), f(inp["v_cache"])
    out, lse = oracle.decode_paged(q, kc, vc, inp["page_table"], inp["kv_lens"], inp["sinks"], spec.q_len,
                                   spec.scale, True, 0)
    P = spec.page_size
    for b, L in enumerate(inp["kv_lens"]):
        # contiguous copy built with a different route: a flat token index into the pool
        tok = np.arange(L)
        phys = inp["page_table"][b][tok // P]
        kb = kc[phys, :, tok % P, :]
        vb = vc[phys, :, tok % P, :]
        o2, l2 = oracle.attend(q[b * 5:(b + 1) * 5], kb, vb, inp["sinks"], spec.scale, True, 0)
        assert np.array_equal(out[b * 5:(b + 1) * 5], o2) and np.array_equal(lse[b * 5:(b + 1) * 5], l2)
    perm = np.random.default_rng(1).permutation(inp["num_pages"])
    inv = np.argsort(perm)
    kc2, vc2 = kc[inv], vc[inv]                       # page p moves to slot perm[p]
    table2 = perm[inp["page_table"]]
    out2, lse2 = oracle.decode_paged(q, kc2, vc2, table2, inp["kv_lens"], inp["sinks"], spec.q_len,
                                     spec.scale, True, 0)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


# ---------------------------------------------------------------------------------------
# c-P8b: chunked prefill on a paged cache, pinned by routes that do not use its gather
# ---------------------------------------------------------------------------------------
def _flat_gather(cache, table_row, L):
    """Contiguous [L, hkv, d] copy through a flat token index (not oracle.gather_pages)."""
    tok = np.arange(L)
    P = cache.shape[2]
    return cache[table_row[tok // P], :, tok % P, :]


def _f64(x):
    return bf16_bits_to_f32(x).astype(np.float64)


def test_paged_prefill_without_context_equals_varlen():
    spec = scaled(CONFIGS["chunked_prefill"], batch=3, q_len=(17, 70), ctx_len=(0, 0), hq=8, hkv=2, seed=21)
    inp = make_paged_prefill(spec)
    q, kc, vc = _f64(inp["q"]), _f64(inp["k_cache"]), _f64(inp["v_cache"])
    cu = inp["cu_seqlens_q"]
    k = np.concatenate([_flat_gather(kc, inp["page_table"][b], L) for b, L in enumerate(inp["kv_lens"])])
    v = np.concatenate([_flat_gather(vc, inp["page_table"][b], L) for b, L in enumerate(inp["kv_lens"])])
    for causal, window in [(True, 0), (True, 9), (False, 0)]:
        a = oracle.prefill_paged(q, kc, vc, inp["page_table"], cu, inp["kv_lens"], inp["sinks"], spec.scale,
                                 causal, window)
        b = oracle.prefill_varlen(q, k, v, cu, cu, inp["sinks"], spec.scale, causal, window)
        np.testing.assert_allclose(a[0], b[0], atol=1e-13, rtol=0)
        np.testing.assert_allclose(a[1], b[1], atol=1e-13, rtol=0)


def test_paged_prefill_chunk_is_the_tail_of_a_full_prefill():
    # The chunk's rows are the last rows of a causal prefill over context + chunk: that pins
    # the alignment of the queries to the newest positions.
    spec = scaled(CONFIGS["chunked_prefill"], batch=2, q_len=(5, 40), ctx_len=(3, 60), hq=4, hkv=1, seed=22)
    inp = make_paged_prefill(spec)
    q, kc, vc = _f64(inp["q"]), _f64(inp["k_cache"]), _f64(inp["v_cache"])
    rng = np.random.default_rng(3)
    for window in (0, 7):
        out, lse = oracle.prefill_paged(q, kc, vc, inp["page_table"], inp["cu_seqlens_q"], inp["kv_lens"],
                                        inp["sinks"], spec.scale, True, window)
        for b, L in enumerate(inp["kv_lens"]):
            q0, q1 = int(inp["cu_seqlens_q"][b]), int(inp["cu_seqlens_q"][b + 1])
            ctx_q = rng.standard_normal((L - (q1 - q0), spec.hq, 64))
            full_q = np.concatenate([ctx_q, q[q0:q1]])
            k, v = _flat_gather(kc, inp["page_table"][b], L), _flat_gather(vc, inp["page_table"][b], L)
            fo, fl = _sdpa_plain(full_q, k, v, spec.scale, True, window)
            sig = 1.0 / (1.0 + np.exp(inp["sinks"][None, :].astype(np.float64) - fl))
            np.testing.assert_allclose(out[q0:q1], (fo * sig[..., None])[L - (q1 - q0):], atol=1e-12, rtol=0)
            np.testing.assert_allclose(lse[q0:q1], np.logaddexp(fl, inp["sinks"][None, :])[L - (q1 - q0):],
                                       atol=1e-12, rtol=0)


def test_paged_prefill_brute_force_50_digits():
    spec = scaled(CONFIGS["chunked_prefill"], batch=2, q_len=(2, 3), ctx_len=(1, 4), hq=2, hkv=1, page_size=2,
                  seed=23)
    inp = make_paged_prefill(spec)
    q, kc, vc = _f64(inp["q"])[..., :8], _f64(inp["k_cache"])[..., :8], _f64(inp["v_cache"])[..., :8]
    out, lse = oracle.prefill_paged(q, kc, vc, inp["page_table"], inp["cu_seqlens_q"], inp["kv_lens"],
                                    inp["sinks"], 0.35, True, 0)
    for b, L in enumerate(inp["kv_lens"]):
        q0, q1 = int(inp["cu_seqlens_q"][b]), int(inp["cu_seqlens_q"][b + 1])
        bo, bl = _brute(q[q0:q1], _flat_gather(kc, inp["page_table"][b], L), _flat_gather(vc, inp["page_table"][b], L),
                        inp["sinks"], 0.35, True, 0)
        np.testing.assert_allclose(out[q0:q1], bo, atol=1e-13, rtol=0)
        np.testing.assert_allclose(lse[q0:q1], bl, atol=1e-13, rtol=0)


def test_paged_prefill_uniform_chunks_equal_decode_paged():
    spec = scaled(CONFIGS["chunked_prefill"], batch=3, q_len=(5, 5), ctx_len=(10, 50), hq=8, hkv=2, seed=24)
    inp = make_paged_prefill(spec)
    q, kc, vc = _f64(inp["q"]), _f64(inp["k_cache"]), _f64(inp["v_cache"])
    a = oracle.prefill_paged(q, kc, vc, inp["page_table"], inp["cu_seqlens_q"], inp["kv_lens"], inp["sinks"],
                             spec.scale, True, 0)
    b = oracle.decode_paged(q, kc, vc, inp["page_table"], inp["kv_lens"], inp["sinks"], 5, spec.scale, True, 0)
    np.testing.assert_allclose(a[0], b[0], atol=1e-13, rtol=0)
    np.testing.assert_allclose(a[1], b[1], atol=1e-13, rtol=0)

# ---------------------------------------------------------------------------------------
# c-P8c: tree-mask verification
# ---------------------------------------------------------------------------------------
def _tree_inputs(seed, batch=3, q_len=6, kv=(20, 90), hq=8, hkv=2):
    spec = scaled(CONFIGS["tree_verify"], batch=batch, q_len=q_len, kv_len=kv, hq=hq, hkv=hkv, seed=seed)
    inp = make_paged(spec)
    return spec, inp, _f64(inp["q"]), _f64(inp["k_cache"]), _f64(inp["v_cache"])


def test_tree_of_a_chain_equals_causal_verify():
    spec, inp, q, kc, vc = _tree_inputs(31)
    chain = np.tile((1 << (np.arange(spec.q_len) + 1)) - 1, spec.batch).astype(np.int32)
    for window in (0, 11):
        a = oracle.decode_paged_tree(q, kc, vc, inp["page_table"], inp["kv_lens"], chain, inp["sinks"], spec.q_len,
                                     spec.scale, window)
        b = oracle.decode_paged(q, kc, vc, inp["page_table"], inp["kv_lens"], inp["sinks"], spec.q_len, spec.scale,
                                True, window)
        np.testing.assert_allclose(a[0], b[0], atol=1e-13, rtol=0)
        np.testing.assert_allclose(a[1], b[1], atol=1e-13, rtol=0)


def test_tree_without_draft_bits_sees_the_prefix_only():
    spec, inp, q, kc, vc = _tree_inputs(32)
    none = np.zeros(spec.batch * spec.q_len, dtype=np.int32)
    out, lse = oracle.decode_paged_tree(q, kc, vc, inp["page_table"], inp["kv_lens"], none, inp["sinks"],
                                        spec.q_len, spec.scale)
    for b, L in enumerate(inp["kv_lens"]):
        pre = int(L) - spec.q_len
        kb = _flat_gather(kc, inp["page_table"][b], L)[:pre]
        vb = _flat_gather(vc, inp["page_table"][b], L)[:pre]
        o2, l2 = oracle.attend(q[b * spec.q_len:(b + 1) * spec.q_len], kb, vb, inp["sinks"], spec.scale, False, 0)
        np.testing.assert_allclose(out[b * spec.q_len:(b + 1) * spec.q_len], o2, atol=1e-13, rtol=0)
        np.testing.assert_allclose(lse[b * spec.q_len:(b + 1) * spec.q_len], l2, atol=1e-13, rtol=0)


def test_tree_verify_against_library_masked_attention():
    spec, inp, q, kc, vc = _tree_inputs(33, q_len=8)
    trees = make_tree_masks(spec)
    out, lse = oracle.decode_paged_tree(q, kc, vc, inp["page_table"], inp["kv_lens"], trees, inp["sinks"],
                                        spec.q_len, spec.scale)
    G = spec.hq // spec.hkv
    for b, L in enumerate(inp["kv_lens"]):
        L = int(L)
        rows = slice(b * spec.q_len, (b + 1) * spec.q_len)
        # the mask written out from the tree's parent links, not from the oracle's helper
        mask = np.ones((spec.q_len, L), dtype=bool)
        mask[:, L - spec.q_len:] = False
        for t in range(spec.q_len):
            for i in range(spec.q_len):
                if trees[b * spec.q_len + t] & (1 << i):
                    mask[t, L - spec.q_len + i] = True
        kb = _flat_gather(kc, inp["page_table"][b], L)
        vb = _flat_gather(vc, inp["page_table"][b], L)
        qt = torch.from_numpy(np.ascontiguousarray(q[rows].transpose(1, 0, 2)))
        kt = torch.from_numpy(np.ascontiguousarray(kb.transpose(1, 0, 2))).repeat_interleave(G, 0)
        vt = torch.from_numpy(np.ascontiguousarray(vb.transpose(1, 0, 2))).repeat_interleave(G, 0)
        po = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(mask),
                                                              scale=spec.scale).numpy().transpose(1, 0, 2)
        s = spec.scale * torch.einsum("hqd,hkd->hqk", qt, kt).numpy()
        pl = np.log(np.where(mask[None], np.exp(s), 0.0).sum(-1)).T
        sig = 1.0 / (1.0 + np.exp(inp["sinks"][None, :].astype(np.float64) - pl))
        np.testing.assert_allclose(out[rows], po * sig[..., None], atol=1e-12, rtol=0)
        np.testing.assert_allclose(lse[rows], np.logaddexp(pl, inp["sinks"][None, :]), atol=1e-12, rtol=0)


def test_tree_masks_are_ancestor_closed():
    spec = CONFIGS["tree_verify"]
    trees = make_tree_masks(spec, batch=50).reshape(50, spec.q_len)
    for row in trees:
        assert row[0] == 1
        for i in range(1, spec.q_len):
            assert row[i] & (1 << i) and row[i] < (1 << (i + 1))      # itself, no later node
            parents = [j for j in range(i) if row[i] & (1 << j) and (row[i] & ~(1 << i)) == row[j]]
            assert len(parents) == 1                                     # exactly one parent

# ---------------------------------------------------------------------------------------
# c-P9: a large sink takes the weight
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("sink", [8.0, 20.0])
def test_large_sink_dominates(sink):
    rng = np.random.default_rng(12)
    q, k, v = _rand(rng, 1, 64) * 0.1, _rand(rng, 4, 64) * 0.1, _rand(rng, 4, 1, 64)
    w, ws, lse = oracle.attention_weights(q, k, sink, 0.125, True, 0)
    s = 0.125 * (q @ k.T)[0]
    expect_ws = 1.0 / (1.0 + np.exp(s - sink).sum())
    assert abs(ws[0] - expect_ws) < 1e-15 and ws[0] > 0.99
    out, _ = oracle.attend(q[:, None, :], k[:, None, :], v, np.array([sink]), 0.125, True, 0)
    assert np.abs(out).max() < 4 * np.exp(np.abs(s).max() - sink) * np.abs(v).max()


# ---------------------------------------------------------------------------------------
# c-P10: integer plan equals its closed form
# ---------------------------------------------------------------------------------------
def test_plan_closed_form():
    lens = [1, 511, 512, 513, 1024, 8192, 0, 7777]
    for chunk in (1, 128, 512, 2048):
        for q_len in (1, 5):
            counts, indptr = oracle.plan_chunks(lens, q_len, chunk)
            exp_counts = np.repeat([max(1, (L + chunk - 1) // chunk) for L in lens], q_len)
            assert counts == exp_counts.tolist()
            assert indptr[0] == 0 and indptr[-1] == int(exp_counts.sum()) and len(indptr) == len(lens) * q_len + 1
            assert np.all(np.diff(indptr) == exp_counts)
    counts, indptr = oracle.plan_chunks(lens, 2, 0)
    assert counts == [1] * 16 and indptr == list(range(17))


def test_split_decode_layout_matches_plan():
    spec = scaled(CONFIGS["verify"], batch=2, kv_len=(30, 50), hq=4, hkv=1, kv_chunk=16, seed=13)
    inp = make_paged(spec)
    f = lambda x: bf16_bits_to_f32(x).astype(np.float64)
    q, kc, vc = f(inp["q"]), f(inp["k_cache"]), f(inp["v_cache"])
    o_p, l_p, counts, indptr = oracle.split_decode(q, kc, vc, inp["page_table"], inp["kv_lens"], inp["sinks"],
                                                   spec.q_len, spec.scale, spec.kv_chunk)
    out, lse = oracle.decode_paged(q, kc, vc, inp["page_table"], inp["kv_lens"], inp["sinks"], spec.q_len,
                                   spec.scale)
    for r in range(len(counts)):
        mo, ml = oracle.merge(o_p[indptr[r]:indptr[r + 1]], l_p[indptr[r]:indptr[r + 1]])
        np.testing.assert_allclose(mo, out[r], atol=1e-12, rtol=0)
        np.testing.assert_allclose(ml, lse[r], atol=1e-12, rtol=0)


# ---------------------------------------------------------------------------------------
# Hand-derived cases
# ---------------------------------------------------------------------------------------
def _ev(x):
    if isinstance(x, list):
        return [_ev(y) for y in x]
    if isinstance(x, str):
        return float(eval(x, {"__builtins__": {}}, {"log": math.log, "exp": math.exp, "e": math.e,
                                                   "inf": math.inf}))
    return float(x)


def _cases():
    with open(GOLDEN) as fh:
        return json.load(fh)["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_hand_derived(case):
    hq, hkv, d = case["hq"], case["hkv"], case["d"]
    q = np.array(_ev(case["q"]), dtype=np.float64).reshape(-1, hq, d)
    k = np.array(_ev(case["k"]), dtype=np.float64).reshape(-1, hkv, d)
    v = np.array(_ev(case["v"]), dtype=np.float64).reshape(-1, hkv, d)
    sinks = np.array(_ev(case["sinks"]), dtype=np.float64)
    out, lse = oracle.attend(q, k, v, sinks, case["scale"], case["causal"], case["window"])
    np.testing.assert_allclose(out, np.array(_ev(case["out"])).reshape(out.shape), atol=1e-13, rtol=1e-13)
    exp_lse = np.array(_ev(case["lse"])).reshape(lse.shape)
    assert np.array_equal(np.isinf(lse), np.isinf(exp_lse))
    fin = np.isfinite(exp_lse)
    np.testing.assert_allclose(lse[fin], exp_lse[fin], atol=1e-13, rtol=0)


# ---------------------------------------------------------------------------------------
# Seeded inputs
# ---------------------------------------------------------------------------------------
def test_inputs_deterministic_and_shaped():
    a = make_varlen(CONFIGS["tiny_causal"])
    b = make_varlen(CONFIGS["tiny_causal"])
    assert all(np.array_equal(a[x], b[x]) for x in ("q", "k", "v", "sinks", "cu_seqlens"))
    assert a["q"].shape == (16, 4, 64) and a["k"].shape == (16, 1, 64) and a["cu_seqlens"].tolist() == [0, 16]
    spec = scaled(CONFIGS["paged_decode"], batch=6, kv_len=(1, 100))
    p = make_paged(spec)
    used = np.concatenate([p["page_table"][b, :(L + 15) // 16] for b, L in enumerate(p["kv_lens"])])
    assert sorted(used.tolist()) == list(range(p["num_pages"]))       # bijection onto the pool
    assert p["page_table"].shape == (6, 7)


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -7 + 2 ** -9, -2.5], dtype=np.float32)
    got = bf16_bits_to_f32(__import__("workloads").bf16_round_bits(x))
    # ties go to the even mantissa; 1 + 2^-7 + 2^-9 rounds up to the nearer 1 + 2^-7
    assert got.tolist() == [1.0, 1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7, -2.5]
    t = torch.from_numpy(np.random.default_rng(0).standard_normal(1000).astype(np.float32))
    ref = t.to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(bf16_bits_to_f32(__import__("workloads").bf16_round_bits(t.numpy())), ref)
