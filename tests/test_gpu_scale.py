"""GPU parity at index ranges the workload shapes do not reach: decode batches of more than 64
sequences (the split kernel locates an item's sequence through a cursor that walks kv_lens 64
sequences at a time) and more than 256 query heads (the decode kernel holds the sinks of heads
0..255 in lane vectors and loads the others directly).

Method ("GPT-OSS on Day 0", section "Attention sinks"): softmax over the scaled scores plus one
sink logit per head, the sink counted only in the first KV chunk, chunk partials merged by
log-sum-exp. Bar as in every parity test: bf16 outputs within 1e-2 + 1e-2 |ref|, LSE within 1e-3,
the -inf pattern of LSE exact, the integer plan bit-exact.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from workloads import CONFIGS, bf16_bits_to_f32, make_paged, make_tree_masks, make_varlen, scaled  # noqa: E402

pytestmark = pytest.mark.gpu

ATOL, RTOL, LSE_TOL = 1e-2, 1e-2, 1e-3
DEV = "cuda:0"


@pytest.fixture(scope="module")
def amd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_attention_sinks_sink_amd as amd
    return amd


def tbits(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def f64(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


def assert_close(out, lse, ro, rl, what):
    sel = ~np.isnan(rl)
    o, r = out[sel], ro[sel]
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    excess = np.abs(o - r) - (ATOL + RTOL * np.abs(r))
    assert excess.max(initial=-1.0) <= 0, f"{what}: out max excess {excess.max():.3e}"
    l, rr = lse[sel], rl[sel]
    inf = np.isinf(rr)
    assert np.array_equal(np.isinf(l), inf) and np.array_equal(l[inf], rr[inf]), f"{what}: lse inf pattern"
    if (~inf).any():
        err = np.abs(l[~inf] - rr[~inf]).max()
        assert err <= LSE_TOL, f"{what}: lse max err {err:.3e}"


def device_paged(inp):
    return dict(q=tbits(inp["q"]), k=tbits(inp["k_cache"]), v=tbits(inp["v_cache"]),
                table=torch.from_numpy(inp["page_table"]).to(DEV), lens=torch.from_numpy(inp["kv_lens"]).to(DEV),
                sinks=torch.from_numpy(inp["sinks"]).to(DEV))


def boundary_lengths(rng, batch, hi, q_len, chunk):
    """Ragged lengths with empty sequences (q_len 1 only), lengths just under, at and over the chunk
    boundary, and the rest uniform."""
    lens = rng.integers(q_len, hi + 1, size=batch)
    edge = [q_len, chunk - 1, chunk, chunk + 1, 2 * chunk, hi]
    if q_len == 1:
        edge.append(0)
    pos = rng.choice(batch, size=min(batch, 3 * len(edge)), replace=False)
    for i, p in enumerate(pos):
        lens[p] = max(edge[i % len(edge)], q_len if q_len > 1 else 0)
    return lens.astype(np.int32)


@pytest.mark.parametrize("batch,q_len,chunk", [(65, 1, 128), (200, 1, 64), (130, 3, 256), (300, 1, 0)])
def test_decode_batches_beyond_one_cursor_window(amd, batch, q_len, chunk):
    rng = np.random.default_rng(900 + batch + q_len)
    c = chunk if chunk > 0 else 512
    spec = scaled(CONFIGS["verify"], batch=batch, q_len=q_len, kv_len=(q_len, 600), hq=16, hkv=2, kv_chunk=chunk,
                  seed=900 + batch)
    inp = make_paged(spec, kv_lens=boundary_lengths(rng, batch, 600, q_len, c))
    d = device_paged(inp)
    need = amd.attn_sink_decode_workspace_size(batch, q_len, inp["max_kv_len"], spec.hq, 64, chunk)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    print(f"decode batch {batch} q_len {q_len} chunk {chunk}", flush=True)
    out, lse = amd.attn_sink_decode_paged(d["q"], d["k"], d["v"], d["table"], d["lens"], d["sinks"], q_len,
                                          inp["max_kv_len"], spec.scale, True, 0, chunk, workspace=ws)
    torch.cuda.synchronize()
    ro, rl = oracle.decode_paged(f64(inp["q"]), f64(inp["k_cache"]), f64(inp["v_cache"]), inp["page_table"],
                                 inp["kv_lens"], inp["sinks"], q_len, spec.scale, True, 0)
    assert_close(out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ro, rl,
                 f"decode batch {batch} q_len {q_len} chunk {chunk}")
    # the plan the kernel wrote for every sequence, bit-exact
    lay = amd.decode_workspace_layout(batch, q_len, inp["max_kv_len"], spec.hq, chunk)
    w = ws.cpu().numpy()
    rows = lay["rows"]
    indptr = w[lay["off_indptr"]:lay["off_indptr"] + 4 * (rows + 1)].view(np.int32)
    counts = w[lay["off_counts"]:lay["off_counts"] + 4 * rows].view(np.int32)
    exp_counts, exp_indptr = oracle.plan_chunks(inp["kv_lens"], q_len, chunk)
    assert counts.tolist() == exp_counts and indptr.tolist() == exp_indptr


def test_tree_verify_batch_beyond_one_cursor_window(amd):
    spec = scaled(CONFIGS["tree_verify"], batch=100, q_len=4, kv_len=(4, 500), hq=16, hkv=2, kv_chunk=128, seed=950)
    inp = make_paged(spec)
    trees = make_tree_masks(spec)
    d = device_paged(inp)
    print("tree verify batch 100", flush=True)
    out, lse = amd.attn_sink_decode_paged_tree(d["q"], d["k"], d["v"], d["table"], d["lens"],
                                               torch.from_numpy(trees).to(DEV), d["sinks"], spec.q_len,
                                               inp["max_kv_len"], spec.scale, 0, spec.kv_chunk)
    torch.cuda.synchronize()
    ro, rl = oracle.decode_paged_tree(f64(inp["q"]), f64(inp["k_cache"]), f64(inp["v_cache"]), inp["page_table"],
                                      inp["kv_lens"], trees, inp["sinks"], spec.q_len, spec.scale, 0)
    assert_close(out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ro, rl,
                 "tree verify batch 100")


@pytest.mark.parametrize("hq,hkv,q_len", [(320, 40, 1), (512, 8, 1), (288, 36, 2)])
def test_decode_more_than_256_query_heads(amd, hq, hkv, q_len):
    """Heads past 255 take their sink from memory rather than from the lane vectors; a per-head
    mix of extreme sinks makes a wrong head's sink visible."""
    rng = np.random.default_rng(960 + hq)
    spec = scaled(CONFIGS["verify"], batch=3, q_len=q_len, kv_len=(q_len, 900), hq=hq, hkv=hkv, kv_chunk=256,
                  seed=960 + hq)
    inp = make_paged(spec)
    inp["sinks"] = rng.choice(np.array([-np.inf, 0.0, 20.0, -20.0, 3.0, 8.0, -5.0], dtype=np.float32), size=hq)
    d = device_paged(inp)
    print(f"decode hq {hq} hkv {hkv} q_len {q_len}", flush=True)
    out, lse = amd.attn_sink_decode_paged(d["q"], d["k"], d["v"], d["table"], d["lens"], d["sinks"], q_len,
                                          inp["max_kv_len"], spec.scale, True, 0, spec.kv_chunk)
    torch.cuda.synchronize()
    ro, rl = oracle.decode_paged(f64(inp["q"]), f64(inp["k_cache"]), f64(inp["v_cache"]), inp["page_table"],
                                 inp["kv_lens"], inp["sinks"], q_len, spec.scale, True, 0)
    assert_close(out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ro, rl,
                 f"decode hq {hq}")


def test_prefill_more_than_256_query_heads(amd):
    spec = scaled(CONFIGS["causal_prefill"], batch=2, seqlen=(40, 300), hq=320, hkv=40, seed=970)
    inp = make_varlen(spec, seqlens=[300, 41])
    rng = np.random.default_rng(970)
    inp["sinks"] = rng.choice(np.array([-np.inf, 0.0, 20.0, -20.0, 3.0, 8.0], dtype=np.float32), size=spec.hq)
    cu = torch.from_numpy(inp["cu_seqlens"]).to(DEV)
    print("prefill hq 320", flush=True)
    out, lse = amd.attn_sink_prefill(tbits(inp["q"]), tbits(inp["k"]), tbits(inp["v"]),
                                     torch.from_numpy(inp["sinks"]).to(DEV), cu, cu, 300, 300, spec.scale, True, 0)
    torch.cuda.synchronize()
    ro, rl = oracle.prefill_varlen(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), inp["cu_seqlens"],
                                   inp["cu_seqlens"], inp["sinks"], spec.scale, True, 0)
    assert_close(out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ro, rl,
                 "prefill hq 320")


@pytest.mark.parametrize("seqlen,hq,hkv,causal,window", [(32768, 8, 1, True, 0), (16384, 16, 2, False, 0),
                                                         (6000, 16, 2, True, 1500)])
def test_prefill_long_sequences_sampled(amd, seqlen, hq, hkv, causal, window):
    """Sequences far longer than the workloads' 4096 tokens: the causal 8-wave kernel over 512
    row blocks, the bidirectional one over 16K keys per row, and the 4-wave kernel with a 1500-key
    window (about 48 tiles per pass, masked at both ends). Sampled rows of the long sequence (block
    edges, the middle, the tail) and every row of a short second sequence."""
    spec = scaled(CONFIGS["causal_prefill"], batch=2, hq=hq, hkv=hkv, causal=causal, window=window,
                  seed=980 + hq + window)
    inp = make_varlen(spec, seqlens=[seqlen, 777])
    rng = np.random.default_rng(980 + seqlen)
    picks = {0, 1, 63, 64, 511, 512, 4095, 4096, seqlen // 2, seqlen - 65, seqlen - 64, seqlen - 1}
    picks |= set(rng.integers(0, seqlen, size=8).tolist())
    rows = {0: sorted(picks), 1: list(range(777))}
    cu = torch.from_numpy(inp["cu_seqlens"]).to(DEV)
    print(f"prefill seqlen {seqlen} hq {hq} hkv {hkv} causal {causal} window {window}", flush=True)
    out, lse = amd.attn_sink_prefill(tbits(inp["q"]), tbits(inp["k"]), tbits(inp["v"]),
                                     torch.from_numpy(inp["sinks"]).to(DEV), cu, cu, seqlen, seqlen, spec.scale,
                                     causal, window)
    torch.cuda.synchronize()
    ro, rl = oracle.prefill_varlen(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), inp["cu_seqlens"],
                                   inp["cu_seqlens"], inp["sinks"], spec.scale, causal, window, seqs=[0, 1],
                                   rows=rows)
    assert_close(out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ro, rl,
                 f"prefill seqlen {seqlen} causal {causal} window {window}")


@pytest.mark.parametrize("q_len,chunk", [(1, 0), (1, 16384), (4, 3072), (1, -1)])
def test_decode_one_very_long_sequence(amd, q_len, chunk):
    """65536 keys in one sequence next to a short one: with one chunk per sequence (chunk 0) an item
    holds 4096 page groups, so every wave walks its page ids through 16 segments of 64 groups.
    chunk -1 takes the planner's choice for this batch."""
    spec = scaled(CONFIGS["verify"], batch=2, q_len=q_len, kv_len=(q_len, 65536), hq=16, hkv=2, kv_chunk=max(chunk, 0),
                  seed=990 + q_len)
    inp = make_paged(spec, kv_lens=[65536, 1000 + q_len])
    if chunk < 0:
        chunk = amd.attn_sink_decode_plan_chunk(inp["kv_lens"], q_len, spec.hq, spec.hkv, spec.page_size)
    d = device_paged(inp)
    print(f"decode 65536 keys q_len {q_len} chunk {chunk}", flush=True)
    out, lse = amd.attn_sink_decode_paged(d["q"], d["k"], d["v"], d["table"], d["lens"], d["sinks"], q_len,
                                          inp["max_kv_len"], spec.scale, True, 0, chunk)
    torch.cuda.synchronize()
    ro, rl = oracle.decode_paged(f64(inp["q"]), f64(inp["k_cache"]), f64(inp["v_cache"]), inp["page_table"],
                                 inp["kv_lens"], inp["sinks"], q_len, spec.scale, True, 0)
    assert_close(out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ro, rl,
                 f"decode 65536 keys q_len {q_len} chunk {chunk}")


@pytest.mark.parametrize("lq,lk,causal,window", [((300, 50, 9), (100, 0, 9), True, 0), ((300, 50, 9), (100, 0, 9), True, 40),
                                                 ((300, 50, 9), (100, 0, 9), False, 0),
                                                 ((2100, 64), (500, 64), True, 0), ((2100, 64), (500, 2100), False, 0)])
def test_prefill_more_queries_than_keys(amd, lq, lk, causal, window):
    """Queries are the last tokens of their sequence, so with more query tokens than keys the first
    Lq - Lk rows have no causal key (out 0, LSE the sink), and a sequence with no keys at all gives
    every row that. The 4-wave kernel (the first three cases) and the 8-wave one (2100 query
    tokens, no window)."""
    spec = scaled(CONFIGS["causal_prefill"], batch=len(lq), hq=16, hkv=2, causal=causal, window=window,
                  seed=1000 + lq[0] + window)
    inp = make_varlen(spec, seqlens=list(lq))
    rng = np.random.default_rng(1000 + lk[0])
    lk = np.asarray(lk)
    cu_kv = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    from workloads import bf16_round_bits
    k = bf16_round_bits(rng.standard_normal((int(lk.sum()), 2, 64), dtype=np.float32))
    v = bf16_round_bits(rng.standard_normal((int(lk.sum()), 2, 64), dtype=np.float32))
    cu = torch.from_numpy(inp["cu_seqlens"]).to(DEV)
    print(f"prefill lq {lq} lk {tuple(lk)} causal {causal} window {window}", flush=True)
    out, lse = amd.attn_sink_prefill(tbits(inp["q"]), tbits(k), tbits(v), torch.from_numpy(inp["sinks"]).to(DEV), cu,
                                     torch.from_numpy(cu_kv).to(DEV), max(lq), int(lk.max()), spec.scale, causal, window)
    torch.cuda.synchronize()
    ro, rl = oracle.prefill_varlen(f64(inp["q"]), f64(k), f64(v), inp["cu_seqlens"], cu_kv, inp["sinks"], spec.scale,
                                   causal, window)
    assert_close(out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ro, rl,
                 f"prefill lq {lq} lk {tuple(lk)} causal {causal} window {window}")


def test_merge_rows_of_many_partials(amd):
    """Rows of 0 to 150 partials (the merge reads 16 per round trip, in two groups of 8), LSEs
    spread over +-80 with empty (-inf) partials mixed in, against the oracle's merge row by row."""
    rng = np.random.default_rng(1010)
    counts = np.array([0, 1, 7, 8, 9, 16, 17, 63, 64, 65, 150] + rng.integers(0, 40, size=21).tolist())
    indptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    n, hq = int(indptr[-1]), 4
    o_p = rng.standard_normal((n, hq, 64)).astype(np.float32)
    l_p = (rng.uniform(-80, 80, size=(n, hq))).astype(np.float32)
    l_p[rng.random((n, hq)) < 0.2] = -np.inf
    print(f"merge of {len(counts)} rows, {n} partials", flush=True)
    out, lse = amd.attn_sink_merge_partials(torch.from_numpy(o_p).to(DEV), torch.from_numpy(l_p).to(DEV),
                                            torch.from_numpy(indptr).to(DEV))
    torch.cuda.synchronize()
    ro = np.zeros((len(counts), hq, 64))
    rl = np.full((len(counts), hq), -np.inf)
    for r in range(len(counts)):
        a, b = int(indptr[r]), int(indptr[r + 1])
        if b > a:
            ro[r], rl[r] = oracle.merge(o_p[a:b].astype(np.float64), l_p[a:b].astype(np.float64))
    assert_close(out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ro, rl,
                 "merge of many partials")
