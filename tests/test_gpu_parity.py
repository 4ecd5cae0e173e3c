"""GPU parity: the HIP kernels (through the C ABI) against the fp64 oracle on the same
seeded inputs.

Bar (fixed for this method): bf16 outputs within |err| <= 1e-2 + 1e-2*|ref|, LSE within
1e-3 absolute, integer plan outputs bit-exact, page-pool permutation bit-identical.
Small cases run the whole oracle; full-size workloads are checked on sampled rows.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from workloads import (CONFIGS, bf16_bits_to_f32, make_paged, make_paged_prefill, make_tree_masks,  # noqa: E402
                       make_varlen, scaled)

pytestmark = pytest.mark.gpu

ATOL, RTOL, LSE_TOL = 1e-2, 1e-2, 1e-3


@pytest.fixture(scope="module")
def amd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_attention_sinks_sink_amd as amd
    return amd


DEV = "cuda:0"


def tbits(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def f64(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


def out_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def assert_close(out, lse, ro, rl, what):
    sel = ~np.isnan(rl)
    o = out[sel]
    r = ro[sel]
    excess = np.abs(o - r) - (ATOL + RTOL * np.abs(r))
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    assert excess.max() <= 0, f"{what}: out max excess {excess.max():.3e} (max err {np.abs(o - r).max():.3e})"
    if lse is not None:
        l, rr = lse[sel], rl[sel]
        inf = np.isinf(rr)
        assert np.array_equal(np.isinf(l), inf) and np.array_equal(l[inf], rr[inf]), f"{what}: lse inf pattern"
        if (~inf).any():
            err = np.abs(l[~inf] - rr[~inf]).max()
            assert err <= LSE_TOL, f"{what}: lse max err {err:.3e}"


# -------------------------------------------------------------------------------------------
# prefill / embedding
# -------------------------------------------------------------------------------------------
def run_prefill(amd, inp, spec, sinks=True, cu_kv=None, k=None, v=None, max_kv=None):
    cu = torch.from_numpy(inp["cu_seqlens"]).to(DEV)
    cukv = cu if cu_kv is None else torch.from_numpy(cu_kv).to(DEV)
    s = torch.from_numpy(inp["sinks"]).to(DEV) if sinks else None
    out, lse = amd.attn_sink_prefill(tbits(inp["q"]), tbits(inp["k"] if k is None else k),
                                     tbits(inp["v"] if v is None else v), s, cu, cukv, inp["max_seqlen"],
                                     inp["max_seqlen"] if max_kv is None else max_kv, spec.scale, spec.causal,
                                     spec.window)
    torch.cuda.synchronize()
    return out_f64(out), lse.cpu().numpy().astype(np.float64)


def oracle_prefill(inp, spec, sinks=True, **kw):
    s = inp["sinks"] if sinks else np.full_like(inp["sinks"], -np.inf)
    return oracle.prefill_varlen(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), inp["cu_seqlens"], inp["cu_seqlens"], s,
                                 spec.scale, spec.causal, spec.window, **kw)


def test_tiny_causal_config(amd):
    spec = CONFIGS["tiny_causal"]
    inp = make_varlen(spec)
    out, lse = run_prefill(amd, inp, spec)
    ro, rl = oracle_prefill(inp, spec)
    assert_close(out, lse, ro, rl, "tiny")


@pytest.mark.parametrize("hq,hkv", [(16, 2), (8, 8), (12, 2), (32, 2), (4, 4)])
@pytest.mark.parametrize("window", [0, 128, 37])
def test_prefill_ragged_causal(amd, hq, hkv, window):
    spec = scaled(CONFIGS["causal_prefill"], batch=3, seqlen=(1, 300), hq=hq, hkv=hkv, window=window, seed=40 + hq)
    inp = make_varlen(spec, seqlens=[300, 129, 1])
    out, lse = run_prefill(amd, inp, spec)
    ro, rl = oracle_prefill(inp, spec)
    assert_close(out, lse, ro, rl, f"prefill G={hq // hkv} W={window}")


@pytest.mark.parametrize("sinks", [False, True])
def test_embedding_bidirectional_ragged(amd, sinks):
    spec = scaled(CONFIGS["embed_sink"], batch=24, hq=4, hkv=4, seed=41)
    inp = make_varlen(spec)
    out, lse = run_prefill(amd, inp, spec, sinks=sinks)
    ro, rl = oracle_prefill(inp, spec, sinks=sinks)
    assert_close(out, lse, ro, rl, f"embed sinks={sinks}")


def test_prefill_edge_cases(amd):
    # empty sequences in the batch, a 1-token sequence, a sequence not a multiple of the tile
    spec = scaled(CONFIGS["causal_prefill"], batch=5, hq=8, hkv=2, seed=42)
    inp = make_varlen(spec, seqlens=[0, 65, 0, 1, 200])
    out, lse = run_prefill(amd, inp, spec)
    ro, rl = oracle_prefill(inp, spec)
    assert_close(out, lse, ro, rl, "prefill edges")
    # sinks pointer NULL == every sink disabled
    out2, lse2 = run_prefill(amd, inp, spec, sinks=False)
    ro2, rl2 = oracle_prefill(inp, spec, sinks=False)
    assert_close(out2, lse2, ro2, rl2, "prefill no sinks")


def test_prefill_mixed_and_extreme_sinks(amd):
    spec = scaled(CONFIGS["causal_prefill"], batch=2, hq=8, hkv=1, seed=43)
    inp = make_varlen(spec, seqlens=[40, 150])
    inp["sinks"] = np.array([-np.inf, 0.0, 20.0, -20.0, 3.0, -np.inf, 8.0, 1.0], dtype=np.float32)
    out, lse = run_prefill(amd, inp, spec)
    ro, rl = oracle_prefill(inp, spec)
    assert_close(out, lse, ro, rl, "extreme sinks")


def test_prefill_queries_shorter_than_keys(amd):
    """Chunked-prefill shape: the last Lq tokens attend to Lk >= Lq keys (bottom-right causal)."""
    spec = scaled(CONFIGS["causal_prefill"], batch=2, hq=8, hkv=2, seed=44)
    inp = make_varlen(spec, seqlens=[70, 33])
    rng = np.random.default_rng(7)
    lk = np.array([200, 33])
    cu_kv = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    from workloads import bf16_round_bits
    k = bf16_round_bits(rng.standard_normal((int(lk.sum()), 2, 64), dtype=np.float32))
    v = bf16_round_bits(rng.standard_normal((int(lk.sum()), 2, 64), dtype=np.float32))
    out, lse = run_prefill(amd, inp, spec, cu_kv=cu_kv, k=k, v=v, max_kv=200)
    ro, rl = oracle.prefill_varlen(f64(inp["q"]), f64(k), f64(v), inp["cu_seqlens"], cu_kv, inp["sinks"], spec.scale,
                                   True, 0)
    assert_close(out, lse, ro, rl, "q shorter than kv")


def test_prefill_deterministic(amd):
    spec = scaled(CONFIGS["causal_prefill"], batch=2, hq=16, hkv=2, seed=45)
    inp = make_varlen(spec, seqlens=[257, 300])
    a = run_prefill(amd, inp, spec)
    b = run_prefill(amd, inp, spec)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("hq,hkv,sinks", [(8, 1, True), (16, 16, True), (32, 2, False), (12, 3, True),
                                           (4, 2, True)])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_long_sequences(amd, hq, hkv, sinks, causal):
    """Batches whose longest sequence has >= 2048 tokens (the 8-wave kernel without a window):
    ragged lengths, a short sequence in the same batch, every packing of query heads per tile
    (GQA group 1, 2, 4, 8, 16), causal and bidirectional, with and without sinks. Sampled rows
    cover whole 64-token blocks at both ends, both wave groups and several row blocks."""
    spec = scaled(CONFIGS["causal_prefill"], batch=3, hq=hq, hkv=hkv, causal=causal, seed=60 + hq + causal)
    inp = make_varlen(spec, seqlens=[2100, 77, 2048 + 37])
    out, lse = run_prefill(amd, inp, spec, sinks=sinks)
    rows = {0: list(range(0, 70)) + [511, 512, 1023, 1500, 2047] + list(range(2030, 2100)),
            1: list(range(77)),
            2: [0, 31, 32, 1000] + list(range(2040, 2085))}
    ro, rl = oracle_prefill(inp, spec, sinks=sinks, seqs=list(rows), rows=rows)
    assert_close(out, lse, ro, rl, f"long prefill hq={hq} hkv={hkv} causal={causal}")


@pytest.mark.parametrize("name", ["causal_prefill", "window_prefill"])
def test_prefill_full_size_sampled(amd, name):
    spec = CONFIGS[name]
    inp = make_varlen(spec)
    out, lse = run_prefill(amd, inp, spec)
    rows = {0: [0, 1, 63, 64, 127, 128, 4095], 5: [2047, 4000], 7: [100, 3071, 4094]}
    ro, rl = oracle_prefill(inp, spec, seqs=list(rows), rows=rows)
    assert_close(out, lse, ro, rl, name)


@pytest.mark.parametrize("name", ["embed_nosink", "embed_sink"])
def test_embedding_full_size_sampled(amd, name):
    spec = CONFIGS[name]
    inp = make_varlen(spec)
    out, lse = run_prefill(amd, inp, spec, sinks=spec.sink_std is not None)
    ro, rl = oracle.prefill_varlen(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), inp["cu_seqlens"],
                                   inp["cu_seqlens"], inp["sinks"], spec.scale, False, 0, seqs=[0, 1, 77, 300, 511])
    assert_close(out, lse, ro, rl, name)


# -------------------------------------------------------------------------------------------
# chunked prefill on a paged cache
# -------------------------------------------------------------------------------------------
def run_prefill_paged(amd, inp, spec, sinks=True, causal=None, window=None):
    s = torch.from_numpy(inp["sinks"]).to(DEV) if sinks else None
    out, lse = amd.attn_sink_prefill_paged(
        tbits(inp["q"]), tbits(inp["k_cache"]), tbits(inp["v_cache"]), torch.from_numpy(inp["page_table"]).to(DEV),
        torch.from_numpy(inp["cu_seqlens_q"]).to(DEV), torch.from_numpy(inp["kv_lens"]).to(DEV), s, inp["max_q"],
        inp["max_kv_len"], spec.scale, spec.causal if causal is None else causal,
        spec.window if window is None else window)
    torch.cuda.synchronize()
    return out_f64(out), lse.cpu().numpy().astype(np.float64)


def oracle_prefill_paged(inp, spec, sinks=True, causal=None, window=None, **kw):
    s = inp["sinks"] if sinks else np.full_like(inp["sinks"], -np.inf)
    return oracle.prefill_paged(f64(inp["q"]), f64(inp["k_cache"]), f64(inp["v_cache"]), inp["page_table"],
                                inp["cu_seqlens_q"], inp["kv_lens"], s, spec.scale,
                                spec.causal if causal is None else causal, spec.window if window is None else window,
                                **kw)


@pytest.mark.parametrize("hq,hkv,page_size", [(16, 2, 16), (8, 8, 32), (64, 8, 16), (12, 3, 64), (4, 4, 256)])
@pytest.mark.parametrize("causal,window", [(True, 0), (True, 45), (False, 0)])
def test_prefill_paged_ragged(amd, hq, hkv, page_size, causal, window):
    spec = scaled(CONFIGS["chunked_prefill"], batch=4, q_len=(1, 300), ctx_len=(0, 700), hq=hq, hkv=hkv,
                  page_size=page_size, seed=hq + hkv + page_size)
    inp = make_paged_prefill(spec)
    out, lse = run_prefill_paged(amd, inp, spec, causal=causal, window=window)
    ro, rl = oracle_prefill_paged(inp, spec, causal=causal, window=window)
    assert_close(out, lse, ro, rl, f"paged prefill hq={hq} hkv={hkv} page={page_size} causal={causal} w={window}")


def test_prefill_paged_edge_lengths_and_no_sink(amd):
    # empty chunks, chunks of one token, no context, context ending mid-page, long single chunk
    spec = scaled(CONFIGS["chunked_prefill"], batch=6, hq=8, hkv=2, seed=71)
    inp = make_paged_prefill(spec, q_lens=[0, 1, 64, 65, 0, 1500], ctx_lens=[5, 0, 0, 17, 0, 33])
    for sinks in (True, False):
        out, lse = run_prefill_paged(amd, inp, spec, sinks=sinks)
        ro, rl = oracle_prefill_paged(inp, spec, sinks=sinks)
        assert_close(out, lse, ro, rl, f"paged prefill edges sinks={sinks}")


@pytest.mark.parametrize("hq,hkv,page_size,causal", [(8, 1, 16, True), (16, 16, 64, True), (12, 3, 32, False)])
def test_prefill_paged_long_chunks(amd, hq, hkv, page_size, causal):
    # chunks of 2048+ tokens run on the 8-wave kernel
    spec = scaled(CONFIGS["chunked_prefill"], batch=3, q_len=(2048, 2200), ctx_len=(0, 700), hq=hq, hkv=hkv,
                  page_size=page_size, seed=80 + hq)
    inp = make_paged_prefill(spec, ctx_lens=[0, 37, 700])
    out, lse = run_prefill_paged(amd, inp, spec, causal=causal)
    rows = {b: [0, 1, 63, 64, 511, 512, 1000, 2047, int(inp["q_lens"][b]) - 1] for b in range(3)}
    ro, rl = oracle_prefill_paged(inp, spec, causal=causal, seqs=list(rows), rows=rows)
    assert_close(out, lse, ro, rl, f"long paged chunks hq={hq} hkv={hkv} page={page_size} causal={causal}")

def test_prefill_paged_page_permutation_bit_identical(amd):
    spec = scaled(CONFIGS["chunked_prefill"], batch=3, q_len=(100, 400), ctx_len=(0, 900), hq=16, hkv=2, seed=72)
    inp = make_paged_prefill(spec)
    a = run_prefill_paged(amd, inp, spec)
    perm = np.random.default_rng(4).permutation(inp["num_pages"])
    inv = np.argsort(perm)
    inp2 = dict(inp)
    inp2["k_cache"], inp2["v_cache"] = inp["k_cache"][inv], inp["v_cache"][inv]
    inp2["page_table"] = perm[inp["page_table"]].astype(np.int32)
    b = run_prefill_paged(amd, inp2, spec)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_prefill_paged_full_size_sampled(amd):
    spec = CONFIGS["chunked_prefill"]
    inp = make_paged_prefill(spec)
    out, lse = run_prefill_paged(amd, inp, spec)
    rows = {0: [0, 1, 63, 64, 2047], 3: [1000, 2046], 7: [5, 1500, 2047]}
    ro, rl = oracle_prefill_paged(inp, spec, seqs=list(rows), rows=rows)
    assert_close(out, lse, ro, rl, "chunked_prefill")

# -------------------------------------------------------------------------------------------
# paged decode / verify
# -------------------------------------------------------------------------------------------
def dev_paged(inp):
    return dict(q=tbits(inp["q"]), k=tbits(inp["k_cache"]), v=tbits(inp["v_cache"]),
                table=torch.from_numpy(inp["page_table"]).to(DEV), lens=torch.from_numpy(inp["kv_lens"]).to(DEV),
                sinks=torch.from_numpy(inp["sinks"]).to(DEV))


def run_decode(amd, d, inp, spec, chunk=None, workspace=None, sinks=True):
    out, lse = amd.attn_sink_decode_paged(d["q"], d["k"], d["v"], d["table"], d["lens"], d["sinks"] if sinks else None,
                                          spec.q_len, inp["max_kv_len"], spec.scale, spec.causal, spec.window,
                                          spec.kv_chunk if chunk is None else chunk, workspace=workspace)
    torch.cuda.synchronize()
    return out_f64(out), lse.cpu().numpy().astype(np.float64)


def oracle_decode(inp, spec, seqs=None, sinks=True):
    s = inp["sinks"] if sinks else np.full_like(inp["sinks"], -np.inf)
    return oracle.decode_paged(f64(inp["q"]), f64(inp["k_cache"]), f64(inp["v_cache"]), inp["page_table"],
                               inp["kv_lens"], s, spec.q_len, spec.scale, spec.causal, spec.window, seqs=seqs)


@pytest.mark.parametrize("q_len,hq,hkv", [(1, 16, 2), (1, 64, 8), (5, 16, 2), (2, 8, 1), (8, 64, 8), (3, 4, 4),
                                          (1, 64, 1)])
def test_decode_small(amd, q_len, hq, hkv):
    spec = scaled(CONFIGS["verify"], kv_chunk=512, batch=5, q_len=q_len, kv_len=(1, 1500), hq=hq, hkv=hkv, seed=50 + q_len + hq)
    inp = make_paged(spec, kv_lens=[1500, 513, 512, 17, 8 if q_len <= 8 else q_len])
    out, lse = run_decode(amd, dev_paged(inp), inp, spec)
    ro, rl = oracle_decode(inp, spec)
    assert_close(out, lse, ro, rl, f"decode q_len={q_len} G={hq // hkv}")


@pytest.mark.parametrize("window", [1, 100, 600])
def test_decode_window(amd, window):
    spec = scaled(CONFIGS["verify"], kv_chunk=512, batch=4, kv_len=(1, 2000), hq=16, hkv=2, window=window, seed=60)
    inp = make_paged(spec)
    out, lse = run_decode(amd, dev_paged(inp), inp, spec)
    ro, rl = oracle_decode(inp, spec)
    assert_close(out, lse, ro, rl, f"decode window {window}")


def test_decode_edge_lengths_and_no_sink(amd):
    spec = scaled(CONFIGS["verify"], kv_chunk=512, batch=5, kv_len=(0, 700), hq=16, hkv=2, seed=61)
    inp = make_paged(spec, kv_lens=[0, 3, 5, 700, 16], max_pages_per_seq=44)
    d = dev_paged(inp)
    for sinks in (True, False):
        out, lse = run_decode(amd, d, inp, spec, sinks=sinks)
        ro, rl = oracle_decode(inp, spec, sinks=sinks)
        assert_close(out, lse, ro, rl, f"decode edges sinks={sinks}")


@pytest.mark.parametrize("page_size,chunk", [(32, 512), (64, 256), (256, 512), (16, 64), (16, 0)])
def test_decode_page_and_chunk_sizes(amd, page_size, chunk):
    spec = scaled(CONFIGS["verify"], batch=4, q_len=2, kv_len=(100, 1300), hq=16, hkv=2, page_size=page_size,
                  kv_chunk=chunk, seed=62)
    inp = make_paged(spec)
    out, lse = run_decode(amd, dev_paged(inp), inp, spec)
    ro, rl = oracle_decode(inp, spec)
    assert_close(out, lse, ro, rl, f"page {page_size} chunk {chunk}")


def test_decode_plan_is_bit_exact_and_partials_match(amd):
    spec = scaled(CONFIGS["verify"], kv_chunk=512, batch=6, kv_len=(1, 1800), hq=16, hkv=2, seed=63)
    inp = make_paged(spec, kv_lens=[1800, 1, 512, 513, 0, 1024])
    d = dev_paged(inp)
    need = amd.attn_sink_decode_workspace_size(6, spec.q_len, inp["max_kv_len"], spec.hq, 64, spec.kv_chunk)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    run_decode(amd, d, inp, spec, workspace=ws)
    lay = amd.decode_workspace_layout(6, spec.q_len, inp["max_kv_len"], spec.hq, spec.kv_chunk)
    w = ws.cpu().numpy()
    rows = lay["rows"]
    indptr = w[:4 * (rows + 1)].view(np.int32)
    counts = w[lay["off_counts"]:lay["off_counts"] + 4 * rows].view(np.int32)
    exp_counts, exp_indptr = oracle.plan_chunks(inp["kv_lens"], spec.q_len, spec.kv_chunk)
    assert counts.tolist() == exp_counts and indptr.tolist() == exp_indptr
    n = exp_indptr[-1]
    o_p = w[lay["off_o"]:lay["off_o"] + 4 * n * spec.hq * 64].view(np.float32).reshape(n, spec.hq, 64)
    l_p = w[lay["off_lse"]:lay["off_lse"] + 4 * n * spec.hq].view(np.float32).reshape(n, spec.hq)
    ro_p, rl_p, _, _ = oracle.split_decode(f64(inp["q"]), f64(inp["k_cache"]), f64(inp["v_cache"]),
                                           inp["page_table"], inp["kv_lens"], inp["sinks"], spec.q_len, spec.scale,
                                           spec.kv_chunk)
    assert_close(o_p.astype(np.float64), l_p.astype(np.float64), ro_p, rl_p, "partials")


def test_decode_partials_then_merge_equals_decode(amd):
    """The split-only entry point followed by attn_sink_merge_partials reproduces attn_sink_decode_paged
    bit for bit (the same kernels run), and its plan and partials match the oracle's."""
    spec = scaled(CONFIGS["verify"], kv_chunk=512, batch=5, q_len=3, kv_len=(1, 1700), hq=16, hkv=2, seed=71)
    inp = make_paged(spec)
    d = dev_paged(inp)
    out, lse = run_decode(amd, d, inp, spec)
    parts = amd.attn_sink_decode_paged_partials(d["q"], d["k"], d["v"], d["table"], d["lens"], d["sinks"],
                                                spec.q_len, inp["max_kv_len"], spec.scale, spec.causal, spec.window,
                                                spec.kv_chunk)
    out2, lse2 = amd.attn_sink_merge_partials(parts["o_partial"], parts["lse_partial"], parts["partial_indptr"])
    torch.cuda.synchronize()
    assert np.array_equal(out_f64(out2), out) and np.array_equal(lse2.cpu().numpy().astype(np.float64), lse)
    exp_counts, exp_indptr = oracle.plan_chunks(inp["kv_lens"], spec.q_len, spec.kv_chunk)
    assert parts["chunk_counts"].cpu().numpy().tolist() == exp_counts
    assert parts["partial_indptr"].cpu().numpy().tolist() == exp_indptr
    n = exp_indptr[-1]
    ro_p, rl_p, _, _ = oracle.split_decode(f64(inp["q"]), f64(inp["k_cache"]), f64(inp["v_cache"]),
                                           inp["page_table"], inp["kv_lens"], inp["sinks"], spec.q_len, spec.scale,
                                           spec.kv_chunk)
    assert_close(parts["o_partial"][:n].cpu().numpy().astype(np.float64),
                 parts["lse_partial"][:n].cpu().numpy().astype(np.float64), ro_p, rl_p, "partials entry point")


def test_merge_kernel_on_oracle_partials(amd):
    spec = scaled(CONFIGS["verify"], kv_chunk=512, batch=4, kv_len=(1, 1600), hq=8, hkv=2, seed=64)
    inp = make_paged(spec, kv_lens=[1600, 2, 700, 0])
    o_p, l_p, counts, indptr = oracle.split_decode(f64(inp["q"]), f64(inp["k_cache"]), f64(inp["v_cache"]),
                                                   inp["page_table"], inp["kv_lens"], inp["sinks"], spec.q_len,
                                                   spec.scale, 256)
    out, lse = amd.attn_sink_merge_partials(torch.from_numpy(o_p.astype(np.float32)).to(DEV),
                                            torch.from_numpy(l_p.astype(np.float32)).to(DEV),
                                            torch.tensor(indptr, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    ro, rl = oracle_decode(inp, spec)
    assert_close(out_f64(out), lse.cpu().numpy().astype(np.float64), ro, rl, "merge on oracle partials")


def test_merge_all_empty_rows(amd):
    o = torch.ones(3, 4, 64, device=DEV)
    l = torch.full((3, 4), float("-inf"), device=DEV)
    indptr = torch.tensor([0, 2, 2, 3], dtype=torch.int32, device=DEV)
    out, lse = amd.attn_sink_merge_partials(o, l, indptr)
    torch.cuda.synchronize()
    assert torch.all(out.float() == 0) and torch.all(torch.isneginf(lse))


def test_merge_ignores_the_output_of_empty_partials(amd):
    # row 0: a live partial and an empty one whose o is NaN; row 1: only the NaN-o empty one
    o = torch.empty(3, 2, 64, device=DEV)
    o[0] = torch.linspace(-1, 1, 64, device=DEV)
    o[1:] = float("nan")
    l = torch.tensor([[0.5, -1.0], [float("-inf"), float("-inf")], [float("-inf"), float("nan")]], device=DEV)
    indptr = torch.tensor([0, 2, 3], dtype=torch.int32, device=DEV)
    out, lse = amd.attn_sink_merge_partials(o, l, indptr)
    torch.cuda.synchronize()
    ref = o[0].to(torch.bfloat16)
    assert torch.equal(out[0], ref)
    assert torch.allclose(lse[0], l[0], atol=1e-6, rtol=0)
    assert torch.all(out[1].float() == 0) and torch.all(torch.isneginf(lse[1]))


def test_page_permutation_bit_identical(amd):
    spec = scaled(CONFIGS["verify"], kv_chunk=512, batch=4, kv_len=(50, 1200), hq=16, hkv=2, seed=65)
    inp = make_paged(spec)
    a = run_decode(amd, dev_paged(inp), inp, spec)
    perm = np.random.default_rng(3).permutation(inp["num_pages"])
    inv = np.argsort(perm)
    inp2 = dict(inp)
    inp2["k_cache"], inp2["v_cache"] = inp["k_cache"][inv], inp["v_cache"][inv]
    inp2["page_table"] = perm[inp["page_table"]].astype(np.int32)
    b = run_decode(amd, dev_paged(inp2), inp2, spec)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_chunk_size_invariance(amd):
    spec = scaled(CONFIGS["paged_decode"], batch=4, kv_len=(1000, 5000), hq=16, hkv=2, seed=66)
    inp = make_paged(spec)
    d = dev_paged(inp)
    ro, rl = oracle_decode(inp, spec)
    for chunk in (128, 512, 2048, 0):
        out, lse = run_decode(amd, d, inp, spec, chunk=chunk)
        assert_close(out, lse, ro, rl, f"chunk {chunk}")


def test_gqa_matches_repeated_mha(amd):
    spec = scaled(CONFIGS["paged_decode"], batch=3, kv_len=(100, 900), hq=16, hkv=2, seed=67)
    inp = make_paged(spec)
    a = run_decode(amd, dev_paged(inp), inp, spec)
    inp2 = dict(inp)
    inp2["k_cache"] = np.repeat(inp["k_cache"], 8, axis=1)
    inp2["v_cache"] = np.repeat(inp["v_cache"], 8, axis=1)
    b = run_decode(amd, dev_paged(inp2), inp2, scaled(spec, hkv=16))
    assert np.abs(a[0] - b[0]).max() <= 2e-2 and np.abs(a[1] - b[1]).max() <= 1e-4


def test_decode_deterministic(amd):
    spec = scaled(CONFIGS["verify"], kv_chunk=512, batch=3, kv_len=(100, 2000), hq=64, hkv=8, seed=68)
    inp = make_paged(spec)
    d = dev_paged(inp)
    a = run_decode(amd, d, inp, spec)
    b = run_decode(amd, d, inp, spec)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("name", ["paged_decode", "verify"])
def test_decode_full_size(amd, name):
    spec = CONFIGS[name]
    inp = make_paged(spec)
    out, lse = run_decode(amd, dev_paged(inp), inp, spec)
    seqs = list(range(spec.batch)) if name == "paged_decode" else [0, 1, 7, 19, 31]
    ro, rl = oracle_decode(inp, spec, seqs=seqs)
    assert_close(out, lse, ro, rl, name)


# -------------------------------------------------------------------------------------------
# draft-tree verification
# -------------------------------------------------------------------------------------------
def run_tree(amd, d, inp, spec, trees, chunk=None, window=None):
    out, lse = amd.attn_sink_decode_paged_tree(d["q"], d["k"], d["v"], d["table"], d["lens"],
                                               torch.from_numpy(trees).to(DEV), d["sinks"], spec.q_len,
                                               inp["max_kv_len"], spec.scale, spec.window if window is None else window,
                                               spec.kv_chunk if chunk is None else chunk)
    torch.cuda.synchronize()
    return out_f64(out), lse.cpu().numpy().astype(np.float64)


def oracle_tree(inp, spec, trees, seqs=None, window=None):
    return oracle.decode_paged_tree(f64(inp["q"]), f64(inp["k_cache"]), f64(inp["v_cache"]), inp["page_table"],
                                    inp["kv_lens"], trees, inp["sinks"], spec.q_len, spec.scale,
                                    spec.window if window is None else window, seqs=seqs)


@pytest.mark.parametrize("q_len,hq,hkv,chunk,window", [(8, 64, 8, 512, 0), (8, 16, 2, 64, 0), (5, 16, 2, 2048, 0),
                                                       (3, 8, 1, 128, 0), (8, 8, 8, 512, 40), (2, 32, 8, 0, 0)])
def test_tree_verify_small(amd, q_len, hq, hkv, chunk, window):
    spec = scaled(CONFIGS["tree_verify"], batch=5, q_len=q_len, kv_len=(q_len, 1500), hq=hq, hkv=hkv, kv_chunk=chunk,
                  window=window, seed=90 + q_len + hq)
    inp = make_paged(spec)
    trees = make_tree_masks(spec)
    out, lse = run_tree(amd, dev_paged(inp), inp, spec, trees)
    ro, rl = oracle_tree(inp, spec, trees)
    assert_close(out, lse, ro, rl, f"tree q_len={q_len} hq={hq} hkv={hkv} chunk={chunk} window={window}")


def test_tree_chain_is_bit_identical_to_causal_verify(amd):
    spec = scaled(CONFIGS["verify"], batch=6, kv_len=(5, 3000), hq=64, hkv=8, kv_chunk=512, seed=97)
    inp = make_paged(spec)
    d = dev_paged(inp)
    chain = np.tile((1 << (np.arange(spec.q_len) + 1)) - 1, spec.batch).astype(np.int32)
    a = run_decode(amd, d, inp, spec)
    b = run_tree(amd, d, inp, spec, chain)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_tree_partials_then_merge_equals_tree_call(amd):
    """The tree split-only entry point followed by attn_sink_merge_partials reproduces
    attn_sink_decode_paged_tree bit for bit (the same kernels run); the plan matches the oracle's."""
    spec = scaled(CONFIGS["tree_verify"], batch=5, kv_len=(8, 1700), hq=16, hkv=2, kv_chunk=256, seed=96)
    inp = make_paged(spec)
    d = dev_paged(inp)
    trees = make_tree_masks(spec)
    out, lse = run_tree(amd, d, inp, spec, trees)
    parts = amd.attn_sink_decode_paged_tree_partials(d["q"], d["k"], d["v"], d["table"], d["lens"],
                                                     torch.from_numpy(trees).to(DEV), d["sinks"], spec.q_len,
                                                     inp["max_kv_len"], spec.scale, spec.window, spec.kv_chunk)
    out2, lse2 = amd.attn_sink_merge_partials(parts["o_partial"], parts["lse_partial"], parts["partial_indptr"])
    torch.cuda.synchronize()
    assert np.array_equal(out_f64(out2), out) and np.array_equal(lse2.cpu().numpy().astype(np.float64), lse)
    exp_counts, exp_indptr = oracle.plan_chunks(inp["kv_lens"], spec.q_len, spec.kv_chunk)
    assert parts["chunk_counts"].cpu().numpy().tolist() == exp_counts
    assert parts["partial_indptr"].cpu().numpy().tolist() == exp_indptr


def test_tree_edge_bitmaps(amd):
    # empty bitmaps (prefix only), all bits (every draft token), bits past q_len (ignored),
    # sequences no longer than the draft block
    spec = scaled(CONFIGS["tree_verify"], batch=4, q_len=6, kv_len=(6, 700), hq=16, hkv=2, kv_chunk=256, seed=98)
    inp = make_paged(spec, kv_lens=[6, 7, 300, 700])
    q = spec.q_len
    for trees in (np.zeros(4 * q, np.int32), np.full(4 * q, (1 << q) - 1, np.int32),
                  (make_tree_masks(spec) | np.int32(-(1 << q))).astype(np.int32)):
        out, lse = run_tree(amd, dev_paged(inp), inp, spec, trees)
        ro, rl = oracle_tree(inp, spec, trees & ((1 << q) - 1))
        assert_close(out, lse, ro, rl, "tree edge bitmaps")


def test_tree_verify_full_size_sampled(amd):
    spec = CONFIGS["tree_verify"]
    inp = make_paged(spec)
    trees = make_tree_masks(spec)
    out, lse = run_tree(amd, dev_paged(inp), inp, spec, trees)
    ro, rl = oracle_tree(inp, spec, trees, seqs=[0, 1, 13, 31])
    assert_close(out, lse, ro, rl, "tree_verify")

# -------------------------------------------------------------------------------------------
# YaRN rotary encoding + append of new tokens into the paged cache
# -------------------------------------------------------------------------------------------
ROPE = dict(rope_theta=150000.0, yarn_factor=32.0, yarn_original_len=4096, yarn_alpha=1.0, yarn_beta=32.0)


def run_rope(amd, inp, k_new, v_new, rope=ROPE, in_place=False):
    kc, vc = tbits(inp["k_cache"]), tbits(inp["v_cache"])
    q = tbits(inp["q"])
    q_out = amd.attn_sink_rope_append(q, tbits(k_new), tbits(v_new), torch.from_numpy(inp["cu_seqlens_q"]).to(DEV),
                                      torch.from_numpy(inp["kv_lens"]).to(DEV),
                                      torch.from_numpy(inp["page_table"]).to(DEV), kc, vc, inp["max_q"],
                                      inp["max_kv_len"], q_out=q if in_place else None, **rope)
    torch.cuda.synchronize()
    bits = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
    return bits(q_out), bits(kc), bits(vc)


def oracle_rope(inp, k_new, v_new, rope=ROPE):
    freqs, m = oracle.yarn_frequencies(64, rope["rope_theta"], rope["yarn_factor"], rope["yarn_original_len"],
                                       rope["yarn_alpha"], rope["yarn_beta"], ramp=rope.get("yarn_ramp", "turns"))
    return oracle.rope_append(f64(inp["q"]), f64(k_new), f64(v_new), inp["cu_seqlens_q"], inp["kv_lens"],
                              inp["page_table"], f64(inp["k_cache"]), f64(inp["v_cache"]), freqs, m)


def assert_bf16_close(got_bits, ref, what):
    got = f64(got_bits)
    excess = np.abs(got - ref) - (ATOL + RTOL * np.abs(ref))
    assert excess.max() <= 0, f"{what}: max excess {excess.max():.3e}"


@pytest.mark.parametrize("hq,hkv,page_size,rope", [
    (64, 8, 16, ROPE), (8, 8, 64, ROPE), (12, 3, 256, dict(ROPE, yarn_factor=1.0)),
    (64, 8, 16, dict(ROPE, yarn_ramp="index")), (8, 2, 32, dict(ROPE, yarn_ramp="index", yarn_alpha=2.0)),
    (16, 2, 32, dict(ROPE, rope_theta=10000.0, yarn_factor=4.0, yarn_original_len=2048))])
def test_rope_append(amd, hq, hkv, page_size, rope):
    spec = scaled(CONFIGS["chunked_prefill"], batch=4, q_len=(1, 300), ctx_len=(0, 9000), hq=hq, hkv=hkv,
                  page_size=page_size, seed=hq + page_size)
    inp = make_paged_prefill(spec, q_lens=[1, 300, 0, 77])
    T = int(inp["cu_seqlens_q"][-1])
    rng = np.random.default_rng(7)
    from workloads import bf16_round_bits
    k_new = bf16_round_bits(rng.standard_normal((T, hkv, 64)).astype(np.float32))
    v_new = bf16_round_bits(rng.standard_normal((T, hkv, 64)).astype(np.float32))
    q_out, kc, vc = run_rope(amd, inp, k_new, v_new, rope)
    rq, rk, rv = oracle_rope(inp, k_new, v_new, rope)
    assert_bf16_close(q_out, rq, "rotated q")
    assert_bf16_close(kc, rk, "k cache")
    # V is copied: bit-exact; every slot no new token owns is unchanged (bit-exact too)
    assert np.array_equal(f64(vc), rv)
    P = page_size
    new = np.zeros((inp["k_cache"].shape[0], P), dtype=bool)
    for b, L in enumerate(inp["kv_lens"]):
        n = int(inp["cu_seqlens_q"][b + 1] - inp["cu_seqlens_q"][b])
        for p in range(int(L) - n, int(L)):
            new[inp["page_table"][b, p // P], p % P] = True
    same = lambda a, b: np.array_equal(np.transpose(a, (0, 2, 1, 3))[~new], np.transpose(b, (0, 2, 1, 3))[~new])
    assert same(kc, inp["k_cache"]) and same(vc, inp["v_cache"])


def test_rope_append_in_place_and_full_size(amd):
    spec = CONFIGS["chunked_prefill"]
    inp = make_paged_prefill(spec)
    T = int(inp["cu_seqlens_q"][-1])
    rng = np.random.default_rng(8)
    from workloads import bf16_round_bits
    k_new = bf16_round_bits(rng.standard_normal((T, spec.hkv, 64)).astype(np.float32))
    v_new = bf16_round_bits(rng.standard_normal((T, spec.hkv, 64)).astype(np.float32))
    q_out, kc, vc = run_rope(amd, inp, k_new, v_new, in_place=True)
    rq, rk, rv = oracle_rope(inp, k_new, v_new)
    assert_bf16_close(q_out, rq, "rotated q (in place)")
    assert_bf16_close(kc, rk, "k cache")
    assert np.array_equal(f64(vc), rv)

# -------------------------------------------------------------------------------------------
# graph capture: launches depend on host scalars only, so calls can be captured and replayed
# -------------------------------------------------------------------------------------------
def test_graph_capture_replays_match_eager(amd):
    spec = scaled(CONFIGS["verify"], kv_chunk=512, batch=4, kv_len=(100, 1500), hq=16, hkv=2, seed=69)
    inp = make_paged(spec)
    d = dev_paged(inp)
    need = amd.attn_sink_decode_workspace_size(4, spec.q_len, inp["max_kv_len"], spec.hq, 64, spec.kv_chunk)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    out = torch.empty_like(d["q"])
    lse = torch.empty(d["q"].shape[0], spec.hq, device=DEV)
    pspec = scaled(CONFIGS["causal_prefill"], batch=2, hq=8, hkv=2, seed=70)
    pin = make_varlen(pspec, seqlens=[200, 77])
    pq, pk, pv = tbits(pin["q"]), tbits(pin["k"]), tbits(pin["v"])
    cu = torch.from_numpy(pin["cu_seqlens"]).to(DEV)
    ps = torch.from_numpy(pin["sinks"]).to(DEV)
    pout = torch.empty_like(pq)
    plse = torch.empty(pq.shape[0], pspec.hq, device=DEV)

    def step():
        amd.attn_sink_decode_paged(d["q"], d["k"], d["v"], d["table"], d["lens"], d["sinks"], spec.q_len,
                                   inp["max_kv_len"], spec.scale, True, 0, spec.kv_chunk, workspace=ws, out=out,
                                   lse=lse)
        amd.attn_sink_prefill(pq, pk, pv, ps, cu, cu, 200, 200, pspec.scale, True, 0, out=pout, lse=plse)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out, lse, pout, plse)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    scratch = torch.randn(512, 512, device=DEV)
    for rep in range(3):
        for t in (out, lse, pout, plse):
            t.zero_()
        scratch = scratch @ scratch.T / 512.0          # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((out, lse, pout, plse), ref):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b), f"replay {rep}"


def test_decode_with_the_planned_chunk(amd):
    """The planner's chunk (asked of the device: workgroups = 0) is a valid kv_chunk, and a decode
    call with it matches the oracle."""
    spec = scaled(CONFIGS["verify"], batch=6, q_len=5, kv_len=(1, 3000), hq=16, hkv=2, seed=72)
    inp = make_paged(spec)
    chunk = amd.attn_sink_decode_plan_chunk(inp["kv_lens"], spec.q_len, spec.hq, spec.hkv, spec.page_size)
    assert chunk % 64 == 0 and chunk % spec.page_size == 0 and chunk >= 256
    out, lse = run_decode(amd, dev_paged(inp), inp, spec, chunk=chunk)
    ro, rl = oracle_decode(inp, spec)
    assert_close(out, lse, ro, rl, f"planned chunk {chunk}")
