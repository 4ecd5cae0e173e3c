"""GPU parity at the sink's edge cases and on whole blocks of the full-size prefill workloads.

The split-KV decode path seeds the running maximum with the sink only in chunk 0, wave 0
("GPT-OSS on Day 0", section "Attention sinks"), moves the maximum lazily and folds four
wave states per chunk; the prefill kernels guard a lazy maximum with the row sum. These
cases drive those paths with sinks that dominate every key (+20), vanish (-20), are
disabled for some heads (-inf) next to finite ones, and with windows that leave chunk 0
without a visible key (the sink must still be counted exactly once).

Bar: bf16 out within 1e-2 + 1e-2 |ref|, lse within 1e-3, as every parity test.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from workloads import CONFIGS, bf16_bits_to_f32, make_paged, make_paged_prefill, make_tree_masks, make_varlen, scaled  # noqa: E402

pytestmark = pytest.mark.gpu

ATOL, RTOL, LSE_TOL = 1e-2, 1e-2, 1e-3
DEV = "cuda:0"
EXTREME = np.array([-np.inf, 0.0, 20.0, -20.0, 3.0, -np.inf, 8.0, 1.0], dtype=np.float32)


def extreme_sinks(hq):
    return np.resize(EXTREME, hq).astype(np.float32)


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


def out_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def assert_close(out, lse, ro, rl, what):
    sel = ~np.isnan(rl)
    assert sel.any(), f"{what}: nothing compared"
    o, r = out[sel], ro[sel]
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    excess = np.abs(o - r) - (ATOL + RTOL * np.abs(r))
    assert excess.max() <= 0, f"{what}: out max excess {excess.max():.3e} (max err {np.abs(o - r).max():.3e})"
    if lse is not None:
        l, rr = lse[sel], rl[sel]
        inf = np.isinf(rr)
        assert np.array_equal(np.isinf(l), inf) and np.array_equal(l[inf], rr[inf]), f"{what}: lse inf pattern"
        if (~inf).any():
            err = np.abs(l[~inf] - rr[~inf]).max()
            assert err <= LSE_TOL, f"{what}: lse max err {err:.3e}"


# -------------------------------------------------------------------------------------------
# split-KV decode, verify and tree verification
# -------------------------------------------------------------------------------------------
def dev_paged(inp):
    return dict(q=tbits(inp["q"]), k=tbits(inp["k_cache"]), v=tbits(inp["v_cache"]),
                table=torch.from_numpy(inp["page_table"]).to(DEV), lens=torch.from_numpy(inp["kv_lens"]).to(DEV),
                sinks=torch.from_numpy(inp["sinks"]).to(DEV))


def run_decode(amd, inp, spec, window=None, chunk=None):
    d = dev_paged(inp)
    out, lse = amd.attn_sink_decode_paged(d["q"], d["k"], d["v"], d["table"], d["lens"], d["sinks"], spec.q_len,
                                          inp["max_kv_len"], spec.scale, spec.causal,
                                          spec.window if window is None else window,
                                          spec.kv_chunk if chunk is None else chunk)
    torch.cuda.synchronize()
    return out_f64(out), lse.cpu().numpy().astype(np.float64)


def oracle_decode(inp, spec, window=None):
    return oracle.decode_paged(f64(inp["q"]), f64(inp["k_cache"]), f64(inp["v_cache"]), inp["page_table"],
                               inp["kv_lens"], inp["sinks"], spec.q_len, spec.scale, spec.causal,
                               spec.window if window is None else window)


@pytest.mark.parametrize("q_len,hq,hkv", [(1, 16, 2), (5, 16, 2), (1, 64, 8), (5, 64, 8), (3, 8, 8)])
@pytest.mark.parametrize("chunk", [512, 64])
def test_decode_extreme_sinks_multi_chunk(amd, q_len, hq, hkv, chunk):
    """Mixed per-head sinks (-inf next to finite, +20 dominating, -20 vanishing) over several
    chunks; the plan's partials are checked too (chunk 0 alone carries the sink)."""
    spec = scaled(CONFIGS["verify"], batch=5, q_len=q_len, kv_len=(q_len, 1500), hq=hq, hkv=hkv, kv_chunk=chunk,
                  seed=300 + q_len + hq + chunk)
    inp = make_paged(spec, kv_lens=[1500, 513, 40, max(q_len, 5), 1100])
    inp["sinks"] = extreme_sinks(hq)
    out, lse = run_decode(amd, inp, spec)
    ro, rl = oracle_decode(inp, spec)
    assert_close(out, lse, ro, rl, f"decode extreme sinks q_len={q_len} G={hq // hkv} chunk={chunk}")
    d = dev_paged(inp)
    parts = amd.attn_sink_decode_paged_partials(d["q"], d["k"], d["v"], d["table"], d["lens"], d["sinks"], q_len,
                                                inp["max_kv_len"], spec.scale, True, 0, chunk)
    torch.cuda.synchronize()
    ro_p, rl_p, counts, indptr = oracle.split_decode(f64(inp["q"]), f64(inp["k_cache"]), f64(inp["v_cache"]),
                                                     inp["page_table"], inp["kv_lens"], inp["sinks"], q_len,
                                                     spec.scale, chunk)
    n = indptr[-1]
    assert parts["partial_indptr"].cpu().numpy().tolist() == indptr
    lp = parts["lse_partial"][:n].cpu().numpy().astype(np.float64)
    op = parts["o_partial"][:n].cpu().numpy().astype(np.float64)
    # partials that saw nothing (a -inf sink outside chunk 0 never happens here; masked chunks
    # do with q_len > 1 only at the tail) carry lse -inf and an o of 0
    assert_close(op, lp, ro_p, rl_p, "extreme-sink partials")


@pytest.mark.parametrize("q_len", [1, 5])
@pytest.mark.parametrize("window", [100, 1])
def test_decode_window_leaves_chunk0_empty(amd, q_len, window):
    """The window ends far past chunk 0, which then has no visible key: chunk 0 must still
    emit the sink (lse = sink, o = 0) and later chunks must not count it."""
    spec = scaled(CONFIGS["verify"], batch=4, q_len=q_len, kv_len=(600, 2000), hq=16, hkv=2, kv_chunk=512,
                  window=window, seed=310 + q_len + window)
    inp = make_paged(spec, kv_lens=[1500, 2000, 600, 1025])
    inp["sinks"] = extreme_sinks(16)
    out, lse = run_decode(amd, inp, spec)
    ro, rl = oracle_decode(inp, spec)
    assert_close(out, lse, ro, rl, f"window {window} chunk 0 empty q_len={q_len}")
    # and the same inputs with ordinary sinks
    inp["sinks"] = (2.0 * np.random.default_rng(9).standard_normal(16)).astype(np.float32)
    out, lse = run_decode(amd, inp, spec)
    ro, rl = oracle_decode(inp, spec)
    assert_close(out, lse, ro, rl, f"window {window} chunk 0 empty q_len={q_len} N(0,2) sinks")


@pytest.mark.parametrize("q_len", [1, 5])
def test_decode_sink_dominates_every_key(amd, q_len):
    """Sinks far above every score (+20 and +30): out is tiny and lse is the sink's, for short
    sequences and for one spanning several chunks."""
    spec = scaled(CONFIGS["verify"], batch=4, q_len=q_len, kv_len=(q_len, 1400), hq=16, hkv=2, kv_chunk=512,
                  seed=320 + q_len)
    inp = make_paged(spec, kv_lens=[max(q_len, 3), 17, 1400, 700])
    inp["sinks"] = np.resize(np.array([20.0, 30.0], dtype=np.float32), 16)
    out, lse = run_decode(amd, inp, spec)
    ro, rl = oracle_decode(inp, spec)
    assert_close(out, lse, ro, rl, f"dominant sinks q_len={q_len}")
    assert np.abs(out).max() < 1e-3


@pytest.mark.parametrize("q_len,hq,hkv,chunk,window", [(8, 64, 8, 512, 0), (8, 16, 2, 64, 0), (5, 16, 2, 2048, 0),
                                                       (6, 8, 1, 512, 100)])
def test_tree_verify_extreme_sinks(amd, q_len, hq, hkv, chunk, window):
    spec = scaled(CONFIGS["tree_verify"], batch=5, q_len=q_len, kv_len=(q_len, 1500), hq=hq, hkv=hkv,
                  kv_chunk=chunk, window=window, seed=330 + q_len + hq)
    inp = make_paged(spec, kv_lens=[1500, 700, q_len, 1025, 60])
    inp["sinks"] = extreme_sinks(hq)
    trees = make_tree_masks(spec)
    d = dev_paged(inp)
    out, lse = amd.attn_sink_decode_paged_tree(d["q"], d["k"], d["v"], d["table"], d["lens"],
                                               torch.from_numpy(trees).to(DEV), d["sinks"], q_len, inp["max_kv_len"],
                                               spec.scale, window, chunk)
    torch.cuda.synchronize()
    ro, rl = oracle.decode_paged_tree(f64(inp["q"]), f64(inp["k_cache"]), f64(inp["v_cache"]), inp["page_table"],
                                      inp["kv_lens"], trees, inp["sinks"], q_len, spec.scale, window)
    assert_close(out_f64(out), lse.cpu().numpy().astype(np.float64), ro, rl,
                 f"tree extreme sinks q_len={q_len} hq={hq} chunk={chunk} window={window}")


# -------------------------------------------------------------------------------------------
# prefill: the 8-wave kernel (2048+ tokens, no window) with extreme sinks
# -------------------------------------------------------------------------------------------
def run_prefill(amd, inp, spec):
    cu = torch.from_numpy(inp["cu_seqlens"]).to(DEV)
    out, lse = amd.attn_sink_prefill(tbits(inp["q"]), tbits(inp["k"]), tbits(inp["v"]),
                                     torch.from_numpy(inp["sinks"]).to(DEV), cu, cu, inp["max_seqlen"],
                                     inp["max_seqlen"], spec.scale, spec.causal, spec.window)
    torch.cuda.synchronize()
    return out_f64(out), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("hq,hkv", [(8, 1), (16, 2), (16, 16)])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_long_extreme_sinks(amd, hq, hkv, causal):
    spec = scaled(CONFIGS["causal_prefill"], batch=3, hq=hq, hkv=hkv, causal=causal, seed=340 + hq + causal)
    inp = make_varlen(spec, seqlens=[2100, 77, 2048 + 37])
    inp["sinks"] = extreme_sinks(hq)
    out, lse = run_prefill(amd, inp, spec)
    rows = {0: list(range(0, 70)) + list(range(1000, 1064)) + list(range(2030, 2100)),
            1: list(range(77)),
            2: list(range(0, 64)) + list(range(2040, 2085))}
    ro, rl = oracle.prefill_varlen(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), inp["cu_seqlens"],
                                   inp["cu_seqlens"], inp["sinks"], spec.scale, causal, 0, seqs=list(rows), rows=rows)
    assert_close(out, lse, ro, rl, f"long prefill extreme sinks hq={hq} hkv={hkv} causal={causal}")


@pytest.mark.parametrize("window", [128, 37])
def test_prefill_window_extreme_sinks(amd, window):
    spec = scaled(CONFIGS["window_prefill"], batch=3, hq=16, hkv=2, window=window, seed=350 + window)
    inp = make_varlen(spec, seqlens=[700, 3, 300])
    inp["sinks"] = extreme_sinks(16)
    out, lse = run_prefill(amd, inp, spec)
    ro, rl = oracle.prefill_varlen(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), inp["cu_seqlens"],
                                   inp["cu_seqlens"], inp["sinks"], spec.scale, True, window)
    assert_close(out, lse, ro, rl, f"window {window} extreme sinks")


# -------------------------------------------------------------------------------------------
# full-size prefill workloads: one whole 64-token block per sequence, every head
# -------------------------------------------------------------------------------------------
def block_rows(n_seqs, lq, salt):
    """One 64-token block per sequence: the first, the last and spread blocks in between."""
    n_blk = (lq + 63) // 64
    out = {}
    for b in range(n_seqs):
        blk = 0 if b == 0 else (n_blk - 1 if b == n_seqs - 1 else (b * 17 + salt) % n_blk)
        out[b] = list(range(64 * blk, min(64 * blk + 64, lq)))
    return out


@pytest.mark.parametrize("name", ["causal_prefill", "window_prefill"])
def test_prefill_full_size_whole_blocks(amd, name):
    spec = CONFIGS[name]
    inp = make_varlen(spec)
    out, lse = run_prefill(amd, inp, spec)
    rows = block_rows(spec.batch, 4096, 5)
    ro, rl = oracle.prefill_varlen(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), inp["cu_seqlens"],
                                   inp["cu_seqlens"], inp["sinks"], spec.scale, spec.causal, spec.window,
                                   seqs=list(rows), rows=rows)
    assert int((~np.isnan(rl)).sum()) == spec.batch * 64 * spec.hq
    assert_close(out, lse, ro, rl, f"{name} whole blocks")


def test_chunked_prefill_full_size_whole_blocks(amd):
    spec = CONFIGS["chunked_prefill"]
    inp = make_paged_prefill(spec)
    out, lse = amd.attn_sink_prefill_paged(
        tbits(inp["q"]), tbits(inp["k_cache"]), tbits(inp["v_cache"]), torch.from_numpy(inp["page_table"]).to(DEV),
        torch.from_numpy(inp["cu_seqlens_q"]).to(DEV), torch.from_numpy(inp["kv_lens"]).to(DEV),
        torch.from_numpy(inp["sinks"]).to(DEV), inp["max_q"], inp["max_kv_len"], spec.scale, spec.causal, spec.window)
    torch.cuda.synchronize()
    rows = block_rows(spec.batch, 2048, 3)
    ro, rl = oracle.prefill_paged(f64(inp["q"]), f64(inp["k_cache"]), f64(inp["v_cache"]), inp["page_table"],
                                  inp["cu_seqlens_q"], inp["kv_lens"], inp["sinks"], spec.scale, spec.causal,
                                  spec.window, seqs=list(rows), rows=rows)
    assert int((~np.isnan(rl)).sum()) == spec.batch * 64 * spec.hq
    assert_close(out_f64(out), lse.cpu().numpy().astype(np.float64), ro, rl, "chunked_prefill whole blocks")
