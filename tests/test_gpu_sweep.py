"""Seeded random sweep of the attention entry points against the fp64 oracle.

Each case draws its own shape from a per-case generator: head counts and GQA ratio, query
length, page size, split-KV chunk length, window, causal flag, draft-tree bitmaps, ragged
lengths (with empty and one-token sequences, lengths at page and chunk boundaries) and the
sinks (the workloads' normal draw, none, or a per-head mix of -inf, 0, +-20 and moderate
values). The same bar as every parity test: bf16 outputs within 1e-2 + 1e-2 |ref|, LSE within
1e-3, the -inf pattern of LSE exact. A failing case names everything it drew.

Method ("GPT-OSS on Day 0", section "Attention sinks"): softmax over the scores plus one sink
logit per head, the sink counted once per row, split-KV partials merged by log-sum-exp; tree
masks as "Accelerating Sonar through speculation" (EAGLE section) describes them; ragged and
paged inputs as in "Fast Embeddings on GPUs".
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from workloads import (CONFIGS, bf16_bits_to_f32, make_paged, make_paged_prefill, make_varlen,  # noqa: E402
                       scaled)

pytestmark = pytest.mark.gpu

ATOL, RTOL, LSE_TOL = 1e-2, 1e-2, 1e-3
DEV = "cuda:0"
EXTREME = np.array([-np.inf, 0.0, 20.0, -20.0, 3.0, -np.inf, 8.0, 1.0, -5.0, 12.0], dtype=np.float32)


@pytest.fixture(scope="module")
def amd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_attention_sinks_sink_amd as amd
    return amd


def tbits(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def f64(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


def out_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


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


def draw_heads(rng, max_cols=None, q_len=1):
    """(hq, hkv): 1..4 KV heads (3 included: not a power of two), GQA ratio 1..16."""
    while True:
        hkv = int(rng.choice([1, 2, 3, 4]))
        group = int(rng.choice([1, 2, 3, 4, 8, 16]))
        if max_cols is None or q_len * group <= max_cols:
            return hkv * group, hkv


def draw_sinks(rng, hq, spec_sinks):
    """The spec's N(0, 2) draw, no sinks (None), or a per-head mix of extreme values."""
    kind = int(rng.integers(0, 3))
    if kind == 0:
        return spec_sinks, "normal"
    if kind == 1:
        return None, "none"
    return rng.permutation(np.resize(EXTREME, hq)).astype(np.float32), "extreme"


def draw_lengths(rng, n, lo, hi, boundaries):
    """Ragged lengths in [lo, hi], about a third of them on or next to a boundary value."""
    lens = rng.integers(lo, hi + 1, size=n)
    for i in range(n):
        if rng.random() < 0.35:
            lens[i] = int(np.clip(int(rng.choice(boundaries)) + int(rng.integers(-1, 2)), lo, hi))
    return [int(x) for x in lens]


# -------------------------------------------------------------------------------------------
# paged decode / verify (split-KV + merge), with and without a draft tree
# -------------------------------------------------------------------------------------------
def decode_case(seed, tree):
    rng = np.random.default_rng([7001, seed, int(tree)])
    q_len = int(rng.integers(1, 9))
    hq, hkv = draw_heads(rng, max_cols=64, q_len=q_len)
    page = int(rng.choice([16, 32, 64, 128, 256]))
    step = max(64, page)
    chunk = int(rng.choice([0, step, 2 * step, 4 * step, 2048 // step * step]))
    window = int(rng.choice([0, 0, 0, int(rng.integers(1, 40)), int(rng.integers(40, 900))]))
    causal = True if tree else bool(rng.random() < 0.85)
    batch = int(rng.integers(1, 10))
    edge = [0, q_len, page, chunk if chunk else 512, 2 * page, 1024]
    lens = draw_lengths(rng, batch, 0 if not tree else q_len, 2600, edge)
    spec = scaled(CONFIGS["verify"], batch=batch, q_len=q_len, kv_len=(0, 2600), hq=hq, hkv=hkv, page_size=page,
                  kv_chunk=chunk, window=window, causal=causal, seed=int(rng.integers(1 << 30)))
    inp = make_paged(spec, kv_lens=lens)
    sinks, sink_kind = draw_sinks(rng, hq, inp["sinks"])
    trees = None
    if tree:
        # arbitrary bitmaps over the q_len draft tokens, own bit not required
        trees = rng.integers(0, 1 << q_len, size=batch * q_len).astype(np.int32)
    what = (f"seed={seed} tree={tree} q_len={q_len} hq={hq} hkv={hkv} page={page} chunk={chunk} window={window} "
            f"causal={causal} lens={lens} sinks={sink_kind}")
    return spec, inp, sinks, trees, what


@pytest.mark.parametrize("seed", range(48))
def test_sweep_decode(amd, seed):
    spec, inp, sinks, _, what = decode_case(seed, tree=False)
    s_dev = torch.from_numpy(sinks).to(DEV) if sinks is not None else None
    out, lse = amd.attn_sink_decode_paged(tbits(inp["q"]), tbits(inp["k_cache"]), tbits(inp["v_cache"]),
                                          i32(inp["page_table"]), i32(inp["kv_lens"]), s_dev, spec.q_len,
                                          inp["max_kv_len"], spec.scale, spec.causal, spec.window, spec.kv_chunk)
    torch.cuda.synchronize()
    s = sinks if sinks is not None else np.full(spec.hq, -np.inf, dtype=np.float32)
    ro, rl = oracle.decode_paged(f64(inp["q"]), f64(inp["k_cache"]), f64(inp["v_cache"]), inp["page_table"],
                                 inp["kv_lens"], s, spec.q_len, spec.scale, spec.causal, spec.window)
    assert_close(out_f64(out), lse.cpu().numpy().astype(np.float64), ro, rl, what)


@pytest.mark.parametrize("seed", range(32))
def test_sweep_tree_verify(amd, seed):
    spec, inp, sinks, trees, what = decode_case(seed, tree=True)
    s_dev = torch.from_numpy(sinks).to(DEV) if sinks is not None else None
    out, lse = amd.attn_sink_decode_paged_tree(tbits(inp["q"]), tbits(inp["k_cache"]), tbits(inp["v_cache"]),
                                               i32(inp["page_table"]), i32(inp["kv_lens"]), i32(trees), s_dev,
                                               spec.q_len, inp["max_kv_len"], spec.scale, spec.window, spec.kv_chunk)
    torch.cuda.synchronize()
    s = sinks if sinks is not None else np.full(spec.hq, -np.inf, dtype=np.float32)
    ro, rl = oracle.decode_paged_tree(f64(inp["q"]), f64(inp["k_cache"]), f64(inp["v_cache"]), inp["page_table"],
                                      inp["kv_lens"], trees, s, spec.q_len, spec.scale, spec.window)
    assert_close(out_f64(out), lse.cpu().numpy().astype(np.float64), ro, rl, what)


# -------------------------------------------------------------------------------------------
# varlen prefill / embedding (both prefill kernels), and chunked prefill on a paged cache
# -------------------------------------------------------------------------------------------
@pytest.mark.parametrize("seed", range(40))
def test_sweep_prefill(amd, seed):
    rng = np.random.default_rng([7002, seed])
    hq, hkv = draw_heads(rng)
    causal = bool(rng.random() < 0.7)
    window = int(rng.choice([0, 0, int(rng.integers(1, 60)), int(rng.integers(60, 700))]))
    long = rng.random() < 0.25  # query ranges of 2048+ tokens (the 8-wave kernel without a window)
    batch = int(rng.integers(1, 4 if long else 7))
    hi = 2300 if long else 700
    lens = draw_lengths(rng, batch, 0, hi, [0, 1, 63, 64, 65, 128, 2048])
    if long:
        lens[0] = int(rng.integers(2048, 2301))
    spec = scaled(CONFIGS["causal_prefill"], batch=batch, hq=hq, hkv=hkv, causal=causal, window=window,
                  seqlen=(0, hi), seed=int(rng.integers(1 << 30)))
    inp = make_varlen(spec, seqlens=lens)
    sinks, sink_kind = draw_sinks(rng, hq, inp["sinks"])
    what = f"seed={seed} hq={hq} hkv={hkv} causal={causal} window={window} lens={lens} sinks={sink_kind}"
    cu = i32(inp["cu_seqlens"])
    s_dev = torch.from_numpy(sinks).to(DEV) if sinks is not None else None
    out, lse = amd.attn_sink_prefill(tbits(inp["q"]), tbits(inp["k"]), tbits(inp["v"]), s_dev, cu, cu,
                                     inp["max_seqlen"], inp["max_seqlen"], spec.scale, causal, window)
    torch.cuda.synchronize()
    s = sinks if sinks is not None else np.full(hq, -np.inf, dtype=np.float32)
    # long sequences: a whole 64-token block at the start, one in the middle and the last rows
    rows = {b: sorted({*range(0, min(64, n)), *range(max(0, n // 2 - 32), min(n, n // 2 + 32)),
                       *range(max(0, n - 64), n)}) for b, n in enumerate(lens) if n > 1024}
    ro, rl = oracle.prefill_varlen(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), inp["cu_seqlens"],
                                   inp["cu_seqlens"], s, spec.scale, causal, window, rows=rows)
    assert_close(out_f64(out), lse.cpu().numpy().astype(np.float64), ro, rl, what)


@pytest.mark.parametrize("seed", range(24))
def test_sweep_prefill_paged(amd, seed):
    rng = np.random.default_rng([7003, seed])
    hq, hkv = draw_heads(rng)
    page = int(rng.choice([16, 32, 64, 128, 256]))
    causal = bool(rng.random() < 0.8)
    window = int(rng.choice([0, 0, int(rng.integers(1, 50)), int(rng.integers(50, 600))]))
    long = rng.random() < 0.25
    batch = int(rng.integers(1, 4 if long else 6))
    q_lens = draw_lengths(rng, batch, 0, 2200 if long else 400, [0, 1, 64, page])
    if long:
        q_lens[0] = int(rng.integers(2048, 2201))
    ctx = draw_lengths(rng, batch, 0, 900, [0, page, 2 * page - 1])
    spec = scaled(CONFIGS["chunked_prefill"], batch=batch, q_len=(0, max(q_lens)), ctx_len=(0, 900), hq=hq,
                  hkv=hkv, page_size=page, causal=causal, window=window, seed=int(rng.integers(1 << 30)))
    inp = make_paged_prefill(spec, q_lens=q_lens, ctx_lens=ctx)
    sinks, sink_kind = draw_sinks(rng, hq, inp["sinks"])
    what = (f"seed={seed} hq={hq} hkv={hkv} page={page} causal={causal} window={window} q_lens={q_lens} ctx={ctx} "
            f"sinks={sink_kind}")
    s_dev = torch.from_numpy(sinks).to(DEV) if sinks is not None else None
    out, lse = amd.attn_sink_prefill_paged(tbits(inp["q"]), tbits(inp["k_cache"]), tbits(inp["v_cache"]),
                                           i32(inp["page_table"]), i32(inp["cu_seqlens_q"]), i32(inp["kv_lens"]),
                                           s_dev, inp["max_q"], inp["max_kv_len"], spec.scale, causal, window)
    torch.cuda.synchronize()
    s = sinks if sinks is not None else np.full(hq, -np.inf, dtype=np.float32)
    rows = {b: sorted({*range(0, min(64, n)), *range(max(0, n - 64), n)}) for b, n in enumerate(q_lens) if n > 1024}
    ro, rl = oracle.prefill_paged(f64(inp["q"]), f64(inp["k_cache"]), f64(inp["v_cache"]), inp["page_table"],
                                  inp["cu_seqlens_q"], inp["kv_lens"], s, spec.scale, causal, window, rows=rows)
    assert_close(out_f64(out), lse.cpu().numpy().astype(np.float64), ro, rl, what)
