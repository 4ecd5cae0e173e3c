"""GPU parity of the key-range split pass (context parallelism).

Each sequence's keys are cut into contiguous page-aligned ranges, as if every range sat on
another device. attn_sink_decode_paged_range_partials emits the chunk partials of one range
with its absolute positions; the partials of all ranges, listed per row and merged by
attn_sink_merge_partials, must match the fp64 oracle over the whole sequence ("GPT-OSS on
Day 0", section "Attention sinks": the attention is split along the sequence, partials are
combined by their log-sum-exp, and the sink counts once, in the range that holds key 0).

Bar: bf16 out within 1e-2 + 1e-2 |ref|, lse within 1e-3, as every parity test; with one range
per sequence the partials equal those of attn_sink_decode_paged_partials bit for bit.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from workloads import CONFIGS, bf16_bits_to_f32, make_paged, scaled  # noqa: E402

pytestmark = pytest.mark.gpu

ATOL, RTOL, LSE_TOL = 1e-2, 1e-2, 1e-3
DEV = "cuda:0"
EXTREME = np.array([-np.inf, 0.0, 20.0, -20.0, 3.0, -np.inf, 8.0, 1.0], dtype=np.float32)


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


def i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def assert_close(out, lse, ro, rl, what):
    o, r = out, ro
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    excess = np.abs(o - r) - (ATOL + RTOL * np.abs(r))
    assert excess.max() <= 0, f"{what}: out max excess {excess.max():.3e} (max err {np.abs(o - r).max():.3e})"
    inf = np.isinf(rl)
    assert np.array_equal(np.isinf(lse), inf) and np.array_equal(lse[inf], rl[inf]), f"{what}: lse inf pattern"
    if (~inf).any():
        err = np.abs(lse[~inf] - rl[~inf]).max()
        assert err <= LSE_TOL, f"{what}: lse max err {err:.3e}"


def cut_ranges(lens, page, n_ranges, rng):
    """Page-aligned cut points per sequence: [0, c1, ..., L]. Later ranges may be empty, the first
    is not (exactly one range of a sequence may start at key 0)."""
    cuts = []
    for L in lens:
        pages = -(-int(L) // page)
        inner = np.sort(rng.integers(1, pages + 1, size=n_ranges - 1)) * page
        c = [0] + [min(int(x), int(L)) for x in inner] + [int(L)]
        cuts.append(c)
    return cuts


def range_inputs(inp, cuts, s, page):
    """Page table, lengths and start positions of range s of every sequence."""
    table = inp["page_table"]
    lens, start = [], []
    rt = np.zeros_like(table)
    for b, c in enumerate(cuts):
        a, e = c[s], c[s + 1]
        lens.append(e - a)
        start.append(a)
        p0, p1 = a // page, -(-e // page)
        rt[b, :p1 - p0] = table[b, p0:p1]
    return rt, np.array(lens, dtype=np.int32), np.array(start, dtype=np.int32)


def merged_ranges(amd, inp, spec, cuts, n_ranges, sinks):
    """Range partials of every range, interleaved per row (range order reversed, to show the
    order does not matter), merged by the merge kernel."""
    q, kc, vc = tbits(inp["q"]), tbits(inp["k_cache"]), tbits(inp["v_cache"])
    total = i32(inp["kv_lens"])
    rows = len(inp["kv_lens"]) * spec.q_len
    o_rows = [[] for _ in range(rows)]
    l_rows = [[] for _ in range(rows)]
    for s in reversed(range(n_ranges)):
        rt, lens, start = range_inputs(inp, cuts, s, spec.page_size)
        max_len = max(int(lens.max()), 1)
        parts = amd.attn_sink_decode_paged_range_partials(q, kc, vc, i32(rt), i32(lens), i32(start), total, sinks,
                                                          spec.q_len, max_len, spec.scale, spec.causal, spec.window,
                                                          spec.kv_chunk)
        torch.cuda.synchronize()
        indptr = parts["partial_indptr"].cpu().numpy()
        o_p, l_p = parts["o_partial"].cpu(), parts["lse_partial"].cpu()
        for r in range(rows):
            o_rows[r].append(o_p[indptr[r]:indptr[r + 1]])
            l_rows[r].append(l_p[indptr[r]:indptr[r + 1]])
    counts = [sum(x.shape[0] for x in o_rows[r]) for r in range(rows)]
    indptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    o_all = torch.cat([torch.cat(o_rows[r]) for r in range(rows)]).to(DEV)
    l_all = torch.cat([torch.cat(l_rows[r]) for r in range(rows)]).to(DEV)
    out, lse = amd.attn_sink_merge_partials(o_all, l_all, i32(indptr))
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("q_len,window,n_ranges,seed", [(1, 0, 3, 81), (5, 0, 2, 82), (5, 100, 3, 83),
                                                        (3, 1, 4, 84), (8, 0, 3, 85), (1, 700, 2, 86)])
def test_range_partials_merge_to_the_whole_sequence(amd, q_len, window, n_ranges, seed):
    spec = scaled(CONFIGS["verify"], kv_chunk=256, batch=6, q_len=q_len, kv_len=(1, 1500), hq=16, hkv=2,
                  window=window, seed=seed)
    # a length-1 sequence, one shorter than a page, and ones whose draft block straddles a cut
    inp = make_paged(spec, kv_lens=[1500, 1, 13, 1025, 640, 777])
    inp["sinks"] = np.resize(EXTREME, spec.hq).astype(np.float32)
    rng = np.random.default_rng(seed)
    cuts = cut_ranges(inp["kv_lens"], spec.page_size, n_ranges, rng)
    # sequence 3 (1025 keys): a cut at key 1024 splits the last q_len positions between two ranges
    cuts[3] = {2: [0, 1024, 1025], 3: [0, 512, 1024, 1025], 4: [0, 512, 1024, 1024, 1025]}[n_ranges]
    sinks = torch.from_numpy(inp["sinks"]).to(DEV)
    out, lse = merged_ranges(amd, inp, spec, cuts, n_ranges, sinks)
    ro, rl = oracle.decode_paged(f64(inp["q"]), f64(inp["k_cache"]), f64(inp["v_cache"]), inp["page_table"],
                                 inp["kv_lens"], inp["sinks"], spec.q_len, spec.scale, spec.causal, spec.window)
    assert_close(out, lse, ro, rl, f"{n_ranges} ranges q_len={q_len} window={window}")


def test_one_range_equals_the_partials_entry_point(amd):
    spec = scaled(CONFIGS["verify"], kv_chunk=512, batch=5, q_len=5, kv_len=(1, 1700), hq=16, hkv=2, window=300,
                  seed=87)
    inp = make_paged(spec)
    q, kc, vc = tbits(inp["q"]), tbits(inp["k_cache"]), tbits(inp["v_cache"])
    table, lens, sinks = i32(inp["page_table"]), i32(inp["kv_lens"]), torch.from_numpy(inp["sinks"]).to(DEV)
    a = amd.attn_sink_decode_paged_partials(q, kc, vc, table, lens, sinks, spec.q_len, inp["max_kv_len"], spec.scale,
                                            spec.causal, spec.window, spec.kv_chunk)
    n = int(a["partial_indptr"][-1].item())
    o_a, l_a = a["o_partial"][:n].clone(), a["lse_partial"][:n].clone()
    b = amd.attn_sink_decode_paged_range_partials(q, kc, vc, table, lens, i32(np.zeros(spec.batch)), lens, sinks,
                                                  spec.q_len, inp["max_kv_len"], spec.scale, spec.causal,
                                                  spec.window, spec.kv_chunk)
    torch.cuda.synchronize()
    assert torch.equal(b["partial_indptr"], a["partial_indptr"])
    assert torch.equal(b["o_partial"][:n], o_a) and torch.equal(b["lse_partial"][:n], l_a)


def test_range_without_key_zero_leaves_the_sink_out(amd):
    """A range that does not start at key 0 never counts the sink: with every key of the range
    masked by the window its partials are empty (lse -inf), whatever the sink."""
    spec = scaled(CONFIGS["verify"], kv_chunk=512, batch=3, q_len=1, kv_len=(64, 64), hq=8, hkv=2, window=16,
                  seed=88)
    inp = make_paged(spec, kv_lens=[64, 64, 64])
    q, kc, vc = tbits(inp["q"]), tbits(inp["k_cache"]), tbits(inp["v_cache"])
    sinks = torch.full((spec.hq,), 20.0, device=DEV)
    # the range holds keys 32..95 of a 4096-key sequence: all of it is outside the 16-key window
    parts = amd.attn_sink_decode_paged_range_partials(q, kc, vc, i32(inp["page_table"]), i32(inp["kv_lens"]),
                                                      i32([32, 32, 32]), i32([4096, 4096, 4096]), sinks,
                                                      spec.q_len, 64, spec.scale, True, spec.window, spec.kv_chunk)
    torch.cuda.synchronize()
    n = int(parts["partial_indptr"][-1].item())
    assert n == 3
    assert torch.isneginf(parts["lse_partial"][:n]).all()
