"""Host-only checks of the C ABI: the library loads, exports every declared symbol, and
rejects bad arguments with the documented status codes before touching the GPU."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_sink.h")

OK, INVALID, UNSUPPORTED, WS_SMALL, HIPERR = 0, 1, 2, 3, 4
FAKE = 0x100000  # a non-NULL, 256-aligned address; never dereferenced on these paths


@pytest.fixture(scope="module")
def amd():
    from gqa_attention_sinks_sink_amd.build import LIB_PATH
    if not os.path.exists(LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    import gqa_attention_sinks_sink_amd as amd
    return amd


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_sink_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("attn_sink_prefill", "attn_sink_decode_paged", "attn_sink_merge_partials",
              "attn_sink_decode_workspace_size", "attn_sink_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol(amd):
    for name in declared_functions():
        assert hasattr(amd.lib, name), name
    nm = subprocess.run(["nm", "-D", "--defined-only", amd.lib._name], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\sT\s(\S+)", nm))
    assert set(declared_functions()) <= exported
    assert set(amd.EXPORTED_SYMBOLS) == set(declared_functions())


def test_status_strings_and_version(amd):
    assert amd.attn_sink_status_string(0) == "ok"
    assert "workspace" in amd.attn_sink_status_string(3)
    assert amd.attn_sink_status_string(99) == "unknown status"
    assert "gfx950" in amd.attn_sink_version()


def test_workspace_size_layout_and_monotone(amd):
    ws = amd.attn_sink_decode_workspace_size
    assert ws(64, 1, 8192, 64, 64, 512) == amd.decode_workspace_layout(64, 1, 8192, 64, 512)["total"]
    assert ws(32, 5, 16384, 64, 64, 512) == amd.decode_workspace_layout(32, 5, 16384, 64, 512)["total"]
    assert ws(4, 1, 100, 8, 64, 0) == amd.decode_workspace_layout(4, 1, 100, 8, 0)["total"]
    assert ws(4, 1, 100, 8, 128, 512) == 0          # unsupported head_dim
    assert ws(-1, 1, 100, 8, 64, 512) == 0
    prev = 0
    for L in (0, 1, 511, 512, 513, 4096, 9000):
        cur = ws(8, 2, L, 16, 64, 512)
        assert cur >= prev and cur % 256 == 0
        prev = cur
    assert ws(9, 2, 9000, 16, 64, 512) >= ws(8, 2, 9000, 16, 64, 512)
    assert ws(8, 3, 9000, 16, 64, 512) >= ws(8, 2, 9000, 16, 64, 512)
    assert ws(8, 2, 9000, 32, 64, 512) >= ws(8, 2, 9000, 16, 64, 512)


def _documented_layout(batch, q_len, max_kv_len, hq, kv_chunk):
    """The workspace layout as the header documents it: R = batch * q_len rows, C = max(1,
    ceil(max_kv_len / chunk)) chunks per row (chunk = kv_chunk, or one chunk when kv_chunk <= 0),
    regions indptr[R + 1], counts[R], o[R C][hq][64], lse[R C][hq], each on a 256-byte boundary."""
    up = lambda x: -(-x // 256) * 256
    R = batch * q_len
    C = 1 if kv_chunk <= 0 else max(1, -(-max_kv_len // kv_chunk))
    P = R * C
    off_counts = up(4 * (R + 1))
    off_o = off_counts + up(4 * R)
    off_lse = off_o + up(4 * P * hq * 64)
    return dict(rows=R, chunks=C, partials=P, off_indptr=0, off_counts=off_counts, off_o=off_o, off_lse=off_lse,
                total=off_lse + up(4 * P * hq))


@pytest.mark.parametrize("batch,q_len,max_kv,hq,chunk", [(64, 1, 8192, 64, 512), (32, 5, 16384, 64, 2048),
                                                          (4, 1, 100, 8, 0), (3, 8, 1, 16, 64), (0, 1, 0, 4, 512),
                                                          (7, 3, 4097, 12, 1024), (1, 1, 0, 1, 0)])
def test_workspace_layout_every_offset(amd, batch, q_len, max_kv, hq, chunk):
    got = amd.attn_sink_decode_workspace_layout(batch, q_len, max_kv, hq, 64, chunk)
    assert got == _documented_layout(batch, q_len, max_kv, hq, chunk)
    assert got["total"] == amd.attn_sink_decode_workspace_size(batch, q_len, max_kv, hq, 64, chunk)


def test_workspace_layout_errors(amd):
    with pytest.raises(amd.AttnSinkError):
        amd.attn_sink_decode_workspace_layout(4, 1, 100, 8, 128, 512)
    with pytest.raises(amd.AttnSinkError):
        amd.attn_sink_decode_workspace_layout(-1, 1, 100, 8, 64, 512)
    assert amd.lib.attn_sink_decode_workspace_layout(4, 1, 100, 8, 64, 512, None) == INVALID


def _prefill(amd, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, sinks=None, cu_q=FAKE, cu_kv=FAKE, batch=1, total_q=16, total_kv=16,
             max_q=16, max_kv=16, hq=4, hkv=1, d=64, scale=0.125, causal=1, window=0, out=FAKE, lse=None, stream=None)
    a.update(kw)
    return amd.lib.attn_sink_prefill(a["q"], a["k"], a["v"], a["sinks"], a["cu_q"], a["cu_kv"], a["batch"],
                                     a["total_q"], a["total_kv"], a["max_q"], a["max_kv"], a["hq"], a["hkv"], a["d"],
                                     a["scale"], a["causal"], a["window"], a["out"], a["lse"], a["stream"])


def _prefill_paged(amd, **kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, table=FAKE, max_pages=4, num_pages=8, cu_q=FAKE, lens=FAKE, sinks=None,
             batch=2, total_q=32, max_q=16, max_kv=64, hq=8, hkv=2, d=64, page=16, scale=0.125, causal=1, window=0,
             out=FAKE, lse=None, stream=None)
    a.update(kw)
    return amd.lib.attn_sink_prefill_paged(a["q"], a["kc"], a["vc"], a["table"], a["max_pages"], a["num_pages"],
                                           a["cu_q"], a["lens"], a["sinks"], a["batch"], a["total_q"], a["max_q"],
                                           a["max_kv"], a["hq"], a["hkv"], a["d"], a["page"], a["scale"], a["causal"],
                                           a["window"], a["out"], a["lse"], a["stream"])


def test_prefill_paged_argument_errors(amd):
    assert _prefill_paged(amd, d=128) == UNSUPPORTED
    assert _prefill_paged(amd, page=8) == UNSUPPORTED
    assert _prefill_paged(amd, page=24) == UNSUPPORTED
    assert _prefill_paged(amd, page=512) == UNSUPPORTED
    assert _prefill_paged(amd, max_q=1 << 18, hq=64, hkv=8) == UNSUPPORTED
    assert _prefill_paged(amd, hq=6, hkv=4) == INVALID
    assert _prefill_paged(amd, hkv=0) == INVALID
    assert _prefill_paged(amd, scale=0.0) == INVALID
    assert _prefill_paged(amd, scale=float("nan")) == INVALID
    assert _prefill_paged(amd, batch=-1) == INVALID
    assert _prefill_paged(amd, max_pages=0) == INVALID
    assert _prefill_paged(amd, max_pages=1 << 23, page=256) == UNSUPPORTED   # capacity 2^31 tokens
    assert _prefill_paged(amd, max_pages=(1 << 23) - 1, page=256, batch=0) == OK
    assert _prefill_paged(amd, num_pages=0) == INVALID
    for name in ("q", "kc", "vc", "table", "cu_q", "lens", "out"):
        assert _prefill_paged(amd, **{name: None}) == INVALID, name
    # nothing to do: accepted without launching anything
    assert _prefill_paged(amd, batch=0, q=None) == OK
    assert _prefill_paged(amd, total_q=0) == OK
    assert _prefill_paged(amd, max_q=0) == OK

def test_prefill_argument_errors(amd):
    assert _prefill(amd, d=128) == UNSUPPORTED
    assert _prefill(amd, hq=6, hkv=4) == INVALID
    assert _prefill(amd, hkv=0) == INVALID
    assert _prefill(amd, scale=0.0) == INVALID
    assert _prefill(amd, scale=float("nan")) == INVALID
    assert _prefill(amd, scale=float("inf")) == INVALID
    assert _prefill(amd, batch=-1) == INVALID
    assert _prefill(amd, total_q=-5) == INVALID
    assert _prefill(amd, q=None) == INVALID
    assert _prefill(amd, out=None) == INVALID
    assert _prefill(amd, cu_q=None) == INVALID
    assert _prefill(amd, k=None) == INVALID
    # one sequence's rows must span less than 2^31 bytes (32-bit offsets in the kernels)
    assert _prefill(amd, max_q=1 << 18, hq=64, hkv=8) == UNSUPPORTED
    assert _prefill(amd, max_kv=1 << 21, hq=8, hkv=8) == UNSUPPORTED
    # nothing to do: accepted without launching anything
    assert _prefill(amd, batch=0, q=None, out=None) == OK
    assert _prefill(amd, total_q=0, q=None, out=None) == OK


def _decode(amd, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, table=FAKE, max_pages=512, num_pages=100, kv_lens=FAKE, sinks=None, batch=4,
             q_len=1, max_kv=8192, hq=64, hkv=8, d=64, page=16, scale=0.125, causal=1, window=0, chunk=512,
             ws=FAKE, ws_bytes=1 << 40, out=FAKE, lse=None, stream=None)
    a.update(kw)
    return amd.lib.attn_sink_decode_paged(a["q"], a["k"], a["v"], a["table"], a["max_pages"], a["num_pages"],
                                          a["kv_lens"], a["sinks"], a["batch"], a["q_len"], a["max_kv"], a["hq"],
                                          a["hkv"], a["d"], a["page"], a["scale"], a["causal"], a["window"],
                                          a["chunk"], a["ws"], a["ws_bytes"], a["out"], a["lse"], a["stream"])


def _decode_tree(amd, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, table=FAKE, max_pages=512, num_pages=100, kv_lens=FAKE, tree=FAKE, sinks=None,
             batch=4, q_len=8, max_kv=8192, hq=64, hkv=8, d=64, page=16, scale=0.125, window=0, chunk=512,
             ws=FAKE, ws_bytes=1 << 40, out=FAKE, lse=None, stream=None)
    a.update(kw)
    return amd.lib.attn_sink_decode_paged_tree(a["q"], a["k"], a["v"], a["table"], a["max_pages"], a["num_pages"],
                                               a["kv_lens"], a["tree"], a["sinks"], a["batch"], a["q_len"],
                                               a["max_kv"], a["hq"], a["hkv"], a["d"], a["page"], a["scale"],
                                               a["window"], a["chunk"], a["ws"], a["ws_bytes"], a["out"], a["lse"],
                                               a["stream"])


def test_decode_tree_argument_errors(amd):
    assert _decode_tree(amd, tree=None) == INVALID
    assert _decode_tree(amd, d=128) == UNSUPPORTED
    assert _decode_tree(amd, q_len=9) == UNSUPPORTED
    assert _decode_tree(amd, hq=72, hkv=8) == UNSUPPORTED      # 8 x 9 columns
    assert _decode_tree(amd, page=8) == UNSUPPORTED
    assert _decode_tree(amd, chunk=100) == UNSUPPORTED
    assert _decode_tree(amd, scale=-1.0) == INVALID
    assert _decode_tree(amd, out=None) == INVALID
    assert _decode_tree(amd, ws_bytes=16) == WS_SMALL
    assert _decode_tree(amd, batch=0, tree=None) == OK        # nothing to do

def _rope(amd, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, cu_q=FAKE, lens=FAKE, table=FAKE, max_pages=64, num_pages=100, kc=FAKE, vc=FAKE,
             batch=2, total_q=32, max_q=16, max_kv=1024, hq=8, hkv=2, d=64, page=16, theta=150000.0, factor=32.0,
             orig=4096, alpha=1.0, beta=32.0, ramp=0, q_out=FAKE, stream=None)
    a.update(kw)
    return amd.lib.attn_sink_rope_append(a["q"], a["k"], a["v"], a["cu_q"], a["lens"], a["table"], a["max_pages"],
                                         a["num_pages"], a["kc"], a["vc"], a["batch"], a["total_q"], a["max_q"],
                                         a["max_kv"], a["hq"], a["hkv"], a["d"], a["page"], a["theta"], a["factor"],
                                         a["orig"], a["alpha"], a["beta"], a["ramp"], a["q_out"], a["stream"])


def test_rope_append_argument_errors(amd):
    assert _rope(amd, d=128) == UNSUPPORTED
    assert _rope(amd, page=8) == UNSUPPORTED
    assert _rope(amd, batch=70000) == UNSUPPORTED
    assert _rope(amd, theta=1.0) == INVALID
    assert _rope(amd, theta=float("nan")) == INVALID
    assert _rope(amd, factor=0.0) == INVALID
    assert _rope(amd, orig=0) == INVALID
    assert _rope(amd, alpha=32.0, beta=1.0) == INVALID
    assert _rope(amd, ramp=2) == INVALID
    assert _rope(amd, ramp=-1) == INVALID
    assert _rope(amd, ramp=1, alpha=0.0) == INVALID           # the index ramp takes ln(r / alpha)
    assert _rope(amd, ramp=1, batch=0) == OK
    assert _rope(amd, hq=6, hkv=4) == INVALID
    assert _rope(amd, max_pages=0) == INVALID
    assert _rope(amd, max_pages=1 << 27, page=16) == UNSUPPORTED              # capacity 2^31 tokens
    for name in ("q", "k", "v", "cu_q", "lens", "table", "kc", "vc", "q_out"):
        assert _rope(amd, **{name: None}) == INVALID, name
    # no YaRN scaling: original length and ramp bounds are not needed
    assert _rope(amd, factor=1.0, orig=0, alpha=5.0, beta=1.0, batch=0) == OK
    assert _rope(amd, total_q=0) == OK

def test_decode_argument_errors(amd):
    assert _decode(amd, d=128) == UNSUPPORTED
    assert _decode(amd, q_len=9) == UNSUPPORTED
    assert _decode(amd, q_len=0) == INVALID
    assert _decode(amd, hq=128, hkv=1) == UNSUPPORTED      # 128 columns per KV head
    assert _decode(amd, q_len=8, hq=72, hkv=8) == UNSUPPORTED   # 8 x 9 = 72 columns
    assert _decode(amd, page=24) == UNSUPPORTED
    assert _decode(amd, page=8) == UNSUPPORTED
    assert _decode(amd, page=512) == UNSUPPORTED
    assert _decode(amd, chunk=100) == UNSUPPORTED
    assert _decode(amd, chunk=64, page=128) == UNSUPPORTED
    assert _decode(amd, hq=60, hkv=8) == INVALID
    assert _decode(amd, scale=-1.0) == INVALID
    assert _decode(amd, num_pages=0) == INVALID
    assert _decode(amd, max_pages=0) == INVALID
    assert _decode(amd, max_pages=1 << 27, page=16) == UNSUPPORTED            # capacity 2^31 tokens
    assert _decode_tree(amd, max_pages=1 << 24, page=128) == UNSUPPORTED
    assert _decode(amd, max_kv=-1) == INVALID
    assert _decode(amd, q=None) == INVALID
    assert _decode(amd, table=None) == INVALID
    assert _decode(amd, ws=None) == INVALID
    assert _decode(amd, ws=FAKE + 16) == INVALID             # workspace must be 256-byte aligned
    need = amd.attn_sink_decode_workspace_size(4, 1, 8192, 64, 64, 512)
    assert _decode(amd, ws_bytes=need - 1) == WS_SMALL
    assert _decode(amd, ws_bytes=0) == WS_SMALL
    assert _decode(amd, batch=0, q=None, ws=None) == OK


def _decode_partials(amd, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, table=FAKE, max_pages=512, num_pages=100, kv_lens=FAKE, sinks=None, batch=4,
             q_len=1, max_kv=8192, hq=64, hkv=8, d=64, page=16, scale=0.125, causal=1, window=0, chunk=512,
             ws=FAKE, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return amd.lib.attn_sink_decode_paged_partials(a["q"], a["k"], a["v"], a["table"], a["max_pages"],
                                                   a["num_pages"], a["kv_lens"], a["sinks"], a["batch"], a["q_len"],
                                                   a["max_kv"], a["hq"], a["hkv"], a["d"], a["page"], a["scale"],
                                                   a["causal"], a["window"], a["chunk"], a["ws"], a["ws_bytes"],
                                                   a["stream"])


def test_decode_partials_argument_errors(amd):
    """The split-only entry point validates exactly like attn_sink_decode_paged (it has no out)."""
    for kw, want in [(dict(d=128), UNSUPPORTED), (dict(q_len=9), UNSUPPORTED), (dict(q_len=0), INVALID),
                     (dict(page=24), UNSUPPORTED), (dict(chunk=100), UNSUPPORTED), (dict(hq=60, hkv=8), INVALID),
                     (dict(scale=float("nan")), INVALID), (dict(q=None), INVALID), (dict(ws=None), INVALID),
                     (dict(ws=FAKE + 16), INVALID), (dict(ws_bytes=0), WS_SMALL),
                     (dict(batch=0, q=None, ws=None), OK)]:
        assert _decode_partials(amd, **kw) == want, kw
        assert _decode(amd, **kw) == want, kw


def test_merge_argument_errors(amd):
    f = amd.lib.attn_sink_merge_partials
    assert f(FAKE, FAKE, 10, FAKE, 4, 8, 128, FAKE, None, None) == UNSUPPORTED
    assert f(FAKE, FAKE, -1, FAKE, 4, 8, 64, FAKE, None, None) == INVALID
    assert f(FAKE, FAKE, 10, FAKE, -4, 8, 64, FAKE, None, None) == INVALID
    assert f(FAKE, FAKE, 10, FAKE, 4, 0, 64, FAKE, None, None) == INVALID
    assert f(FAKE, FAKE, 10, None, 4, 8, 64, FAKE, None, None) == INVALID
    assert f(None, FAKE, 10, FAKE, 4, 8, 64, FAKE, None, None) == INVALID
    assert f(FAKE, FAKE, 10, FAKE, 4, 8, 64, None, None, None) == INVALID
    assert f(None, None, 0, None, 0, 8, 64, None, None, None) == OK


def test_misaligned_tensors_are_rejected(amd):
    # bf16 rows and fp32 partials move in 16-byte pieces: pointers off a 16-byte boundary are refused
    odd = FAKE + 2
    assert _prefill(amd, q=odd) == INVALID
    assert _prefill(amd, k=odd) == INVALID
    assert _prefill(amd, out=odd) == INVALID
    assert _prefill_paged(amd, kc=odd) == INVALID
    assert _prefill_paged(amd, out=odd) == INVALID
    assert _decode(amd, q=odd) == INVALID
    assert _decode(amd, v=odd) == INVALID
    assert _decode(amd, out=odd) == INVALID
    assert _decode_tree(amd, k=odd) == INVALID
    assert _rope(amd, q=odd) == INVALID
    assert _rope(amd, vc=odd) == INVALID
    assert _rope(amd, q_out=odd) == INVALID
    f = amd.lib.attn_sink_merge_partials
    assert f(odd, FAKE, 10, FAKE, 4, 8, 64, FAKE, None, None) == INVALID
    assert f(FAKE, FAKE, 10, FAKE, 4, 8, 64, odd, None, None) == INVALID


def test_binding_refuses_cpu_tensors(amd):
    import torch
    q = torch.zeros(16, 4, 64, dtype=torch.bfloat16)
    cu = torch.tensor([0, 16], dtype=torch.int32)
    with pytest.raises((TypeError, ValueError, RuntimeError)):
        amd.attn_sink_prefill(q.float(), q, q, None, cu, cu, 16, 16)


def _noalloc(amd, **kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, table=FAKE, max_pages=64, num_pages=100, lens=FAKE, sinks=None, batch=4,
             q_len=1, max_kv=1024, hq=16, hkv=2, d=64, page=16, scale=0.125, causal=1, window=0, chunk=512, out=FAKE,
             lse=None, stream=None)
    a.update(kw)
    return amd.lib.attn_sink_decode_paged_noalloc(a["q"], a["kc"], a["vc"], a["table"], a["max_pages"],
                                                  a["num_pages"], a["lens"], a["sinks"], a["batch"], a["q_len"],
                                                  a["max_kv"], a["hq"], a["hkv"], a["d"], a["page"], a["scale"],
                                                  a["causal"], a["window"], a["chunk"], a["out"], a["lse"],
                                                  a["stream"])


def test_decode_noalloc_argument_errors(amd):
    """Every rejection happens on the host, before the scratch is looked up or anything launched."""
    cap = amd.attn_sink_decode_noalloc_capacity()
    assert cap == 64 << 20
    assert _noalloc(amd, d=128) == UNSUPPORTED
    assert _noalloc(amd, q_len=9) == UNSUPPORTED
    assert _noalloc(amd, chunk=100) == UNSUPPORTED
    assert _noalloc(amd, scale=0.0) == INVALID
    assert _noalloc(amd, out=None) == INVALID
    for name in ("q", "kc", "vc", "table", "lens"):
        assert _noalloc(amd, **{name: None}) == INVALID, name
    assert _noalloc(amd, q=FAKE + 8) == INVALID
    # beyond the scratch: the workspace these scalars need exceeds the capacity
    big = dict(batch=64, q_len=8, max_kv=131072, hq=64, hkv=8, chunk=64, max_pages=8192)
    assert amd.attn_sink_decode_workspace_size(64, 8, 131072, 64, 64, 64) > cap
    assert _noalloc(amd, **big) == WS_SMALL
    assert _noalloc(amd, batch=0) == OK


def _tree_partials(amd, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, table=FAKE, max_pages=512, num_pages=100, kv_lens=FAKE, tree=FAKE, sinks=None,
             batch=4, q_len=8, max_kv=8192, hq=64, hkv=8, d=64, page=16, scale=0.125, window=0, chunk=512,
             ws=FAKE, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return amd.lib.attn_sink_decode_paged_tree_partials(a["q"], a["k"], a["v"], a["table"], a["max_pages"],
                                                        a["num_pages"], a["kv_lens"], a["tree"], a["sinks"],
                                                        a["batch"], a["q_len"], a["max_kv"], a["hq"], a["hkv"],
                                                        a["d"], a["page"], a["scale"], a["window"], a["chunk"],
                                                        a["ws"], a["ws_bytes"], a["stream"])


def test_decode_tree_partials_argument_errors(amd):
    assert _tree_partials(amd, tree=None) == INVALID
    assert _tree_partials(amd, q_len=9) == UNSUPPORTED
    assert _tree_partials(amd, chunk=100) == UNSUPPORTED
    assert _tree_partials(amd, ws=None) == INVALID
    assert _tree_partials(amd, ws=FAKE + 16) == INVALID      # workspace not 256-byte aligned
    assert _tree_partials(amd, ws_bytes=16) == WS_SMALL
    assert _tree_partials(amd, scale=float("inf")) == INVALID
    assert _tree_partials(amd, batch=0, tree=None) == OK


def _range_partials(amd, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, table=FAKE, max_pages=512, num_pages=100, kv_lens=FAKE, start=FAKE,
             total=FAKE, sinks=None, batch=4, q_len=5, max_kv=8192, hq=64, hkv=8, d=64, page=16, scale=0.125,
             causal=1, window=0, chunk=512, ws=FAKE, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return amd.lib.attn_sink_decode_paged_range_partials(a["q"], a["k"], a["v"], a["table"], a["max_pages"],
                                                         a["num_pages"], a["kv_lens"], a["start"], a["total"],
                                                         a["sinks"], a["batch"], a["q_len"], a["max_kv"], a["hq"],
                                                         a["hkv"], a["d"], a["page"], a["scale"], a["causal"],
                                                         a["window"], a["chunk"], a["ws"], a["ws_bytes"],
                                                         a["stream"])


def test_decode_range_partials_argument_errors(amd):
    assert _range_partials(amd, start=None) == INVALID
    assert _range_partials(amd, total=None) == INVALID
    assert _range_partials(amd, q_len=9) == UNSUPPORTED
    assert _range_partials(amd, chunk=100) == UNSUPPORTED
    assert _range_partials(amd, ws=None) == INVALID
    assert _range_partials(amd, ws=FAKE + 16) == INVALID      # workspace not 256-byte aligned
    assert _range_partials(amd, ws_bytes=16) == WS_SMALL
    assert _range_partials(amd, hq=60) == INVALID             # not a multiple of hkv
    assert _range_partials(amd, batch=0, start=None, total=None) == OK


def _plan(amd, lens, q_len=5, hq=64, hkv=8, page=16, wgs=512):
    import ctypes
    import numpy as np
    out = ctypes.c_int32(-1)
    arr = np.ascontiguousarray(np.asarray(lens, dtype=np.int32))
    st = amd.lib.attn_sink_decode_plan_chunk(arr.ctypes.data if arr.size else None, int(arr.size), q_len, hq, hkv,
                                             page, wgs, ctypes.byref(out))
    return st, out.value


def _plan_model(lens, hkv, page, wgs, item_keys=1024, merge_keys=384):
    """The planner's documented rule, written out: deal (sequence, chunk, KV head) items
    round-robin to wgs workgroups, charge keys + item_keys each, add merge_keys per 16 partials
    of the sequence with the most chunks, keep the chunk with the lowest cost (ties: the longer
    chunk)."""
    step = max(256, page)
    top = max(step, -(-max([0] + list(lens)) // step) * step)
    best = None
    for c in range(step, top + 1, step):
        items = sum(max(1, -(-max(0, L) // c)) for L in lens) * hkv
        if items > 64 * wgs and c != top:
            continue
        load = [0] * wgs
        i = 0
        for L in lens:
            L = max(0, L)
            for ch in range(max(1, -(-L // c))):
                keys = max(0, min(c, L - ch * c))
                for _ in range(hkv):
                    load[i % wgs] += keys + item_keys
                    i += 1
        most = max([1] + [max(1, -(-max(0, L) // c)) for L in lens])
        w = max(load) + merge_keys * -(-most // 16)
        if best is None or w <= best[0]:
            best = (w, c)
    return best[1]


def test_plan_chunk_argument_errors(amd):
    import ctypes
    out = ctypes.c_int32(0)
    assert amd.lib.attn_sink_decode_plan_chunk(None, 3, 5, 64, 8, 16, 512, ctypes.byref(out)) == INVALID
    assert _plan(amd, [100], q_len=9)[0] == UNSUPPORTED
    assert _plan(amd, [100], page=8)[0] == UNSUPPORTED
    assert _plan(amd, [100], hq=60)[0] == INVALID
    assert amd.lib.attn_sink_decode_plan_chunk(None, 0, 5, 64, 8, 16, 512, None) == INVALID
    assert _plan(amd, []) == (OK, 256)


@pytest.mark.parametrize("seed", range(6))
def test_plan_chunk_follows_its_rule(amd, seed):
    import numpy as np
    rng = np.random.default_rng(seed)
    batch = int(rng.integers(1, 40))
    lens = rng.integers(0, 20000, size=batch).tolist()
    page = int(rng.choice([16, 64, 256]))
    hkv = int(rng.choice([1, 2, 8]))
    wgs = int(rng.choice([64, 512, 1024]))
    st, c = _plan(amd, lens, hq=hkv * 4, hkv=hkv, page=page, wgs=wgs)
    assert st == OK
    assert c % 64 == 0 and c % page == 0 and c >= 256
    assert c == _plan_model(lens, hkv, page, wgs)


def test_plan_chunk_on_the_verify_workloads(amd):
    """On the verify-shaped bench workloads the rule picks the chunk lengths that measured fastest
    on MI355X among 1024-7424 (verify 5632, 101.5 us vs 116.1 at 2048; draft trees 7168)."""
    from workloads import CONFIGS, make_paged
    for name, want in (("verify", 5632), ("tree_verify", 7168)):
        spec = CONFIGS[name]
        lens = make_paged(spec)["kv_lens"]
        assert _plan(amd, lens, q_len=spec.q_len, hq=spec.hq, hkv=spec.hkv, page=spec.page_size) == (OK, want)
