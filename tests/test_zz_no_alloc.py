"""The allocation-free decode entry point (attn_sink_decode_paged_noalloc) against the entry point
it varies (attn_sink_decode_paged): the same kernels over a scratch array inside the library in
place of a caller workspace, so the results must be identical. Two calls in a row, the second
with a smaller input (the scratch keeps the first call's contents), then the workspace entry
point again; the first call is also held to the parity bar against the oracle."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from workloads import CONFIGS, bf16_bits_to_f32, make_paged, scaled  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def amd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_attention_sinks_sink_amd as amd
    return amd


def tbits(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def dev(inp):
    return dict(q=tbits(inp["q"]), k=tbits(inp["k_cache"]), v=tbits(inp["v_cache"]),
                table=torch.from_numpy(inp["page_table"]).to(DEV), lens=torch.from_numpy(inp["kv_lens"]).to(DEV),
                sinks=torch.from_numpy(inp["sinks"]).to(DEV))


def both(amd, inp, spec):
    d = dev(inp)
    args = (d["q"], d["k"], d["v"], d["table"], d["lens"], d["sinks"], spec.q_len, inp["max_kv_len"], spec.scale,
            spec.causal, spec.window, spec.kv_chunk)
    out_na = torch.empty_like(d["q"])
    lse_na = torch.empty(d["q"].shape[0], spec.hq, dtype=torch.float32, device=DEV)
    amd.attn_sink_decode_paged_noalloc(*args, out=out_na, lse=lse_na)
    torch.cuda.synchronize()
    ref_out, ref_lse = amd.attn_sink_decode_paged(*args)
    torch.cuda.synchronize()
    return out_na, lse_na, ref_out, ref_lse


def test_noalloc_matches_workspace_entry_point_twice(amd):
    assert amd.attn_sink_decode_noalloc_capacity() == 64 << 20
    big = CONFIGS["paged_decode"]                 # the full decode batch: 16.3 MiB of scratch
    inp = make_paged(big)
    need = amd.attn_sink_decode_workspace_size(big.batch, big.q_len, inp["max_kv_len"], big.hq, 64, big.kv_chunk)
    assert 0 < need <= amd.attn_sink_decode_noalloc_capacity()
    out_na, lse_na, ref_out, ref_lse = both(amd, inp, big)
    assert torch.equal(out_na.view(torch.int16), ref_out.view(torch.int16))
    assert torch.equal(lse_na, ref_lse)
    # parity bar on sampled sequences
    f64 = lambda b: bf16_bits_to_f32(b).astype(np.float64)
    seqs = [0, 17, 63]
    ro, rl = oracle.decode_paged(f64(inp["q"]), f64(inp["k_cache"]), f64(inp["v_cache"]), inp["page_table"],
                                 inp["kv_lens"], inp["sinks"], big.q_len, big.scale, big.causal, big.window, seqs=seqs)
    sel = ~np.isnan(rl)
    got = out_na.float().cpu().numpy().astype(np.float64)[sel]
    assert (np.abs(got - ro[sel]) - (1e-2 + 1e-2 * np.abs(ro[sel]))).max() <= 0
    assert np.abs(lse_na.cpu().numpy()[sel] - rl[sel]).max() <= 1e-3

    # second call, smaller (verify-shaped, fewer sequences): the scratch still holds the first
    # call's plan and partials
    small = scaled(CONFIGS["verify"], batch=5, kv_len=(1, 1500), hq=16, hkv=2, kv_chunk=512, seed=401)
    inp2 = make_paged(small, kv_lens=[1500, 1, 700, 0, 512])
    out_na, lse_na, ref_out, ref_lse = both(amd, inp2, small)
    assert torch.equal(out_na.view(torch.int16), ref_out.view(torch.int16))
    assert torch.equal(lse_na, ref_lse)


def test_noalloc_rejects_a_call_beyond_its_capacity(amd):
    spec = scaled(CONFIGS["paged_decode"], batch=2, kv_len=(100, 200))
    inp = make_paged(spec)
    d = dev(inp)
    out = torch.empty_like(d["q"])
    # 64 sequences x 8 rows x 2048 chunks of 64 keys: far beyond 64 MiB of partials
    need = amd.attn_sink_decode_workspace_size(64, 8, 131072, 64, 64, 64)
    assert need > amd.attn_sink_decode_noalloc_capacity()
    st = amd.lib.attn_sink_decode_paged_noalloc(d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(),
                                                d["table"].data_ptr(), d["table"].shape[1], d["k"].shape[0],
                                                d["lens"].data_ptr(), None, 64, 8, 131072, 64, 8, 64, 16, 0.125, 1, 0,
                                                64, out.data_ptr(), None, None)
    assert st == 3
