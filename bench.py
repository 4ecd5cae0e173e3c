"""Benchmark of the sink-attention hot path on one MI355X.

Default workload: paged split-KV decode (64 sequences, q_len 1, KV lengths uniform in
[1024, 8192], 64 query / 8 KV heads, head_dim 64, bf16, 16-token pages in a seeded random
order, 512-token chunks merged by log-sum-exp). One step = one attn_sink_decode_paged call
(split-KV kernel + merge kernel) over the whole batch, inputs resident in HBM.

Other workloads (--workload): causal_prefill, window_prefill, verify, embed (two passes:
sinks disabled, then N(0,1) sinks), chunked_prefill (2048-token chunks appended to paged
caches of 0..6144 tokens), tree_verify (8-node draft trees per sequence, one-step
verification), rope_append (YaRN rotary encoding of the chunked-prefill workload's 16384 new
tokens and the append of their K/V into the paged cache), tiny_causal.

Prints ONE JSON line. ``value`` is the algorithmic rate of the whole step (GB/s for the
memory-bound paths, TFLOP/s for prefill); ``roofline`` describes the dominant kernel, timed
with HIP events on the stream it runs on; ``cpu_baseline`` times the fp64 CPU oracle on a
bounded sample of the same workload (rank 0, N=1 only).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from workloads import (CONFIGS, bf16_bits_to_f32, make_paged, make_paged_prefill, make_tree_masks,  # noqa: E402
                       make_varlen)

METRIC = "sink-attn decode HBM GB/s (% peak); prefill TFLOP/s (% bf16 MFMA peak)"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2516.6
KERNEL_SOURCES = {
    "rope": ["rope.hip", "common.hpp", "kernels.hpp"],
    "decode": ["decode.hip", "common.hpp", "kernels.hpp"],
    "prefill": ["prefill.hip", "common.hpp", "kernels.hpp"],
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="paged_decode",
                    choices=["paged_decode", "verify", "tree_verify", "causal_prefill", "window_prefill", "embed",
                             "chunked_prefill", "rope_append", "tiny_causal"])
    ap.add_argument("--kv-chunk", type=int, default=None,
                    help="split-KV chunk length for the paged workloads (default: the workload's)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="bounded CPU oracle sample (wall seconds)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache timing (profiling runs: every call is then a warm, timed one)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run a plain 1 GiB device copy (counter calibration for rocprofv3 --pmc)")
    ap.add_argument("--record-traffic", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE outputs (workload, then the plain copy) into "
                         "profiles/traffic.json for --workload; runs on the host only")
    return ap.parse_args()


def tbits(torch, bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def source_hash(kind):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "gqa_attention_sinks_sink_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(name, kind):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on the
    current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        data = json.load(fh)
    rec = data.get(name)
    if rec is None or rec.get("source_hash") != source_hash(kind):
        return None
    return rec.get("bytes_per_launch")


def _pmc_per_dispatch(directory, counter):
    """{dispatch id: (kernel name, value)} for one counter of a rocprofv3 --pmc CSV output."""
    import csv
    import glob
    vals = {}
    for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as fh:
            for row in csv.DictReader(fh):
                if row["Counter_Name"] != counter:
                    continue
                key = row["Dispatch_Id"]
                name, v = vals.get(key, (row["Kernel_Name"], 0.0))
                vals[key] = (name, v + float(row["Counter_Value"]))
    return vals


def prefill_kernel_name(spec, max_seqlen):
    """The prefill kernel the library launches for this shape (8-wave ping-pong kernel for
    sequences of 2048+ tokens without a window, else the 4-wave kernel)."""
    return "prefill_pp_kernel" if (spec.window <= 0 and max_seqlen >= 2048) else "prefill_kernel"


def dominant_kernel(name):
    if name in ("paged_decode", "verify", "tree_verify"):
        return "decode_split_kernel"
    if name == "rope_append":
        return "rope_append_kernel"
    if name == "chunked_prefill":
        spec = CONFIGS[name]
        return "prefill_pp_kernel" if (spec.window <= 0 and spec.q_len[1] >= 2048) else "prefill_kernel"
    spec = CONFIGS["embed_sink" if name == "embed" else name]
    return prefill_kernel_name(spec, spec.seqlen[1])


def record_traffic(name, kind, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir):
    """HBM bytes per launch of the dominant kernel from rocprofv3 FETCH_SIZE / WRITE_SIZE (KiB
    per dispatch), each scaled so that a plain 1 GiB device copy reads and writes 1 GiB."""
    kernel = dominant_kernel(name)

    def mean_for(directory, counter, pattern):
        v = [val for (k, val) in _pmc_per_dispatch(directory, counter).values()
             if ("::" + pattern + "<") in k or ("::" + pattern + "(") in k]
        if not v:
            raise SystemExit(f"no {counter} dispatch of {pattern} under {directory}")
        return float(np.mean(v)), len(v)

    def copy_kib(directory, counter):
        v = [val for (_, val) in _pmc_per_dispatch(directory, counter).values()]
        return max(v)

    gib_kib = float(1 << 20)
    f_scale = gib_kib / copy_kib(copy_fetch_dir, "FETCH_SIZE")
    w_scale = gib_kib / copy_kib(copy_write_dir, "WRITE_SIZE")
    fetch_kib, nf = mean_for(fetch_dir, "FETCH_SIZE", kernel)
    write_kib, nw = mean_for(write_dir, "WRITE_SIZE", kernel)
    fetch_b = fetch_kib * 1024 * f_scale
    write_b = write_kib * 1024 * w_scale
    path = os.path.join(ROOT, "profiles", "traffic.json")
    data = {}
    if os.path.exists(path):
        with open(path) as fh:
            data = json.load(fh)
    data[name] = {"kernel": kernel, "source_hash": source_hash(kind), "bytes_per_launch": int(fetch_b + write_b),
                  "fetch_bytes_per_launch": int(fetch_b), "write_bytes_per_launch": int(write_b),
                  "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
                  "dispatches": {"fetch": nf, "write": nw}}
    with open(path, "w") as fh:
        json.dump(data, fh, indent=1, sort_keys=True)
    print(json.dumps({name: data[name]}))


def time_calls(torch, fn, steps, warmup):
    """Average ms per step over exactly `steps` steps after `warmup` eager steps.

    The steps are captured once into a HIP graph and replayed, so host launch overhead does not
    enter the device timing; HIP events bracket the replay on the stream the kernels run on.
    """
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(steps):
            fn()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    graph.replay()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / steps


def cold_time(torch, fn, steps, scratch):
    """Median per-call time with a 1 GiB read before each call (L2 and MALL flushed).

    The flush reads a buffer written once beforehand: a write-based flush would leave dirty
    lines whose write-back competes with the timed call."""
    ts = []
    scratch.fill_(1)
    flat = scratch.view(torch.int64)
    for _ in range(steps):
        flat.sum()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        torch.cuda.synchronize()
        ts.append(s.elapsed_time(e))
    return float(np.median(ts))


# ------------------------------------------------------------------------------------------
# CPU oracle baseline (bounded sample)
# ------------------------------------------------------------------------------------------
def cpu_baseline_paged(inp, spec, seconds, bytes_per_seq, trees=None):
    import oracle
    from threadpoolctl import threadpool_limits
    f64 = lambda b: bf16_bits_to_f32(b).astype(np.float64)
    q, kc, vc = f64(inp["q"]), inp["k_cache"], inp["v_cache"]
    done_bytes, n = 0, 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        while time.perf_counter() - t0 < seconds:
            b = n % spec.batch
            L = int(inp["kv_lens"][b])
            pages = inp["page_table"][b, :(L + spec.page_size - 1) // spec.page_size]
            # the oracle reads only this sequence's pages; pass it a compact pool of them
            sub_k = f64(kc[pages])
            sub_v = f64(vc[pages])
            table = np.arange(len(pages), dtype=np.int32)[None, :]
            rows = slice(b * spec.q_len, (b + 1) * spec.q_len)
            if trees is None:
                oracle.decode_paged(q[rows], sub_k, sub_v, table, np.array([L], dtype=np.int32), inp["sinks"],
                                    spec.q_len, spec.scale, spec.causal, spec.window)
            else:
                oracle.decode_paged_tree(q[rows], sub_k, sub_v, table, np.array([L], dtype=np.int32), trees[rows],
                                         inp["sinks"], spec.q_len, spec.scale, spec.window)
            done_bytes += bytes_per_seq[b]
            n += 1
    dt = time.perf_counter() - t0
    return done_bytes / dt / 1e9, n, dt


def cpu_baseline_varlen(inp, spec, seconds, flops_per_seq, sinks):
    import oracle
    from threadpoolctl import threadpool_limits
    f64 = lambda b: bf16_bits_to_f32(b).astype(np.float64)
    cu = inp["cu_seqlens"]
    done, n = 0.0, 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        while time.perf_counter() - t0 < seconds:
            b = n % len(flops_per_seq)
            s0, s1 = int(cu[b]), int(cu[b + 1])
            sub_cu = np.array([0, s1 - s0], dtype=np.int32)
            oracle.prefill_varlen(f64(inp["q"][s0:s1]), f64(inp["k"][s0:s1]), f64(inp["v"][s0:s1]), sub_cu, sub_cu,
                                  sinks, spec.scale, spec.causal, spec.window)
            done += flops_per_seq[b]
            n += 1
    dt = time.perf_counter() - t0
    return done / dt / 1e12, n, dt


# ------------------------------------------------------------------------------------------
def pairs_visible(L, causal, window):
    L = np.asarray(L, dtype=np.int64)
    if not causal:
        return L * L if window <= 0 else None
    if window <= 0:
        return L * (L + 1) // 2
    W = window
    full = np.minimum(L, W)
    return full * (full + 1) // 2 + np.maximum(L - W, 0) * W


def bench_paged(args, torch, amd, name):
    spec = CONFIGS[name]
    if args.kv_chunk is not None:
        import dataclasses
        spec = dataclasses.replace(spec, kv_chunk=args.kv_chunk)
    inp = make_paged(spec)
    dev = torch.device("cuda:0")
    q = tbits(torch, inp["q"], dev)
    kc = tbits(torch, inp["k_cache"], dev)
    vc = tbits(torch, inp["v_cache"], dev)
    table = torch.from_numpy(inp["page_table"]).to(dev)
    lens = torch.from_numpy(inp["kv_lens"]).to(dev)
    sinks = torch.from_numpy(inp["sinks"]).to(dev)
    B, ql, hq, hkv = spec.batch, spec.q_len, spec.hq, spec.hkv
    need = amd.attn_sink_decode_workspace_size(B, ql, inp["max_kv_len"], hq, 64, spec.kv_chunk)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty((B * ql, hq), dtype=torch.float32, device=dev)
    tree = name == "tree_verify"
    trees = make_tree_masks(spec) if tree else None
    trees_d = torch.from_numpy(trees).to(dev) if tree else None

    def step():
        if tree:
            amd.attn_sink_decode_paged_tree(q, kc, vc, table, lens, trees_d, sinks, ql, inp["max_kv_len"], spec.scale,
                                            spec.window, spec.kv_chunk, workspace=ws, out=out, lse=lse)
        else:
            amd.attn_sink_decode_paged(q, kc, vc, table, lens, sinks, ql, inp["max_kv_len"], spec.scale, spec.causal,
                                       spec.window, spec.kv_chunk, workspace=ws, out=out, lse=lse)

    L = inp["kv_lens"].astype(np.int64)
    kv_bytes_seq = L * hkv * 64 * 2 * 2
    pages_seq = (L + spec.page_size - 1) // spec.page_size
    q_bytes = B * ql * hq * 64 * 2
    tree_bytes = B * ql * 4 if tree else 0
    algo_bytes = int(kv_bytes_seq.sum() + q_bytes * 2 + B * ql * hq * 4 + pages_seq.sum() * 4 + B * 4 + hq * 4
                     + tree_bytes)
    kernel_bytes = int(kv_bytes_seq.sum() + q_bytes + pages_seq.sum() * 4 + tree_bytes)   # split-KV kernel, per launch
    if tree:   # visible keys per row: the prefix plus the row's draft bits
        bits = np.array([bin(int(x) & ((1 << ql) - 1)).count("1") for x in trees], dtype=np.int64).reshape(B, ql)
        flops = int(((L[:, None] - ql + bits) * hq).sum() * 4 * 64)
    else:
        flops = int((L * hkv).sum() * (hq // hkv) * ql * 4 * 64)

    ms = time_calls(torch, step, args.steps, args.warmup)
    # the split-KV kernel alone (the split-only entry point: the same kernel, no merge)
    def split_only():
        amd.attn_sink_decode_paged_partials(q, kc, vc, table, lens, sinks, ql, inp["max_kv_len"], spec.scale,
                                            spec.causal, spec.window, spec.kv_chunk, workspace=ws)
    split_ms = None if tree else time_calls(torch, split_only, args.steps, args.warmup)
    # merge kernel alone on the same partials
    lay = amd.decode_workspace_layout(B, ql, inp["max_kv_len"], hq, spec.kv_chunk)
    n_p = lay["partials"]
    o_p = ws[lay["off_o"]:lay["off_o"] + 4 * n_p * hq * 64].view(torch.float32).view(n_p, hq, 64)
    l_p = ws[lay["off_lse"]:lay["off_lse"] + 4 * n_p * hq].view(torch.float32).view(n_p, hq)
    indptr = ws[:4 * (lay["rows"] + 1)].view(torch.int32)
    out2 = torch.empty_like(out)
    merge_ms = time_calls(torch, lambda: amd.attn_sink_merge_partials(o_p, l_p, indptr, out=out2, return_lse=False),
                          args.steps, args.warmup)
    if split_ms is None:   # tree mode has no split-only entry point: the call minus its merge
        split_ms = ms - merge_ms
    cold_ms = None
    if not args.no_cold:
        scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        cold_ms = cold_time(torch, step, max(5, min(args.steps, 20)), scratch)
        del scratch

    value = algo_bytes / (ms * 1e-3) / 1e9
    achieved = kernel_bytes / (split_ms * 1e-3) / 1e9
    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{name}: {B} seqs x q_len {ql}{' (8-node random draft trees)' if tree else ''}, "
                               f"kv {spec.kv_len[0]}..{spec.kv_len[1]} "
                               f"(sum {int(L.sum())}), {hq}/{hkv} heads, d 64, {spec.page_size}-token pages, "
                               f"{spec.kv_chunk}-token chunks, sinks N(0,{spec.sink_std}^2)",
                   "algorithmic_bytes": algo_bytes, "algorithmic_flops": flops},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "roofline": {"kernel": "decode_split_kernel", "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(name, "decode"), "algorithmic_bytes_per_launch": kernel_bytes,
                     "kernel_ms": round(split_ms, 5), "merge_ms": round(merge_ms, 5)},
    }
    if cold_ms is not None:
        res["cold_l2_mall_ms_per_step"] = round(cold_ms, 5)
        res["cold_value"] = round(algo_bytes / (cold_ms * 1e-3) / 1e9, 1)
    if not args.no_cpu_baseline:
        v, n, dt = cpu_baseline_paged(inp, spec, args.cpu_seconds, kv_bytes_seq, trees)
        res["cpu_baseline"] = {"value": round(v, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
                               "sample": f"{n} sequences of this batch (cycled from sequence 0), {dt:.1f} s wall, "
                                         f"fp64 NumPy, BLAS limited to 1 thread"}
    return res


def bench_varlen(args, torch, amd, name):
    if name == "embed":
        specs = [CONFIGS["embed_nosink"], CONFIGS["embed_sink"]]
    else:
        specs = [CONFIGS[name]]
    spec = specs[-1]
    inp = make_varlen(spec)
    dev = torch.device("cuda:0")
    q, k, v = (tbits(torch, inp[x], dev) for x in ("q", "k", "v"))
    cu = torch.from_numpy(inp["cu_seqlens"]).to(dev)
    sinks = torch.from_numpy(inp["sinks"]).to(dev)
    out = torch.empty_like(q)
    lse = torch.empty((q.shape[0], spec.hq), dtype=torch.float32, device=dev)
    mx = inp["max_seqlen"]

    def one(s, use_sinks):
        amd.attn_sink_prefill(q, k, v, sinks if use_sinks else None, cu, cu, mx, mx, s.scale, s.causal, s.window,
                              out=out, lse=lse)

    def step():
        for s in specs:
            one(s, s.sink_std is not None)

    lens = inp["seqlens"].astype(np.int64)
    pairs = pairs_visible(lens, spec.causal, spec.window)
    flops_seq = pairs * 4 * 64 * spec.hq
    flops = int(flops_seq.sum()) * len(specs)
    T = int(lens.sum())
    io_bytes = T * (spec.hq * 64 * 2 * 2 + spec.hkv * 64 * 2 * 2 + spec.hq * 4)
    algo_bytes = io_bytes * len(specs)

    ms = time_calls(torch, step, args.steps, args.warmup)
    kernel_ms = ms / len(specs)
    tflops = flops / (ms * 1e-3) / 1e12
    gbs = algo_bytes / (ms * 1e-3) / 1e9
    ai = flops / algo_bytes
    bound = "mfma" if ai > MFMA_BF16_PEAK_TFLOPS / HBM_PEAK_GBS * 1e3 else "hbm"
    if bound == "mfma":
        roof = {"kernel": prefill_kernel_name(spec, mx), "bound": "mfma", "achieved": round(flops / len(specs) / (kernel_ms * 1e-3) / 1e12, 2),
                "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"kernel": prefill_kernel_name(spec, mx), "bound": "hbm", "achieved": round(io_bytes / (kernel_ms * 1e-3) / 1e9, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = measured_traffic(name, "prefill")
    roof["algorithmic_flops_per_launch"] = int(flops_seq.sum())
    roof["algorithmic_bytes_per_launch"] = io_bytes
    roof["kernel_ms"] = round(kernel_ms, 5)
    res = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{name}: {spec.batch} seqs, lengths {spec.seqlen[0]}..{spec.seqlen[1]} (sum {T}), "
                               f"{spec.hq}/{spec.hkv} heads, d 64, causal={spec.causal}, window={spec.window}, "
                               f"passes={len(specs)}",
                   "algorithmic_flops": flops, "algorithmic_bytes": algo_bytes},
        "pct_mfma_peak": round(100 * tflops / MFMA_BF16_PEAK_TFLOPS, 2), "gb_per_s": round(gbs, 1),
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        s = inp["sinks"] if spec.sink_std is not None else np.full(spec.hq, -np.inf, dtype=np.float32)
        v, n, dt = cpu_baseline_varlen(inp, spec, args.cpu_seconds, flops_seq, s)
        res["cpu_baseline"] = {"value": round(v, 6), "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
                               "sample": f"{n} sequences of this batch (cycled from sequence 0), {dt:.1f} s wall, "
                                         f"fp64 NumPy, BLAS limited to 1 thread"}
    return res


def chunk_pairs(q_lens, kv_lens, causal, window):
    """Visible (query, key) pairs per sequence of a chunked prefill (queries are the newest
    q_len of kv_len tokens)."""
    out = []
    for lq, lk in zip(np.asarray(q_lens, dtype=np.int64), np.asarray(kv_lens, dtype=np.int64)):
        pos = np.arange(lk - lq, lk)
        vis = np.minimum(pos + 1, lk) if causal else np.full(lq, lk)
        if window > 0:
            vis = np.minimum(vis, window)
        out.append(int(vis.sum()))
    return np.asarray(out, dtype=np.int64)


def cpu_baseline_chunked(inp, spec, seconds, sinks, block=64):
    """The fp64 oracle on blocks of 64 chunk rows, cycling over sequences."""
    import oracle
    from threadpoolctl import threadpool_limits
    f64 = lambda b: bf16_bits_to_f32(b).astype(np.float64)
    cu, lens = inp["cu_seqlens_q"], inp["kv_lens"]
    q, kc, vc = f64(inp["q"]), f64(inp["k_cache"]), f64(inp["v_cache"])  # input widening, not timed
    done, n = 0.0, 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        while time.perf_counter() - t0 < seconds:
            b = n % len(lens)
            q0, lq = int(cu[b]), int(cu[b + 1] - cu[b])
            rows = np.arange(min(block, lq))
            # one sequence at a time, as the varlen baseline does
            oracle.prefill_paged(q[q0:q0 + lq], kc, vc, inp["page_table"][b:b + 1], np.array([0, lq]), lens[b:b + 1],
                                 sinks, spec.scale, spec.causal, spec.window, rows={0: rows})
            pos = int(lens[b]) - lq + rows
            vis = np.minimum(pos + 1, int(lens[b])) if spec.causal else np.full(len(rows), int(lens[b]))
            if spec.window > 0:
                vis = np.minimum(vis, spec.window)
            done += float(vis.sum()) * 4 * 64 * spec.hq
            n += 1
    dt = time.perf_counter() - t0
    return done / dt / 1e12, n, dt


def bench_chunked(args, torch, amd, name):
    spec = CONFIGS[name]
    inp = make_paged_prefill(spec)
    dev = torch.device("cuda:0")
    q, kc, vc = (tbits(torch, inp[x], dev) for x in ("q", "k_cache", "v_cache"))
    table = torch.from_numpy(inp["page_table"]).to(dev)
    cu = torch.from_numpy(inp["cu_seqlens_q"]).to(dev)
    lens = torch.from_numpy(inp["kv_lens"]).to(dev)
    sinks = torch.from_numpy(inp["sinks"]).to(dev)
    out = torch.empty_like(q)
    lse = torch.empty((q.shape[0], spec.hq), dtype=torch.float32, device=dev)

    def step():
        amd.attn_sink_prefill_paged(q, kc, vc, table, cu, lens, sinks, inp["max_q"], inp["max_kv_len"], spec.scale,
                                    spec.causal, spec.window, out=out, lse=lse)

    pairs = chunk_pairs(inp["q_lens"], inp["kv_lens"], spec.causal, spec.window)
    flops_seq = pairs * 4 * 64 * spec.hq
    flops = int(flops_seq.sum())
    T = int(inp["q_lens"].sum())
    kv_tokens = int(inp["kv_lens"].astype(np.int64).sum())
    pages = int(((inp["kv_lens"].astype(np.int64) + spec.page_size - 1) // spec.page_size).sum())
    algo_bytes = T * (spec.hq * 64 * 2 * 2 + spec.hq * 4) + kv_tokens * spec.hkv * 64 * 2 * 2 + 4 * pages

    ms = time_calls(torch, step, args.steps, args.warmup)
    tflops = flops / (ms * 1e-3) / 1e12
    gbs = algo_bytes / (ms * 1e-3) / 1e9
    bound = "mfma" if flops / algo_bytes > MFMA_BF16_PEAK_TFLOPS / HBM_PEAK_GBS * 1e3 else "hbm"
    kname = "prefill_pp_kernel" if (spec.window <= 0 and inp["max_q"] >= 2048) else "prefill_kernel"
    if bound == "mfma":
        roof = {"kernel": kname, "bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s"}
    else:
        roof = {"kernel": kname, "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = measured_traffic(name, "prefill")
    roof["algorithmic_flops_per_launch"] = flops
    roof["algorithmic_bytes_per_launch"] = algo_bytes
    roof["kernel_ms"] = round(ms, 5)
    res = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{name}: {spec.batch} seqs, chunks of {spec.q_len[0]}..{spec.q_len[1]} tokens on "
                               f"{spec.ctx_len[0]}..{spec.ctx_len[1]} cached (sum {T} queries, {kv_tokens} keys), "
                               f"{spec.hq}/{spec.hkv} heads, d 64, {spec.page_size}-token pages, causal={spec.causal}",
                   "algorithmic_flops": flops, "algorithmic_bytes": algo_bytes},
        "pct_mfma_peak": round(100 * tflops / MFMA_BF16_PEAK_TFLOPS, 2), "gb_per_s": round(gbs, 1),
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        v, n, dt = cpu_baseline_chunked(inp, spec, args.cpu_seconds, inp["sinks"])
        res["cpu_baseline"] = {"value": round(v, 6), "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
                               "sample": f"{n} blocks of 64 chunk rows (cycling over the sequences), {dt:.1f} s wall, "
                                         f"fp64 NumPy, BLAS limited to 1 thread"}
    return res


ROPE_ARGS = dict(rope_theta=150000.0, yarn_factor=32.0, yarn_original_len=4096, yarn_alpha=1.0, yarn_beta=32.0)


def cpu_baseline_rope(inp, k_new, v_new, seconds, bytes_per_seq):
    """The fp64 oracle, one sequence at a time (a compact pool of the sequence's pages)."""
    import oracle
    from threadpoolctl import threadpool_limits
    f64 = lambda b: bf16_bits_to_f32(b).astype(np.float64)
    q, kn, vn = f64(inp["q"]), f64(k_new), f64(v_new)
    freqs, m = oracle.yarn_frequencies(64, ROPE_ARGS["rope_theta"], ROPE_ARGS["yarn_factor"],
                                       ROPE_ARGS["yarn_original_len"], ROPE_ARGS["yarn_alpha"], ROPE_ARGS["yarn_beta"])
    cu, lens = inp["cu_seqlens_q"], inp["kv_lens"]
    P = inp["k_cache"].shape[2]
    done, n = 0, 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        while time.perf_counter() - t0 < seconds:
            b = n % len(lens)
            L = int(lens[b])
            pages = inp["page_table"][b, :(L + P - 1) // P]
            r0, r1 = int(cu[b]), int(cu[b + 1])
            oracle.rope_append(q[r0:r1], kn[r0:r1], vn[r0:r1], np.array([0, r1 - r0]), lens[b:b + 1],
                               np.arange(len(pages))[None, :], f64(inp["k_cache"][pages]), f64(inp["v_cache"][pages]),
                               freqs, m)
            done += bytes_per_seq[b]
            n += 1
    dt = time.perf_counter() - t0
    return done / dt / 1e9, n, dt


def bench_rope(args, torch, amd, name):
    spec = CONFIGS["chunked_prefill"]
    inp = make_paged_prefill(spec)
    dev = torch.device("cuda:0")
    T = int(inp["cu_seqlens_q"][-1])
    rng = np.random.default_rng(11)
    from workloads import bf16_round_bits
    k_new = bf16_round_bits(rng.standard_normal((T, spec.hkv, 64)).astype(np.float32))
    v_new = bf16_round_bits(rng.standard_normal((T, spec.hkv, 64)).astype(np.float32))
    q, kn, vn = tbits(torch, inp["q"], dev), tbits(torch, k_new, dev), tbits(torch, v_new, dev)
    kc, vc = tbits(torch, inp["k_cache"], dev), tbits(torch, inp["v_cache"], dev)
    cu = torch.from_numpy(inp["cu_seqlens_q"]).to(dev)
    lens = torch.from_numpy(inp["kv_lens"]).to(dev)
    table = torch.from_numpy(inp["page_table"]).to(dev)
    q_out = torch.empty_like(q)

    def step():
        amd.attn_sink_rope_append(q, kn, vn, cu, lens, table, kc, vc, inp["max_q"], inp["max_kv_len"], q_out=q_out,
                                  **ROPE_ARGS)

    q_lens = inp["q_lens"].astype(np.int64)
    row_bytes = (spec.hq * 64 * 2) * 2 + (spec.hkv * 64 * 2) * 4     # q in + out, k/v in + cache out
    bytes_seq = q_lens * row_bytes + q_lens * 4                      # + one page id per token
    algo_bytes = int(bytes_seq.sum() + 4 * (2 * spec.batch + 1))
    ms = time_calls(torch, step, args.steps, args.warmup)
    gbs = algo_bytes / (ms * 1e-3) / 1e9
    res = {
        "metric": METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{name}: YaRN rotary encoding (theta 150000, factor 32, original 4096) of {T} new "
                               f"tokens ({spec.batch} chunks of 2048 on 0..6144 cached), {spec.hq}/{spec.hkv} heads, "
                               f"d 64, K/V appended into 16-token pages",
                   "algorithmic_bytes": algo_bytes},
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "roofline": {"kernel": "rope_append_kernel", "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(name, "rope"),
                     "algorithmic_bytes_per_launch": algo_bytes, "kernel_ms": round(ms, 5)},
    }
    if not args.no_cpu_baseline:
        v, n, dt = cpu_baseline_rope(inp, k_new, v_new, args.cpu_seconds, bytes_seq)
        res["cpu_baseline"] = {"value": round(v, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
                               "sample": f"{n} sequences' chunks (cycled from sequence 0), {dt:.1f} s wall, fp64 "
                                         f"NumPy, BLAS limited to 1 thread"}
    return res


def main():
    args = parse()
    if args.record_traffic:
        kind = ("decode" if args.workload in ("paged_decode", "verify", "tree_verify") else
                "rope" if args.workload == "rope_append" else "prefill")
        record_traffic(args.workload, kind, *args.record_traffic)
        return
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported (this build measures the "
              f"one-GPU shard of the path).", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (HIP device)", file=sys.stderr)
        sys.exit(1)
    import gqa_attention_sinks_sink_amd as amd
    if args.calibrate_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0").fill_(3)
        for _ in range(3):
            b = a.clone()
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "copy", "bytes_read": 1 << 30, "bytes_written": 1 << 30}))
        return
    if args.workload in ("paged_decode", "verify", "tree_verify"):
        res = bench_paged(args, torch, amd, args.workload)
    elif args.workload == "chunked_prefill":
        res = bench_chunked(args, torch, amd, args.workload)
    elif args.workload == "rope_append":
        res = bench_rope(args, torch, amd, args.workload)
    else:
        res = bench_varlen(args, torch, amd, args.workload)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
