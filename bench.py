"""Benchmark of the sink-attention hot path on one MI355X.

Default run: the two halves of the headline metric on one line.
  * paged decode (top level): 64 sequences, q_len 1, KV lengths uniform in [1024, 8192],
    64 query / 8 KV heads, head_dim 64, bf16, 16-token pages in a seeded random order,
    512-token chunks merged by log-sum-exp. One step = one attn_sink_decode_paged call
    (split-KV kernel + merge kernel) over the whole batch; HBM GB/s.
  * causal prefill (the "prefill" object): 8 x 4096 tokens packed, 64 query / 8 KV heads;
    one step = one attn_sink_prefill call; TFLOP/s against the bf16 MFMA peak.
Other workloads (--workload): verify, tree_verify, window_prefill, embed (two passes: sinks
disabled, then N(0,1) sinks), chunked_prefill, rope_append, tiny_causal, and each half alone.

Every timed call is first checked against the fp64 CPU oracle on sampled rows (the accuracy
gate comes before any timing); a mismatch exits with status 3 and no timing line. Then:
  * value: the whole step, W eager warmup steps, then exactly K steps captured in a HIP graph
    and replayed between two HIP events on the launch stream, inputs resident in HBM;
  * cold_*: the median of single calls each preceded by a 1 GiB read that flushes the L2 and
    the MALL (the flush is outside the timed region);
  * roofline: the dominant kernel's algorithmic bytes (or FLOPs) per launch over its average
    launch time, measured the same way (decode: the split-only entry point);
  * cpu_baseline: the fp64 oracle, unchanged, run before the GPU is touched, by a pool of
    worker processes on the host's cores (at most 16), each with BLAS on one thread, over a
    bounded sample of the same workload.
Prints ONE JSON line. --record-traffic and --summarize turn rocprofv3 outputs into the
summaries under profiles/ (host only).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from workloads import (CONFIGS, bf16_bits_to_f32, bf16_round_bits, make_paged, make_paged_prefill,  # noqa: E402
                       make_tree_masks, make_varlen)

METRIC = "sink-attn decode HBM GB/s (% peak); prefill TFLOP/s (% bf16 MFMA peak)"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2516.6
ATOL, RTOL, LSE_TOL = 1e-2, 1e-2, 1e-3
KERNEL_SOURCES = {
    "rope": ["rope.hip", "common.hpp", "kernels.hpp"],
    "decode": ["decode.hip", "common.hpp", "kernels.hpp"],
    "prefill": ["prefill.hip", "common.hpp", "kernels.hpp"],
}
WORKLOADS = ["default", "paged_decode", "verify", "tree_verify", "causal_prefill", "window_prefill", "embed",
             "chunked_prefill", "rope_append", "tiny_causal", "paged_decode_tp4", "causal_prefill_tp4"]
DECODE_WORKLOADS = ("paged_decode", "verify", "tree_verify", "paged_decode_tp4")
ROPE_ARGS = dict(rope_theta=150000.0, yarn_factor=32.0, yarn_original_len=4096, yarn_alpha=1.0, yarn_beta=32.0)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="default", choices=WORKLOADS,
                    help="default: paged decode with causal prefill as its 'prefill' object")
    ap.add_argument("--kv-chunk", type=int, default=None,
                    help="split-KV chunk length for the paged workloads (default: the workload's)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="bounded CPU oracle sample (wall seconds)")
    ap.add_argument("--cpu-workers", type=int, default=None,
                    help="oracle worker processes (default: the host cores this process may use, at most 16)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache timing (profiling runs: every call is then a warm, timed one)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run a plain 1 GiB device copy (counter calibration for rocprofv3 --pmc)")
    ap.add_argument("--record-traffic", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE outputs (workload, then the plain copy) into "
                         "profiles/traffic.json for --workload; runs on the host only")
    ap.add_argument("--summarize", nargs=3, metavar=("STATS_DIR", "OUT_MD", "TITLE"),
                    help="write a markdown summary of a rocprofv3 --stats output (kernel_stats.csv) to OUT_MD; "
                         "--summary-command names the command that produced it; runs on the host only")
    ap.add_argument("--summary-command", default="", help="the command recorded in a --summarize summary")
    ap.add_argument("--summary-workload", default=None,
                    help="append this workload's HBM traffic (profiles/traffic.json) to a --summarize summary")
    ap.add_argument("--pmc-table", nargs=2, metavar=("PMC_DIR", "KERNEL"),
                    help="print, as one JSON line, the per-dispatch average of every counter in a rocprofv3 --pmc "
                         "output over the dispatches of KERNEL (a name such as prefill_pp_kernel); host only")
    return ap.parse_args()


# ------------------------------------------------------------------------------------------
# host-side helpers
# ------------------------------------------------------------------------------------------
def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_workers(args):
    n = len(os.sched_getaffinity(0))
    return max(1, min(n, 16) if args.cpu_workers is None else args.cpu_workers)


def f64(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


def code_only(text):
    """C++ source text without its comments, whitespace runs collapsed to one space: what the
    compiler sees, so that editing a comment does not orphan a counter record."""
    out, i, n = [], 0, len(text)
    while i < n:
        ch = text[i]
        if ch in "\"'":  # string or character literal, copied whole
            j = i + 1
            while j < n and text[j] != ch:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
            out.append(" ")
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(ch)
            i += 1
    return " ".join("".join(out).split())


def source_hash(kind):
    """Hash of the code (comments and layout aside) of the sources a kernel kind is built from."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "gqa_attention_sinks_sink_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(code_only(fh.read()).encode("utf-8"))
        h.update(b"\0")
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


def prefill_kernel_name(window, max_seqlen):
    """The prefill kernel the library launches for this shape (8-wave ping-pong kernel for
    query ranges of 2048+ tokens without a window, else the 4-wave kernel)."""
    return "prefill_pp_kernel" if (window <= 0 and max_seqlen >= 2048) else "prefill_kernel"


def dominant_kernel(name):
    if name in DECODE_WORKLOADS + ("default",):
        return "decode_split_kernel"
    if name == "rope_append":
        return "rope_append_kernel"
    if name == "chunked_prefill":
        spec = CONFIGS[name]
        return prefill_kernel_name(spec.window, spec.q_len[1])
    spec = CONFIGS["embed_sink" if name == "embed" else name]
    return prefill_kernel_name(spec.window, spec.seqlen[1])


def kernel_kind(name):
    return ("decode" if name in DECODE_WORKLOADS + ("default",) else
            "rope" if name == "rope_append" else "prefill")


def record_traffic(name, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir):
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
        return max(val for (_, val) in _pmc_per_dispatch(directory, counter).values())

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
    data[name] = {"kernel": kernel, "source_hash": source_hash(kernel_kind(name)),
                  "bytes_per_launch": int(fetch_b + write_b), "fetch_bytes_per_launch": int(fetch_b),
                  "write_bytes_per_launch": int(write_b), "fetch_scale": round(f_scale, 4),
                  "write_scale": round(w_scale, 4), "dispatches": {"fetch": nf, "write": nw}}
    with open(path, "w") as fh:
        json.dump(data, fh, indent=1, sort_keys=True)
    print(json.dumps({name: data[name]}))


def summarize(stats_dir, out_md, title, command, workload=None):
    """Markdown table of a rocprofv3 --kernel-trace --stats output: per kernel, calls and the
    average / min / max duration in microseconds (from kernel_stats.csv); with a workload, its HBM
    traffic record from profiles/traffic.json when that was taken on the current kernel source."""
    paths = glob.glob(os.path.join(stats_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not paths:
        raise SystemExit(f"no kernel_stats.csv under {stats_dir}")
    rows = []
    with open(paths[0]) as fh:
        for r in csv.DictReader(fh):
            rows.append((r["Name"], int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                         float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    rows.sort(key=lambda x: -x[5])
    short = lambda n: n if len(n) <= 90 else n[:87] + "..."
    lines = [f"# {title}", "", "Command (run from /tmp on the GPU host, $REPO = repository root):", "",
             f"    {command}", "",
             "Source: rocprofv3 `--kernel-trace --stats` kernel_stats.csv; durations in microseconds.", "",
             "| kernel | calls | avg us | min us | max us | % time |", "|---|---|---|---|---|---|"]
    for n, c, a, lo, hi, pct in rows:
        lines.append(f"| `{short(n)}` | {c} | {a:.2f} | {lo:.2f} | {hi:.2f} | {pct:.1f} |")
    if workload is not None:
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as fh:
            rec = json.load(fh).get(workload)
        if rec is not None and rec["source_hash"] == source_hash(kernel_kind(workload)):
            # paged decode's line also times the planner's chunk length (context), so its counters
            # are taken with the workload's 512-token chunks alone
            chunk = " --kv-chunk 512" if workload == "paged_decode" else ""
            lines += ["", f"HBM traffic of `{rec['kernel']}` per launch (rocprofv3 `--pmc FETCH_SIZE`, then `--pmc "
                          f"WRITE_SIZE`, each in its own run of `bench.py --workload {workload}{chunk} --steps 2 --warmup 1 "
                          f"--no-cold --no-cpu-baseline`; KiB per dispatch scaled so that a plain 1 GiB copy "
                          f"(`bench.py --calibrate-copy`) reads and writes 1 GiB: fetch x{rec['fetch_scale']}, write "
                          f"x{rec['write_scale']}; recorded by `bench.py --record-traffic`, source hash "
                          f"{rec['source_hash']}):", "",
                      "| fetched bytes | written bytes | total | dispatches averaged |", "|---|---|---|---|",
                      f"| {rec['fetch_bytes_per_launch']:,} | {rec['write_bytes_per_launch']:,} | "
                      f"{rec['bytes_per_launch']:,} | {rec['dispatches']['fetch']} |"]
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(out_md)


def pmc_table(directory, kernel):
    """Per-dispatch averages of every counter of a rocprofv3 --pmc output over the dispatches of
    one kernel (counters summed over the chip per dispatch, as rocprofv3 reports them)."""
    per = {}     # counter -> {dispatch: value}
    names = set()
    for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as fh:
            for row in csv.DictReader(fh):
                k = row["Kernel_Name"]
                if ("::" + kernel + "<") not in k and ("::" + kernel + "(") not in k:
                    continue
                names.add(k)
                d = per.setdefault(row["Counter_Name"], {})
                d[row["Dispatch_Id"]] = d.get(row["Dispatch_Id"], 0.0) + float(row["Counter_Value"])
    if not per:
        raise SystemExit(f"no dispatch of {kernel} under {directory}")
    out = {"kernel": sorted(names), "dispatches": max(len(v) for v in per.values())}
    out.update({c: float(np.mean(list(v.values()))) for c, v in sorted(per.items())})
    print(json.dumps(out))


# ------------------------------------------------------------------------------------------
# CPU oracle baseline: a pool of worker processes forked before the GPU is initialised
# ------------------------------------------------------------------------------------------
_CPU_JOB = None   # (task function, number of tasks, seconds); read by the forked workers


def _cpu_worker(args):
    wid, n_workers = args
    from threadpoolctl import threadpool_limits
    task, n_tasks, seconds = _CPU_JOB
    done, n = 0.0, 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        i = wid
        while time.perf_counter() - t0 < seconds:
            done += task(i % n_tasks)
            n += 1
            i += n_workers
    return done, n


def cpu_pool(task, n_tasks, seconds, workers):
    """Runs task(i) (returning the units it processed) on `workers` processes for about `seconds`
    of wall time; returns (units per second over the pool's wall time, tasks done, wall)."""
    import multiprocessing as mp
    global _CPU_JOB
    _CPU_JOB = (task, n_tasks, seconds)
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(workers) as pool:
        res = pool.map(_cpu_worker, [(w, workers) for w in range(workers)])
    wall = time.perf_counter() - t0
    _CPU_JOB = None
    units = sum(r[0] for r in res)
    return units / wall, sum(r[1] for r in res), wall


def cpu_baseline_record(value, unit, n, wall, workers, what):
    return {"value": value, "unit": unit, "cores": workers, "kind": "oracle",
            "sample": f"{n} {what} in {wall:.1f} s wall by {workers} worker processes (fp64 NumPy oracle, BLAS on "
                      f"one thread each)",
            "cpu_model": cpu_model(), "host_cores_available": len(os.sched_getaffinity(0))}


# ------------------------------------------------------------------------------------------
# GPU timing and the parity gate
# ------------------------------------------------------------------------------------------
def tbits(torch, bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


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


def cold_time(torch, fn, steps, dev):
    """Median per-call time with a 1 GiB read before each call (L2 and MALL flushed).

    The flush reads a buffer written once beforehand: a write-based flush would leave dirty
    lines whose write-back competes with the timed call."""
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    scratch.fill_(1)
    flat = scratch.view(torch.int64)
    ts = []
    for _ in range(steps):
        flat.sum()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        torch.cuda.synchronize()
        ts.append(s.elapsed_time(e))
    del scratch
    return float(np.median(ts))


def parity_gate(name, out, lse, ro, rl):
    """Compares sampled rows (those the oracle computed, rl not NaN) with the bar; exits 3 on a
    mismatch, before anything is timed."""
    sel = ~np.isnan(rl)
    o, r = out[sel], ro[sel]
    err = np.abs(o - r)
    excess = float((err - (ATOL + RTOL * np.abs(r))).max())
    ok = bool(np.isfinite(o).all()) and excess <= 0
    lse_err = 0.0
    if lse is not None:
        l, rr = lse[sel], rl[sel]
        inf = np.isinf(rr)
        ok = ok and np.array_equal(np.isinf(l), inf) and np.array_equal(l[inf], rr[inf])
        if (~inf).any():
            lse_err = float(np.abs(l[~inf] - rr[~inf]).max())
            ok = ok and lse_err <= LSE_TOL
    rec = {"rows": int(sel.sum()), "max_abs_err": round(float(err.max()), 6), "max_excess": round(excess, 6),
           "lse_max_err": round(lse_err, 6), "bar": "|err| <= 1e-2 + 1e-2 |ref|, lse <= 1e-3"}
    if not ok:
        print(json.dumps({"error": f"{name}: parity gate failed before timing", "parity": rec}), file=sys.stderr)
        sys.exit(3)
    return rec


def out_np(t):
    return t.float().cpu().numpy().astype(np.float64)


def pairs_visible(L, causal, window):
    L = np.asarray(L, dtype=np.int64)
    if not causal:
        return L * L if window <= 0 else None
    if window <= 0:
        return L * (L + 1) // 2
    W = window
    full = np.minimum(L, W)
    return full * (full + 1) // 2 + np.maximum(L - W, 0) * W


def block_pairs(lq, lk, rows, causal, window):
    """Visible (query, key) pairs of the given query rows of a sequence whose Lq queries are the
    last of its Lk keys."""
    pos = lk - lq + np.asarray(list(rows), dtype=np.int64)
    vis = np.minimum(pos + 1, lk) if causal else np.full(len(pos), lk)
    if window > 0:
        vis = np.minimum(vis, window)
    return int(vis.sum())


def oracle():
    import oracle as _oracle
    return _oracle


def spread_block(k, n_blk):
    """The k-th block of a sample that visits a sequence's n_blk blocks in an order spread over the
    whole sequence (a stride coprime with n_blk), so that any prefix of the sample covers early and
    late causal blocks alike."""
    stride = next(st for st in (29, 31, 37, 41, 43, 1) if np.gcd(st, n_blk) == 1)
    return (k * stride) % n_blk


_SEQ_CACHE = {}


def seq_f64(key, make):
    """The fp64 widening of one sequence's K/V, kept for the next call with the same key (a worker
    of the CPU pool keeps drawing the same sequence); one entry."""
    if key not in _SEQ_CACHE:
        _SEQ_CACHE.clear()
        _SEQ_CACHE[key] = make()
    return _SEQ_CACHE[key]


# ------------------------------------------------------------------------------------------
# workloads
# ------------------------------------------------------------------------------------------
class Paged:
    """Paged decode / verify / draft-tree verification (split-KV + merge)."""

    def __init__(self, name, args):
        import dataclasses
        self.name = name
        spec = CONFIGS[name]
        if args.kv_chunk is not None:
            spec = dataclasses.replace(spec, kv_chunk=args.kv_chunk)
        # Verify-shaped calls leave the chunk length open: the library's planner picks it from the
        # lengths and the device's workgroup count (paged decode keeps the 512-token chunks its
        # workload names).
        self.planned = args.kv_chunk is None and name in ("verify", "tree_verify")
        self.spec = spec
        self.inp = make_paged(spec)
        self.tree = name == "tree_verify"
        self.trees = make_tree_masks(spec) if self.tree else None
        B, ql, hq, hkv = spec.batch, spec.q_len, spec.hq, spec.hkv
        L = self.inp["kv_lens"].astype(np.int64)
        self.kv_bytes_seq = L * hkv * 64 * 2 * 2
        pages_seq = (L + spec.page_size - 1) // spec.page_size
        q_bytes = B * ql * hq * 64 * 2
        tree_bytes = B * ql * 4 if self.tree else 0
        self.algo_bytes = int(self.kv_bytes_seq.sum() + q_bytes * 2 + B * ql * hq * 4 + pages_seq.sum() * 4 + B * 4
                              + hq * 4 + tree_bytes)
        self.kernel_bytes = int(self.kv_bytes_seq.sum() + q_bytes + pages_seq.sum() * 4 + tree_bytes)
        if self.tree:   # visible keys per row: the prefix plus the row's draft bits
            bits = np.array([bin(int(x) & ((1 << ql) - 1)).count("1") for x in self.trees],
                            dtype=np.int64).reshape(B, ql)
            self.flops = int(((L[:, None] - ql + bits) * hq).sum() * 4 * 64)
        else:
            self.flops = int((L * hkv).sum() * (hq // hkv) * ql * 4 * 64)

    def _oracle_seq(self, b):
        spec, inp = self.spec, self.inp
        L = int(inp["kv_lens"][b])
        pages = inp["page_table"][b, :(L + spec.page_size - 1) // spec.page_size]
        # the sequence's pages as a compact pool of their own
        sub_k, sub_v = f64(inp["k_cache"][pages]), f64(inp["v_cache"][pages])
        table = np.arange(len(pages), dtype=np.int32)[None, :]
        rows = slice(b * spec.q_len, (b + 1) * spec.q_len)
        q = f64(inp["q"][rows])
        lens = np.array([L], dtype=np.int32)
        if self.tree:
            return rows, oracle().decode_paged_tree(q, sub_k, sub_v, table, lens, self.trees[rows], inp["sinks"],
                                                    spec.q_len, spec.scale, spec.window)
        return rows, oracle().decode_paged(q, sub_k, sub_v, table, lens, inp["sinks"], spec.q_len, spec.scale,
                                           spec.causal, spec.window)

    def cpu_baseline(self, args, workers):
        def task(b):
            self._oracle_seq(b)
            return float(self.kv_bytes_seq[b])
        v, n, wall = cpu_pool(task, self.spec.batch, args.cpu_seconds, workers)
        return cpu_baseline_record(round(v / 1e9, 4), "GB/s", n, wall, workers,
                                   "sequences of this batch (each worker from its own start, cycling)")

    def config(self):
        spec, L = self.spec, self.inp["kv_lens"]
        return {"workload": f"{self.name}: {spec.batch} seqs x q_len {spec.q_len}"
                            f"{' (8-node random draft trees)' if self.tree else ''}, kv {spec.kv_len[0]}..{spec.kv_len[1]} "
                            f"(sum {int(L.sum())}), {spec.hq}/{spec.hkv} heads, d 64, {spec.page_size}-token pages, "
                            f"{spec.kv_chunk}-token chunks{' (planner)' if self.planned else ''}, "
                            f"sinks N(0,{spec.sink_std}^2)",
                "algorithmic_bytes": self.algo_bytes, "algorithmic_flops": self.flops}

    def gpu(self, torch, amd, args, dev):
        if self.planned:
            import dataclasses
            s0 = self.spec
            chunk = amd.attn_sink_decode_plan_chunk(self.inp["kv_lens"], s0.q_len, s0.hq, s0.hkv, s0.page_size)
            self.spec = dataclasses.replace(s0, kv_chunk=chunk)
        spec, inp = self.spec, self.inp
        q, kc, vc = tbits(torch, inp["q"], dev), tbits(torch, inp["k_cache"], dev), tbits(torch, inp["v_cache"], dev)
        table = torch.from_numpy(inp["page_table"]).to(dev)
        lens = torch.from_numpy(inp["kv_lens"]).to(dev)
        sinks = torch.from_numpy(inp["sinks"]).to(dev)
        B, ql, hq = spec.batch, spec.q_len, spec.hq
        mkv = inp["max_kv_len"]
        need = amd.attn_sink_decode_workspace_size(B, ql, mkv, hq, 64, spec.kv_chunk)
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
        out = torch.empty_like(q)
        lse = torch.empty((B * ql, hq), dtype=torch.float32, device=dev)
        trees_d = torch.from_numpy(self.trees).to(dev) if self.tree else None

        def step():
            if self.tree:
                amd.attn_sink_decode_paged_tree(q, kc, vc, table, lens, trees_d, sinks, ql, mkv, spec.scale,
                                                spec.window, spec.kv_chunk, workspace=ws, out=out, lse=lse)
            else:
                amd.attn_sink_decode_paged(q, kc, vc, table, lens, sinks, ql, mkv, spec.scale, spec.causal,
                                           spec.window, spec.kv_chunk, workspace=ws, out=out, lse=lse)

        def split_only():
            if self.tree:
                amd.attn_sink_decode_paged_tree_partials(q, kc, vc, table, lens, trees_d, sinks, ql, mkv, spec.scale,
                                                         spec.window, spec.kv_chunk, workspace=ws)
            else:
                amd.attn_sink_decode_paged_partials(q, kc, vc, table, lens, sinks, ql, mkv, spec.scale, spec.causal,
                                                    spec.window, spec.kv_chunk, workspace=ws)

        # accuracy gate: the timed call on sampled sequences against the oracle
        step()
        torch.cuda.synchronize()
        got_o, got_l = out_np(out), lse.cpu().numpy().astype(np.float64)
        ro = np.full(got_o.shape, np.nan)
        rl = np.full(got_l.shape, np.nan)
        for b in sorted({0, B // 3, (2 * B) // 3, B - 1}):
            rows, (o, l) = self._oracle_seq(b)
            ro[rows], rl[rows] = o, l
        parity = parity_gate(self.name, got_o, got_l, ro, rl)

        ms = time_calls(torch, step, args.steps, args.warmup)
        split_ms = time_calls(torch, split_only, args.steps, args.warmup)
        lay = amd.decode_workspace_layout(B, ql, mkv, hq, spec.kv_chunk)
        n_p = lay["partials"]
        o_p = ws[lay["off_o"]:lay["off_o"] + 4 * n_p * hq * 64].view(torch.float32).view(n_p, hq, 64)
        l_p = ws[lay["off_lse"]:lay["off_lse"] + 4 * n_p * hq].view(torch.float32).view(n_p, hq)
        indptr = ws[lay["off_indptr"]:lay["off_indptr"] + 4 * (lay["rows"] + 1)].view(torch.int32)
        out2 = torch.empty_like(out)
        merge_ms = time_calls(torch, lambda: amd.attn_sink_merge_partials(o_p, l_p, indptr, out=out2, return_lse=False),
                              args.steps, args.warmup)
        res = {"value": round(self.algo_bytes / (ms * 1e-3) / 1e9, 1), "unit": "GB/s", "ms_per_step": round(ms, 5)}
        res["pct_hbm_peak"] = round(100 * res["value"] / HBM_PEAK_GBS, 2)
        if not args.no_cold:
            cold_ms = cold_time(torch, step, max(20, args.steps), dev)
            res["cold_ms_per_step"] = round(cold_ms, 5)
            res["cold_value"] = round(self.algo_bytes / (cold_ms * 1e-3) / 1e9, 1)
            res["cold_pct_hbm_peak"] = round(100 * res["cold_value"] / HBM_PEAK_GBS, 2)
        achieved = self.kernel_bytes / (split_ms * 1e-3) / 1e9
        res["roofline"] = {"kernel": "decode_split_kernel", "bound": "hbm", "achieved": round(achieved, 1),
                           "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                           "traffic": measured_traffic(self.name, "decode"),
                           "algorithmic_bytes_per_launch": self.kernel_bytes, "kernel_ms": round(split_ms, 5),
                           "merge_ms": round(merge_ms, 5)}
        res["parity_checked"] = True
        res["parity"] = parity
        if self.tree:
            res["tree_overhead"] = self._tree_overhead(torch, amd, args, q, kc, vc, table, lens, sinks, ws, ms,
                                                       split_ms)
        if self.name in ("paged_decode", "paged_decode_tp4") and args.kv_chunk is None:
            res["planner_chunk"] = self._planner_chunk(torch, amd, args, q, kc, vc, table, lens, sinks)
        return res

    def _planner_chunk(self, torch, amd, args, q, kc, vc, table, lens, sinks):
        """Context, not the metric (the workload names 512-token chunks): the same batch with the
        chunk length the library's planner picks for it, output checked against the 512-token call."""
        spec, inp = self.spec, self.inp
        B, ql, hq, mkv = spec.batch, spec.q_len, spec.hq, inp["max_kv_len"]
        chunk = amd.attn_sink_decode_plan_chunk(inp["kv_lens"], ql, hq, spec.hkv, spec.page_size)
        ws = torch.empty(amd.attn_sink_decode_workspace_size(B, ql, mkv, hq, 64, chunk), dtype=torch.uint8, device=q.device)
        out, lse = torch.empty_like(q), torch.empty((B * ql, hq), dtype=torch.float32, device=q.device)
        ref_out, ref_lse = torch.empty_like(q), torch.empty_like(lse)

        def call(c, w, o, l):
            amd.attn_sink_decode_paged(q, kc, vc, table, lens, sinks, ql, mkv, spec.scale, spec.causal, spec.window, c,
                                       workspace=w, out=o, lse=l)

        ws512 = torch.empty(amd.attn_sink_decode_workspace_size(B, ql, mkv, hq, 64, spec.kv_chunk), dtype=torch.uint8,
                            device=q.device)
        call(spec.kv_chunk, ws512, ref_out, ref_lse)
        call(chunk, ws, out, lse)
        torch.cuda.synchronize()
        d_out = float((out.float() - ref_out.float()).abs().max())
        d_lse = float((lse - ref_lse).abs().max())
        if d_out > 2e-2 or d_lse > 2e-3:
            print(f"{self.name}: planner-chunk call differs from the 512-token call (out {d_out}, lse {d_lse})",
                  file=sys.stderr)
            sys.exit(3)
        t = time_calls(torch, lambda: call(chunk, ws, out, lse), args.steps, args.warmup)
        v = self.algo_bytes / (t * 1e-3) / 1e9
        return {"kv_chunk": chunk, "ms_per_step": round(t, 5), "value": round(v, 1),
                "pct_hbm_peak": round(100 * v / HBM_PEAK_GBS, 2), "max_abs_diff_vs_512": round(d_out, 6),
                "what": "context only: the same batch at the chunk attn_sink_decode_plan_chunk picks"}

    def _tree_overhead(self, torch, amd, args, q, kc, vc, table, lens, sinks, ws, tree_ms, tree_split_ms):
        """The same inputs verified as a causal chain (attn_sink_decode_paged, q_len 8): the cost of
        the per-row bitmaps against the causal mask at the same shape."""
        spec, mkv = self.spec, self.inp["max_kv_len"]
        out = torch.empty_like(q)

        def causal_call():
            amd.attn_sink_decode_paged(q, kc, vc, table, lens, sinks, spec.q_len, mkv, spec.scale, True, spec.window,
                                       spec.kv_chunk, workspace=ws, out=out, return_lse=False)

        def causal_split():
            amd.attn_sink_decode_paged_partials(q, kc, vc, table, lens, sinks, spec.q_len, mkv, spec.scale, True,
                                                spec.window, spec.kv_chunk, workspace=ws)

        c_ms = time_calls(torch, causal_call, args.steps, args.warmup)
        c_split = time_calls(torch, causal_split, args.steps, args.warmup)
        return {"tree_ms": round(tree_ms, 5), "causal_chain_ms": round(c_ms, 5),
                "overhead_pct": round(100 * (tree_ms / c_ms - 1), 2),
                "tree_split_ms": round(tree_split_ms, 5), "causal_chain_split_ms": round(c_split, 5),
                "split_overhead_pct": round(100 * (tree_split_ms / c_split - 1), 2),
                "what": "the same q/K/V/pages at q_len 8: random 8-node trees vs the causal chain"}


class Varlen:
    """Packed varlen self-attention: causal / window prefill, embedding batches, tiny case."""

    def __init__(self, name, args):
        self.name = name
        self.specs = [CONFIGS["embed_nosink"], CONFIGS["embed_sink"]] if name == "embed" else [CONFIGS[name]]
        self.spec = self.specs[-1]
        self.inp = make_varlen(self.spec)
        spec, lens = self.spec, self.inp["seqlens"].astype(np.int64)
        self.flops_seq = pairs_visible(lens, spec.causal, spec.window) * 4 * 64 * spec.hq
        self.flops_pass = int(self.flops_seq.sum())
        self.flops = self.flops_pass * len(self.specs)
        T = int(lens.sum())
        self.io_bytes = T * (spec.hq * 64 * 2 * 2 + spec.hkv * 64 * 2 * 2 + spec.hq * 4)
        self.algo_bytes = self.io_bytes * len(self.specs)
        self.long = spec.seqlen[1] >= 1024      # the CPU sample and the gate work on 64-row blocks

    def _sinks(self, s):
        return self.inp["sinks"] if s.sink_std is not None else np.full(s.hq, -np.inf, dtype=np.float32)

    def _oracle(self, s, b, rows=None):
        """oracle.attend on sequence b (the given query rows, else all), NaN-free [Lq or rows]."""
        inp = self.inp
        cu = inp["cu_seqlens"]
        s0, s1 = int(cu[b]), int(cu[b + 1])
        kb, vb = seq_f64(("varlen", b), lambda: (f64(inp["k"][s0:s1]), f64(inp["v"][s0:s1])))
        rows = np.arange(s1 - s0) if rows is None else np.asarray(rows, dtype=np.int64)
        return rows, oracle().attend(f64(inp["q"][s0 + rows]), kb, vb, self._sinks(s), s.scale, s.causal, s.window,
                                     q_pos=rows)

    def cpu_baseline(self, args, workers):
        spec, lens = self.spec, self.inp["seqlens"]
        if self.long:
            n_blk = int(lens.max() + 63) // 64

            def task(i):
                b, blk = i % spec.batch, spread_block(i // spec.batch, n_blk)
                lq = int(lens[b])
                rows = list(range(64 * blk, min(64 * blk + 64, lq)))
                if not rows:
                    return 0.0
                self._oracle(spec, b, rows)
                return float(block_pairs(lq, lq, rows, spec.causal, spec.window) * 4 * 64 * spec.hq)
            v, n, wall = cpu_pool(task, spec.batch * n_blk, args.cpu_seconds, workers)
            what = "blocks of 64 query rows (all heads; sequences and blocks cycled)"
        else:
            def task(b):
                self._oracle(spec, b)
                return float(self.flops_seq[b])
            v, n, wall = cpu_pool(task, spec.batch, args.cpu_seconds, workers)
            what = "whole sequences of this batch (cycled)"
        return cpu_baseline_record(round(v / 1e12, 6), "TFLOP/s", n, wall, workers, what)

    def config(self):
        spec, T = self.spec, int(self.inp["seqlens"].sum())
        return {"workload": f"{self.name}: {spec.batch} seqs, lengths {spec.seqlen[0]}..{spec.seqlen[1]} (sum {T}), "
                            f"{spec.hq}/{spec.hkv} heads, d 64, causal={spec.causal}, window={spec.window}, "
                            f"passes={len(self.specs)}",
                "algorithmic_flops": self.flops, "algorithmic_bytes": self.algo_bytes}

    def gpu(self, torch, amd, args, dev):
        inp, spec = self.inp, self.spec
        q, k, v = (tbits(torch, inp[x], dev) for x in ("q", "k", "v"))
        cu = torch.from_numpy(inp["cu_seqlens"]).to(dev)
        sinks = torch.from_numpy(inp["sinks"]).to(dev)
        out = torch.empty_like(q)
        lse = torch.empty((q.shape[0], spec.hq), dtype=torch.float32, device=dev)
        mx = inp["max_seqlen"]

        def one(s):
            amd.attn_sink_prefill(q, k, v, sinks if s.sink_std is not None else None, cu, cu, mx, mx, s.scale,
                                  s.causal, s.window, out=out, lse=lse)

        def step():
            for s in self.specs:
                one(s)

        # accuracy gate, every pass: sampled rows (a 64-row block of the first and of the last
        # sequence for long sequences, three whole sequences otherwise)
        lens, cu_h = inp["seqlens"], inp["cu_seqlens"]
        B = spec.batch
        gate = None
        for s in self.specs:
            one(s)
            torch.cuda.synchronize()
            got_o, got_l = out_np(out), lse.cpu().numpy().astype(np.float64)
            ro = np.full(got_o.shape, np.nan)
            rl = np.full(got_l.shape, np.nan)
            if self.long:
                picks = [(0, list(range(0, min(64, int(lens[0]))))),
                         (B - 1, list(range(max(0, int(lens[B - 1]) - 64), int(lens[B - 1]))))]
            else:
                picks = [(b, None) for b in sorted({0, B // 2, B - 1})]
            for b, rows in picks:
                rws, (o, l) = self._oracle(s, b, rows)
                idx = int(cu_h[b]) + rws
                ro[idx], rl[idx] = o, l
            rec = parity_gate(self.name, got_o, got_l, ro, rl)
            gate = rec if gate is None else {**rec, "rows": gate["rows"] + rec["rows"],
                                             "max_abs_err": max(gate["max_abs_err"], rec["max_abs_err"]),
                                             "max_excess": max(gate["max_excess"], rec["max_excess"]),
                                             "lse_max_err": max(gate["lse_max_err"], rec["lse_max_err"])}

        ms = time_calls(torch, step, args.steps, args.warmup)
        kernel_ms = ms / len(self.specs)
        tflops = self.flops / (ms * 1e-3) / 1e12
        gbs = self.algo_bytes / (ms * 1e-3) / 1e9
        kname = prefill_kernel_name(spec.window, mx)
        if self.flops / self.algo_bytes > MFMA_BF16_PEAK_TFLOPS / HBM_PEAK_GBS * 1e3:
            roof = {"kernel": kname, "bound": "mfma", "achieved": round(self.flops_pass / (kernel_ms * 1e-3) / 1e12, 2),
                    "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s"}
        else:
            roof = {"kernel": kname, "bound": "hbm", "achieved": round(self.io_bytes / (kernel_ms * 1e-3) / 1e9, 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s"}
        roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
        roof["traffic"] = measured_traffic(self.name, "prefill")
        roof["algorithmic_flops_per_launch"] = self.flops_pass
        roof["algorithmic_bytes_per_launch"] = self.io_bytes
        roof["kernel_ms"] = round(kernel_ms, 5)
        res = {"value": round(tflops, 2), "unit": "TFLOP/s", "ms_per_step": round(ms, 5),
               "pct_mfma_peak": round(100 * tflops / MFMA_BF16_PEAK_TFLOPS, 2), "gb_per_s": round(gbs, 1),
               "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2)}
        if not args.no_cold:
            cold_ms = cold_time(torch, step, max(20, args.steps), dev)
            res["cold_ms_per_step"] = round(cold_ms, 5)
            res["cold_value"] = round(self.flops / (cold_ms * 1e-3) / 1e12, 2)
        res["roofline"] = roof
        res["parity_checked"] = True
        res["parity"] = gate
        return res


class Chunked:
    """Chunked prefill against the paged cache."""

    def __init__(self, name, args):
        self.name = name
        self.spec = spec = CONFIGS[name]
        self.inp = inp = make_paged_prefill(spec)
        self.pairs = np.array([block_pairs(int(lq), int(lk), range(int(lq)), spec.causal, spec.window)
                               for lq, lk in zip(inp["q_lens"], inp["kv_lens"])], dtype=np.int64)
        self.flops = int((self.pairs * 4 * 64 * spec.hq).sum())
        T = int(inp["q_lens"].sum())
        kv_tokens = int(inp["kv_lens"].astype(np.int64).sum())
        pages = int(((inp["kv_lens"].astype(np.int64) + spec.page_size - 1) // spec.page_size).sum())
        self.T, self.kv_tokens = T, kv_tokens
        self.algo_bytes = T * (spec.hq * 64 * 2 * 2 + spec.hq * 4) + kv_tokens * spec.hkv * 64 * 2 * 2 + 4 * pages

    def _oracle(self, b, rows):
        """oracle.prefill_paged on the given chunk rows of sequence b (its pages as a compact pool)."""
        spec, inp = self.spec, self.inp
        cu, lens = inp["cu_seqlens_q"], inp["kv_lens"]
        q0, lq = int(cu[b]), int(cu[b + 1] - cu[b])
        L = int(lens[b])
        pages = inp["page_table"][b, :(L + spec.page_size - 1) // spec.page_size]
        table = np.arange(len(pages), dtype=np.int32)[None, :]
        kc, vc = seq_f64(("chunked", b), lambda: (f64(inp["k_cache"][pages]), f64(inp["v_cache"][pages])))
        rows = np.asarray(rows, dtype=np.int64)
        # only the rows asked for are widened; the oracle reads no other row of q
        qb = np.zeros((lq, spec.hq, 64))
        qb[rows] = f64(inp["q"][q0 + rows])
        o, l = oracle().prefill_paged(qb, kc, vc, table, np.array([0, lq]), lens[b:b + 1], inp["sinks"], spec.scale,
                                      spec.causal, spec.window, rows={0: rows})
        return o[rows], l[rows]

    def cpu_baseline(self, args, workers):
        spec, inp = self.spec, self.inp
        n_blk = int(inp["q_lens"].max() + 63) // 64

        def task(i):
            b, blk = i % spec.batch, spread_block(i // spec.batch, n_blk)
            lq, lk = int(inp["q_lens"][b]), int(inp["kv_lens"][b])
            rows = list(range(64 * blk, min(64 * blk + 64, lq)))
            if not rows:
                return 0.0
            self._oracle(b, rows)
            return float(block_pairs(lq, lk, rows, spec.causal, spec.window) * 4 * 64 * spec.hq)
        v, n, wall = cpu_pool(task, spec.batch * n_blk, args.cpu_seconds, workers)
        return cpu_baseline_record(round(v / 1e12, 6), "TFLOP/s", n, wall, workers,
                                   "blocks of 64 chunk rows (all heads; sequences and blocks cycled)")

    def config(self):
        spec = self.spec
        return {"workload": f"{self.name}: {spec.batch} seqs, chunks of {spec.q_len[0]}..{spec.q_len[1]} tokens on "
                            f"{spec.ctx_len[0]}..{spec.ctx_len[1]} cached (sum {self.T} queries, {self.kv_tokens} "
                            f"keys), {spec.hq}/{spec.hkv} heads, d 64, {spec.page_size}-token pages, "
                            f"causal={spec.causal}",
                "algorithmic_flops": self.flops, "algorithmic_bytes": self.algo_bytes}

    def gpu(self, torch, amd, args, dev):
        spec, inp = self.spec, self.inp
        q, kc, vc = (tbits(torch, inp[x], dev) for x in ("q", "k_cache", "v_cache"))
        table = torch.from_numpy(inp["page_table"]).to(dev)
        cu = torch.from_numpy(inp["cu_seqlens_q"]).to(dev)
        lens = torch.from_numpy(inp["kv_lens"]).to(dev)
        sinks = torch.from_numpy(inp["sinks"]).to(dev)
        out = torch.empty_like(q)
        lse = torch.empty((q.shape[0], spec.hq), dtype=torch.float32, device=dev)

        def step():
            amd.attn_sink_prefill_paged(q, kc, vc, table, cu, lens, sinks, inp["max_q"], inp["max_kv_len"],
                                        spec.scale, spec.causal, spec.window, out=out, lse=lse)

        step()
        torch.cuda.synchronize()
        got_o, got_l = out_np(out), lse.cpu().numpy().astype(np.float64)
        ro = np.full(got_o.shape, np.nan)
        rl = np.full(got_l.shape, np.nan)
        B = spec.batch
        for b, first in ((0, True), (B - 1, False)):
            lq = int(inp["q_lens"][b])
            rows = np.arange(0, min(64, lq)) if first else np.arange(max(0, lq - 64), lq)
            o, l = self._oracle(b, rows)
            q0 = int(inp["cu_seqlens_q"][b])
            ro[q0 + rows], rl[q0 + rows] = o, l
        parity = parity_gate(self.name, got_o, got_l, ro, rl)

        ms = time_calls(torch, step, args.steps, args.warmup)
        tflops = self.flops / (ms * 1e-3) / 1e12
        gbs = self.algo_bytes / (ms * 1e-3) / 1e9
        kname = prefill_kernel_name(spec.window, inp["max_q"])
        if self.flops / self.algo_bytes > MFMA_BF16_PEAK_TFLOPS / HBM_PEAK_GBS * 1e3:
            roof = {"kernel": kname, "bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s"}
        else:
            roof = {"kernel": kname, "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s"}
        roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
        roof["traffic"] = measured_traffic(self.name, "prefill")
        roof["algorithmic_flops_per_launch"] = self.flops
        roof["algorithmic_bytes_per_launch"] = self.algo_bytes
        roof["kernel_ms"] = round(ms, 5)
        res = {"value": round(tflops, 2), "unit": "TFLOP/s", "ms_per_step": round(ms, 5),
               "pct_mfma_peak": round(100 * tflops / MFMA_BF16_PEAK_TFLOPS, 2), "gb_per_s": round(gbs, 1),
               "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2)}
        if not args.no_cold:
            cold_ms = cold_time(torch, step, max(20, args.steps), dev)
            res["cold_ms_per_step"] = round(cold_ms, 5)
            res["cold_value"] = round(self.flops / (cold_ms * 1e-3) / 1e12, 2)
        res["roofline"] = roof
        res["parity_checked"] = True
        res["parity"] = parity
        return res


class Rope:
    """YaRN rotary encoding of the chunked-prefill workload's new tokens and their append into the
    paged cache."""

    def __init__(self, name, args):
        self.name = name
        self.spec = spec = CONFIGS["chunked_prefill"]
        self.inp = inp = make_paged_prefill(spec)
        T = int(inp["cu_seqlens_q"][-1])
        rng = np.random.default_rng(11)
        self.k_new = bf16_round_bits(rng.standard_normal((T, spec.hkv, 64)).astype(np.float32))
        self.v_new = bf16_round_bits(rng.standard_normal((T, spec.hkv, 64)).astype(np.float32))
        q_lens = inp["q_lens"].astype(np.int64)
        row_bytes = (spec.hq * 64 * 2) * 2 + (spec.hkv * 64 * 2) * 4     # q in + out, k/v in + cache out
        self.bytes_seq = q_lens * row_bytes + q_lens * 4                 # + one page id per token
        self.algo_bytes = int(self.bytes_seq.sum() + 4 * (2 * spec.batch + 1))
        self.T = T

    def _oracle_seq(self, b):
        inp, P = self.inp, self.inp["k_cache"].shape[2]
        cu, lens = inp["cu_seqlens_q"], inp["kv_lens"]
        L = int(lens[b])
        pages = inp["page_table"][b, :(L + P - 1) // P]
        r0, r1 = int(cu[b]), int(cu[b + 1])
        freqs, m = oracle().yarn_frequencies(64, ROPE_ARGS["rope_theta"], ROPE_ARGS["yarn_factor"],
                                             ROPE_ARGS["yarn_original_len"], ROPE_ARGS["yarn_alpha"],
                                             ROPE_ARGS["yarn_beta"], ramp="turns")
        return pages, r0, r1, oracle().rope_append(f64(inp["q"][r0:r1]), f64(self.k_new[r0:r1]),
                                                   f64(self.v_new[r0:r1]), np.array([0, r1 - r0]), lens[b:b + 1],
                                                   np.arange(len(pages))[None, :], f64(inp["k_cache"][pages]),
                                                   f64(inp["v_cache"][pages]), freqs, m)

    def cpu_baseline(self, args, workers):
        def task(b):
            self._oracle_seq(b)
            return float(self.bytes_seq[b])
        v, n, wall = cpu_pool(task, self.spec.batch, args.cpu_seconds, workers)
        return cpu_baseline_record(round(v / 1e9, 4), "GB/s", n, wall, workers,
                                   "sequences' chunks (each worker from its own start, cycling)")

    def config(self):
        spec = self.spec
        return {"workload": f"{self.name}: YaRN rotary encoding (theta 150000, factor 32, original 4096, ramp over "
                            f"the turns) of {self.T} new tokens ({spec.batch} chunks of 2048 on 0..6144 cached), "
                            f"{spec.hq}/{spec.hkv} heads, d 64, K/V appended into 16-token pages",
                "algorithmic_bytes": self.algo_bytes}

    def gpu(self, torch, amd, args, dev):
        spec, inp = self.spec, self.inp
        q, kn, vn = tbits(torch, inp["q"], dev), tbits(torch, self.k_new, dev), tbits(torch, self.v_new, dev)
        kc, vc = tbits(torch, inp["k_cache"], dev), tbits(torch, inp["v_cache"], dev)
        cu = torch.from_numpy(inp["cu_seqlens_q"]).to(dev)
        lens = torch.from_numpy(inp["kv_lens"]).to(dev)
        table = torch.from_numpy(inp["page_table"]).to(dev)
        q_out = torch.empty_like(q)

        def step():
            amd.attn_sink_rope_append(q, kn, vn, cu, lens, table, kc, vc, inp["max_q"], inp["max_kv_len"],
                                      q_out=q_out, yarn_ramp="turns", **ROPE_ARGS)

        step()
        torch.cuda.synchronize()
        # gate: rotated q rows and the appended K/V of two sequences (every call writes the same
        # values, so the timed calls leave the caches as checked here)
        P = spec.page_size
        got_q = out_np(q_out)
        excess, rows = -np.inf, 0
        for b in (0, spec.batch - 1):
            pages, r0, r1, (rq, rk, rv) = self._oracle_seq(b)
            excess = max(excess, float((np.abs(got_q[r0:r1] - rq) - (ATOL + RTOL * np.abs(rq))).max()))
            idx = torch.from_numpy(pages.astype(np.int64)).to(dev)
            kc_b, vc_b = out_np(kc[idx]), out_np(vc[idx])
            L = int(inp["kv_lens"][b])
            pos = np.arange(L - (r1 - r0), L)
            gk, ek = kc_b[pos // P, :, pos % P], rk[pos // P, :, pos % P]
            excess = max(excess, float((np.abs(gk - ek) - (ATOL + RTOL * np.abs(ek))).max()))
            v_err = float(np.abs(vc_b[pos // P, :, pos % P] - rv[pos // P, :, pos % P]).max())
            excess = max(excess, v_err if v_err > 0 else -1.0)     # v is copied: exact
            rows += r1 - r0
        parity = {"rows": rows, "max_excess": round(excess, 6),
                  "bar": "|err| <= 1e-2 + 1e-2 |ref| (q, k); v copied exactly"}
        if not excess <= 0:
            print(json.dumps({"error": f"{self.name}: parity gate failed before timing", "parity": parity}),
                  file=sys.stderr)
            sys.exit(3)

        ms = time_calls(torch, step, args.steps, args.warmup)
        gbs = self.algo_bytes / (ms * 1e-3) / 1e9
        res = {"value": round(gbs, 1), "unit": "GB/s", "ms_per_step": round(ms, 5),
               "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2)}
        if not args.no_cold:
            cold_ms = cold_time(torch, step, max(20, args.steps), dev)
            res["cold_ms_per_step"] = round(cold_ms, 5)
            res["cold_value"] = round(self.algo_bytes / (cold_ms * 1e-3) / 1e9, 1)
        res["roofline"] = {"kernel": "rope_append_kernel", "bound": "hbm", "achieved": round(gbs, 1),
                           "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                           "traffic": measured_traffic(self.name, "rope"),
                           "algorithmic_bytes_per_launch": self.algo_bytes, "kernel_ms": round(ms, 5)}
        res["parity_checked"] = True
        res["parity"] = parity
        return res


def make_workload(name, args):
    if name in DECODE_WORKLOADS:
        return Paged(name, args)
    if name == "chunked_prefill":
        return Chunked(name, args)
    if name == "rope_append":
        return Rope(name, args)
    return Varlen(name, args)


def main():
    args = parse()
    if args.record_traffic:
        record_traffic("paged_decode" if args.workload == "default" else args.workload, *args.record_traffic)
        return
    if args.summarize:
        summarize(*args.summarize, args.summary_command, args.summary_workload)
        return
    if args.pmc_table:
        pmc_table(*args.pmc_table)
        return
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported (it measures the "
              f"one-GPU shard of the path).", file=sys.stderr)
        sys.exit(2)
    import torch
    if torch.cuda.device_count() < 1:       # counts devices without initialising the GPU
        print("bench.py needs a GPU (HIP device)", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0").fill_(3)
        for _ in range(3):
            b = a.clone()
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "copy", "bytes_read": 1 << 30, "bytes_written": 1 << 30}))
        return

    names = ["paged_decode", "causal_prefill"] if args.workload == "default" else [args.workload]
    work = [make_workload(n, args) for n in names]
    # The CPU oracle runs first, in processes forked before the GPU is initialised.
    cpu = {}
    if not args.no_cpu_baseline:
        workers = cpu_workers(args)
        for w in work:
            cpu[w.name] = w.cpu_baseline(args, workers)

    import gqa_attention_sinks_sink_amd as amd
    dev = torch.device("cuda:0")
    results = []
    for w in work:
        r = w.gpu(torch, amd, args, dev)
        r["config"] = w.config()
        if w.name in cpu:
            r["cpu_baseline"] = cpu[w.name]
        results.append(r)

    head = results[0]
    line = {"metric": METRIC, "value": head["value"], "unit": head["unit"], "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic", "config": head["config"]}
    line.update({k: v for k, v in head.items() if k not in line})
    if len(results) > 1:
        line["prefill"] = results[1]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
