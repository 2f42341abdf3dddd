#!/usr/bin/env python3
"""Benchmark: MLA speculative-decoding verify attention on one MI355X.

One step = one verify_attn() call (split + merge kernels) over the
long-context workload by default: 1 sequence, 64 heads, 16 verify positions in
a causal chain, prefix 185,000, page_size 1 with shuffled kv_indices into a
512k-slot pool, bf16 N(0,1) latents, q = 0.5 N(0,1), scale 1/sqrt(192)
(--config picks another workload). Inputs are seeded and synthetic and are
resident in HBM before timing starts.

Before each cold call a 1 GiB read evicts the caches (the 256 MiB last-level
cache would otherwise hold most of the 213 MB KV working set); call and split
kernel times come from HIP events on the call's stream. The JSON line reports
us/call (lower is better), algorithmic HBM GB/s against 8 TB/s, the split
kernel's roofline fraction (MFMA or HBM, whichever binds the workload), and
the fp64 CPU oracle timed on a bounded sample of the same workload.

--summarize-trace CSV turns a rocprofv3 kernel trace of a bench run into the
per-kernel averages of the timed calls alone (warmup calls dropped, cold and
warm calls apart), for the profile summaries.
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

METRIC = "verify-attn µs/call + achieved HBM GB/s (% of peak), 64 heads, 185k prefix"   # the long185k line
PEAK_HBM = 8.0e12            # MI355X HBM3E, bytes/s
PEAK_MFMA_BF16 = 2.5e15      # MI355X dense bf16/fp16 MFMA, FLOP/s
FLOP_PER_PAIR = 2 * (576 + 512)   # q.k over 576 dims + p*v over 512 dims, per visible (row, key)
KERNEL_SRC = os.path.join(ROOT, "speculative_decoding_verify_03_amd", "csrc", "verify_attn_kernels.hip")
PMC_SUMMARY = os.path.join(ROOT, "profiles", "split_kernel_long185k_pmc.json")

WORKLOAD_TEXT = {
    "long185k": "B=1 H=64 Q=16 prefix=185000 causal chain; page_size 1, kv_indices = first 185016 of a "
                "seeded permutation of a 524288-slot pool; bf16 latents N(0,1), q 0.5*N(0,1), scale 1/sqrt(192)",
    "long185k_h8": "B=1 H=8 Q=16 prefix=185000 causal chain (per-rank shape of 8-way head sharding); "
                   "524288-slot pool, shuffled kv_indices; bf16 N(0,1), q 0.5*N(0,1)",
    "p4k": "B=1 H=64 Q=16 prefix=4096 causal chain, contiguous kv_indices; bf16 N(0,1)",
    "tree32k": "B=1 H=64 Q=16 prefix=32768 random draft tree (depth<=8), 262144-slot pool, shuffled",
    "batch8": "B=8 H=64 Q=8 prefixes U[1024,131072], random draft trees, 2097152-slot pool, shuffled",
    "tiny": "B=1 H=8 Q=4 prefix=256 causal chain, 1024-slot pool, shuffled",
    "long185k_contig": "long185k over a defragmented cache: contiguous kv_indices (arange), 185016-slot pool",
    "long185k_h8_contig": "long185k_h8 over a defragmented cache: contiguous kv_indices (arange), 185016-slot pool",
}


def metric_for(name: str, w) -> str:
    """The metric string of a bench line, naming the workload actually run (the 64-head,
    185k-prefix workload keeps the headline metric's own wording)."""
    if name == "long185k":
        return METRIC
    prefix = (f"{int(w.prefix_lens[0])} prefix" if w.B == 1 else
              f"{w.B} sequences, prefixes {int(w.prefix_lens.min())}..{int(w.prefix_lens.max())}")
    return f"verify-attn µs/call + achieved HBM GB/s (% of peak), {w.H} heads, {w.Q} verify positions, {prefix}"


def algorithmic_bytes(w) -> int:
    """HBM bytes a perfect implementation moves once: KV rows, indices, q, mask, lengths, out, lse."""
    B, Q, H = w.B, w.Q, w.H
    kv = int(w.total_kv) * 1152
    return (kv + w.total_kv * 4 + B * Q * H * 1152 + B * Q * Q + B * 4
            + B * Q * H * 512 * 4 + B * Q * H * 4)


def visible_pairs(w) -> int:
    """Number of visible (query-head row, key) pairs."""
    tot = 0
    for b in range(w.B):
        P = int(w.prefix_lens[b])
        per_query = P + w.tree_mask[b].astype(np.int64).sum(axis=1)
        tot += int(per_query.sum()) * w.H
    return tot


def kernel_sha() -> str:
    """Digest of the kernel source with comments and blank lines removed, so that the
    committed counter summary stays tied to the code it was taken on."""
    import re
    with open(KERNEL_SRC) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = [ln.split("//", 1)[0].rstrip() for ln in text.splitlines()]
    code = "\n".join(ln for ln in lines if ln.strip())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per split launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source and on this workload (else None)."""
    try:
        with open(PMC_SUMMARY) as f:
            s = json.load(f)
    except (OSError, ValueError):
        return None
    if s.get("kernel_sha") != kernel_sha() or s.get("workload") != workload:
        return None
    return s.get("traffic_bytes_per_launch")


def cpu_baseline(w, heads, min_seconds=10.0, max_reps=20):
    """The fp64 oracle (as is) on the same workload, repeated until at least
    `min_seconds` of CPU work have run, reported per call."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([t.get("num_threads", 1) for t in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = None
    t0 = time.perf_counter()
    reps = 0
    while reps < max_reps and (reps == 0 or time.perf_counter() - t0 < min_seconds):
        oracle.verify_attention(w.q, w.kv_pool, w.kv_indices, w.prefix_lens, w.tree_mask, w.scale,
                                heads=heads)
        reps += 1
    total = time.perf_counter() - t0
    dt = total / reps
    scale_up = w.H / len(heads)
    what = "all heads" if len(heads) == w.H else f"heads {heads} of {w.H}, scaled by {scale_up:g}"
    return {
        "value": round(dt * scale_up * 1e6, 1),
        "unit": "µs/call",
        "cores": blas_threads if blas_threads else len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": f"oracle.verify_attention on the same workload ({what}), {reps} calls in "
                  f"{total:.1f} s; host has {len(os.sched_getaffinity(0))} usable cores ({cpu_model()})",
    }


def cpu_model() -> str:
    """The host CPU's model name, as /proc/cpuinfo gives it (or 'unknown CPU')."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


class Evictor:
    """Evicts the caches (L2 and the last-level cache) before a cold call by
    reading a 1 GiB buffer: a reduction whose 4-byte result is dropped. A read
    leaves no dirty lines behind; a 1 GiB fill would leave the last-level cache
    full of dirty lines, whose write-back then competes with the timed call."""

    def __init__(self, torch, dev):
        self.buf = torch.zeros(1 << 28, dtype=torch.float32, device=dev)

    def __call__(self):
        self.buf.sum()


def _event_times(torch, fn, steps, flush=None):
    """Mean and median µs of `fn` over `steps` calls timed with HIP events on the
    current stream (each preceded by a cache eviction when `flush` is given)."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in ev:
        if flush is not None:
            flush()
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    t = np.array([e0.elapsed_time(e1) for e0, e1 in ev]) * 1e3
    return float(t.mean()), float(np.median(t))


def bench_defrag(args, torch, va) -> int:
    """KV defragmentation of the 185k-prefix workload's 185,016 positions into a
    contiguous run: µs/call and algorithmic HBM GB/s (row read + row write + index
    read + index write per position) against 8 TB/s; the oracle as CPU baseline."""
    from workloads import make_config
    w = make_config(args.config)
    dev = torch.device("cuda:0")
    src = torch.from_numpy(w.kv_pool.view(np.int16)).to(dev)
    idx = torch.from_numpy(w.kv_indices).to(dev)
    n = int(w.total_kv)
    dst = torch.empty((n, 576), dtype=torch.int16, device=dev)
    new_idx = torch.empty(n, dtype=torch.int32, device=dev)
    flush = Evictor(torch, dev)

    def call():
        va.kv_defrag(src, idx, dst, 0, new_indices=new_idx)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    cold, cold_med = _event_times(torch, call, args.steps, flush)
    warm, _ = _event_times(torch, call, args.steps)
    nbytes = n * (2 * 1152 + 8)
    res = {
        "metric": "kv-defrag µs/call + achieved HBM GB/s (% of peak)", "value": round(cold, 2), "unit": "µs/call",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(cold / 1e3, 5),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "u8", "data": "synthetic",
        "config": {"workload": f"{args.config}: {n} positions, pool rows of 1152 B, shuffled slots, "
                               "copied into a contiguous run", "cache_flush_between_calls": True},
        "us_per_call_median": round(cold_med, 2), "us_per_call_warm": round(warm, 2),
        "algorithmic_bytes": nbytes,
        "roofline": {"bound": "hbm", "achieved": round(nbytes / (cold * 1e-6) / 1e9, 1), "peak": PEAK_HBM / 1e9,
                     "unit": "GB/s", "frac": round(nbytes / (cold * 1e-6) / PEAK_HBM, 4), "traffic": None,
                     "kernel": "defrag_kernel"},
    }
    if not args.no_cpu_baseline:
        import oracle
        t0 = time.perf_counter()
        reps = 0
        while reps == 0 or time.perf_counter() - t0 < 5.0:
            oracle.defrag(w.kv_pool, w.kv_indices, np.zeros((n, 576), np.uint16), 0)
            reps += 1
        dt = (time.perf_counter() - t0) / reps
        res["cpu_baseline"] = {"value": round(dt * 1e6, 1), "unit": "µs/call", "cores": 1, "kind": "oracle",
                               "sample": f"oracle.defrag on all {n} positions, {reps} calls, {dt:.2f} s each"}
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)
    return 0


def bench_tree_accept(args, torch, va) -> int:
    """Greedy acceptance over 256 draft trees of 64 nodes (depth <= 8): µs/call
    (launch-latency bound); the oracle as CPU baseline."""
    from workloads import make_tree_accept_case
    B, Q = 256, 64
    par, dr, tg = make_tree_accept_case(700, B, Q, vocab=8, p_follow=0.9)
    dev = torch.device("cuda:0")
    ins = [torch.from_numpy(a).to(dev) for a in (par, dr, tg)]
    out = va.tree_accept(*ins)

    def call():
        va.tree_accept(*ins, out=out)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    mean, med = _event_times(torch, call, args.steps)
    res = {
        "metric": "tree-accept µs/call", "value": round(mean, 2), "unit": "µs/call", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(mean / 1e3, 5),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "int32", "data": "synthetic",
        "config": {"workload": f"B={B} draft trees of Q={Q} nodes, depth <= 8, vocabulary 8, target follows a "
                               "child with p=0.9"},
        "us_per_call_median": round(med, 2),
        "roofline": {"bound": "latency", "achieved": None, "peak": None, "unit": None, "frac": None,
                     "traffic": None, "kernel": "tree_accept_kernel"},
    }
    if not args.no_cpu_baseline:
        import oracle
        t0 = time.perf_counter()
        reps = 0
        while reps == 0 or time.perf_counter() - t0 < 2.0:
            oracle.tree_accept_batch(par, dr, tg)
            reps += 1
        dt = (time.perf_counter() - t0) / reps
        res["cpu_baseline"] = {"value": round(dt * 1e6, 1), "unit": "µs/call", "cores": 1, "kind": "oracle",
                               "sample": f"oracle.tree_accept_batch on the same inputs, {reps} calls"}
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)
    return 0


def summarize_trace(path: str, config: str, warmup: int, steps: int) -> str:
    """Markdown summary of a rocprofv3 kernel-trace CSV of `bench.py --config config
    --warmup W --steps K`: the split and merge kernels of the timed calls only. The run
    makes W warmup steps, then K timed steps, each of four calls (cold call, cold
    split-kernel timing, warm call, warm split-kernel timing); each call is one split
    and one merge dispatch, in that order."""
    import csv
    rows = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Start_Timestamp"]))
    split = [r for r in rows if "split_kernel" in r["Kernel_Name"]]
    merge = [r for r in rows if "merge" in r["Kernel_Name"] and "va" in r["Kernel_Name"]]
    first = 4 * warmup   # calls of the warmup steps
    n = first + 4 * steps
    if len(split) != n or len(merge) != n:
        raise SystemExit(f"expected {n} split and merge dispatches, found {len(split)} and {len(merge)}")
    dur = lambda r: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3  # noqa: E731
    kinds = {"cold": (0, 1), "warm": (2, 3)}
    w = None
    out = [f"Timed calls only: the first {first} calls ({warmup} warmup steps) are dropped; {steps} steps of four calls "
           "remain (cold call, cold split-kernel timing, warm call, warm split-kernel timing).", "",
           "| kernel | calls | kind | avg us | min us | max us |", "|---|---:|---|---:|---:|---:|"]
    stats = {}
    for kind, idx in kinds.items():
        sel = [first + 4 * k + i for k in range(steps) for i in idx]
        for name, lst in (("split_kernel", split), (merge[0]["Kernel_Name"].split("(")[0], merge)):
            d = np.array([dur(lst[i]) for i in sel])
            stats[(name, kind)] = d
            short = next((k for k in ("split_kernel", "merge_few_kernel", "merge_slice_kernel", "merge_kernel") if k in name), name)
            out.append(f"| {short} | {len(d)} | {kind} | {d.mean():.2f} | {d.min():.2f} | {d.max():.2f} |")
        calls = np.array([(int(merge[i]["End_Timestamp"]) - int(split[i]["Start_Timestamp"])) / 1e3 for i in sel])
        out.append(f"| whole call (split start to merge end) | {len(calls)} | {kind} | {calls.mean():.2f} | "
                   f"{calls.min():.2f} | {calls.max():.2f} |")
        stats[("call", kind)] = calls
    from workloads import make_config
    w = make_config(config)
    flops = visible_pairs(w) * FLOP_PER_PAIR
    split_bytes = int(w.total_kv) * 1152
    cold = float(stats[("split_kernel", "cold")].mean())
    if flops / PEAK_MFMA_BF16 >= split_bytes / PEAK_HBM:
        a = flops / (cold * 1e-6) / 1e12
        roof = f"MFMA-bound: {flops} FLOP per launch / {cold:.2f} us = {a:.1f} TFLOP/s, frac {a * 1e12 / PEAK_MFMA_BF16:.4f} of 2500 TFLOP/s"
    else:
        a = split_bytes / (cold * 1e-6) / 1e9
        roof = f"HBM-bound: {split_bytes} B of KV rows per launch / {cold:.2f} us = {a:.1f} GB/s, frac {a * 1e9 / PEAK_HBM:.4f} of 8000 GB/s"
    out += ["", f"Roofline of the split kernel from the cold average above: {roof}."]
    return "\n".join(out)


def copy_calibration(nbytes: int = 1 << 30, reps: int = 3) -> None:
    """A plain device copy of known size, for scaling rocprofv3 FETCH_SIZE/WRITE_SIZE."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "reps": reps}), flush=True)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--config", default="long185k", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-flush", action="store_true", help="skip the cache eviction between calls")
    ap.add_argument("--chunk", type=int, default=0, help="keys-per-chunk override (0 = automatic)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--summarize-trace", metavar="CSV", default=None,
                    help="print the timed-call summary of a rocprofv3 kernel trace of a bench run made with "
                         "the same --config, --warmup and --steps, and exit (no GPU needed)")
    ap.add_argument("--op", default="attn", choices=["attn", "defrag", "tree_accept"],
                    help="attn (default): the verify-attention call; defrag / tree_accept: the steps next "
                         "to it, each with its own metric line")
    args = ap.parse_args()

    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace, args.config, args.warmup, args.steps))
        return 0

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the one-GPU value is the per-GPU share; sharding is described in the design notes)",
              file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    if args.copy_calibration:
        copy_calibration()
        return 0

    import speculative_decoding_verify_03_amd as va
    from workloads import make_config
    if args.op == "defrag":
        return bench_defrag(args, torch, va)
    if args.op == "tree_accept":
        return bench_tree_accept(args, torch, va)

    print(f"[bench] generating workload {args.config}", file=sys.stderr, flush=True)
    w = make_config(args.config)
    dev = torch.device("cuda:0")
    q = torch.from_numpy(w.q.view(np.int16)).to(dev)
    kv = torch.from_numpy(w.kv_pool.view(np.int16)).to(dev)
    idx = torch.from_numpy(w.kv_indices).to(dev)
    pl = torch.from_numpy(w.prefix_lens).to(dev)
    tm = torch.from_numpy(w.tree_mask).to(dev)
    plan = va.query_plan(w.B, w.Q, w.H, w.total_kv, chunk_keys=args.chunk)
    ws = va.alloc_workspace(w.B, w.Q, w.H, w.total_kv, device=dev, chunk_keys=args.chunk)
    out = torch.empty((w.B, w.Q, w.H, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((w.B, w.Q, w.H), dtype=torch.float32, device=dev)
    flush = None if args.no_flush else Evictor(torch, dev)
    scale = float(w.scale)

    def call(split_events=None):
        va.verify_attn(q, kv, idx, pl, tm, scale, out=out, lse=lse, workspace=ws, chunk_keys=args.chunk,
                       split_events=split_events)

    def timed(n, do_flush):
        """n timed steps. Each step makes four calls, so that any drift of the
        GPU's clocks during the run affects every figure alike: a cold call (after
        a cache eviction when do_flush), a cold call timing the split kernel alone,
        then a warm call and a warm split-kernel timing (each right after the
        previous call). Whole calls are timed from the library's event before its
        first launch (the split kernel) to an event after the call; split-kernel
        timings use the library's event pair around that launch. Returns the four
        arrays (us) and the wall time of the loop."""
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(8)] for _ in range(n)]
        for e in ev:          # torch creates the HIP events on first record; the
            for x in e:       # library then re-records them inside the calls
                x.record()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(n):
            e = ev[k]
            for j, cold in ((0, True), (4, False)):
                if cold and do_flush:
                    flush()
                call(split_events=(e[j], None))
                e[j + 1].record()
                if cold and do_flush:
                    flush()
                call(split_events=(e[j + 2], e[j + 3]))
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        t = lambda i: np.array([x[i].elapsed_time(x[i + 1]) for x in ev]) * 1e3  # noqa: E731
        return t(0), t(2), t(4), t(6), wall

    # Warmup steps run the timed pattern, evictions included: the 1 GiB reads
    # change the GPU's power state, and its clocks take tens of calls to
    # settle after they start (a warmup of plain calls left the first timed
    # calls up to 25% slower than the later ones).
    print(f"[bench] plan {plan}; warmup {args.warmup} steps", file=sys.stderr, flush=True)
    timed(args.warmup, flush is not None)
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    calls, splits, warm_calls, warm_splits, wall = timed(args.steps, flush is not None)

    us = float(calls.mean())
    abytes = algorithmic_bytes(w)
    flops = visible_pairs(w) * FLOP_PER_PAIR
    split_us = float(splits.mean())
    achieved_tflops = flops / (split_us * 1e-6) / 1e12
    # The split kernel's binding roof: matrix cores when there are enough
    # query-head rows per latent row (64 heads), HBM when there are few (8).
    split_bytes = int(w.total_kv) * 1152
    if flops / PEAK_MFMA_BF16 >= split_bytes / PEAK_HBM:
        roof = {"bound": "mfma", "achieved": round(achieved_tflops, 1), "peak": PEAK_MFMA_BF16 / 1e12,
                "unit": "TFLOP/s", "frac": round(achieved_tflops * 1e12 / PEAK_MFMA_BF16, 4)}
    else:
        gbps = split_bytes / (split_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM / 1e9,
                "unit": "GB/s", "frac": round(gbps * 1e9 / PEAK_HBM, 4)}
    result = {
        "metric": metric_for(args.config, w),
        "value": round(us, 2),
        "unit": "µs/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.config}: {WORKLOAD_TEXT[args.config]}",
                   "plan": plan, "cache_flush_between_calls": flush is not None},
        "hbm_gbps": round(abytes / (us * 1e-6) / 1e9, 1),
        "hbm_frac": round(abytes / (us * 1e-6) / PEAK_HBM, 4),
        "algorithmic_bytes": abytes,
        "algorithmic_flops": flops,
        "us_per_call_median": round(float(np.median(calls)), 2),
        "us_per_call_warm": round(float(warm_calls.mean()), 2),
        "split_kernel_us": round(split_us, 2),
        "split_kernel_us_warm": round(float(warm_splits.mean()), 2),
        "wall_ms_per_step_of_4_calls": round(wall / args.steps * 1e3, 4),
        "roofline": dict(roof, traffic=measured_traffic(args.config), kernel="split_kernel"),
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w, heads=list(range(w.H)))
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
