"""Benchmark of the paged MLA KV-cache gather on one MI355X.

One step = one call of the library on one batch (all of the hot path: page-task
build, block lookup, page copy / dequant), inputs already resident in HBM.
Headline workload: one request of 307,200 tokens (4,800 pages of 64), 576 fp8
e4m3fn codes per token upconverted to bf16 with a per-tensor scale, shuffled
physical blocks.  The same run also times, with the same steps and warmup,
the second single-request gather (61,440 bf16 tokens, raw copy) and the
indexer quant-cache gather (307,200 rows of 128 value bytes and a 4-byte
scale, flat records), each reported as a nested object under its workload
name.  Metric: effective HBM GB/s (algorithmic bytes read +
written per step / time per step).

Timing: exactly K back-to-back calls bracketed by torch.cuda.synchronize(),
with one HIP event pair on the launch stream around them.  `value` and
`ms_per_step` come from the events (the GPU time of the K calls); a short spin
kernel enqueued before the first event keeps the GPU busy while the host
enqueues the first calls, so the events see the calls back to back.
`wall_ms_per_step` is the host clock over the same bracket, which adds the two
synchronisation latencies and the spin.  The timed steps rotate over several copies of the
inputs and outputs whose total is far above the 256 MB Infinity Cache, so no
step finds its data in a cache.  Each workload also reports one cold call's
latency (median, p10, p90 of 100: a 1 GiB fill or read, then events around one
call) and the GB/s at that median; a single call timed on its own carries the
launch's own fixed cost (an empty kernel takes about 6 us that way).  Printed
on stdout: ONE JSON line.  Progress goes to stderr.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--also NAME,NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

REPO = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, REPO)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published peak
SPACER_CYCLES = 200_000  # GPU clock cycles of the spin before the timed calls (tens of us)
METRIC = "effective HBM GB/s (read+write) and % of peak; median gather latency, 1 GPU"
DEFAULT_WORKLOAD = "single_300k_fp8_upconvert"
ALSO_WORKLOADS = ("single_60k_raw", "indexer_single_300k_flat")
TRAFFIC_DIR = os.path.join(REPO, "profiles")
KERNEL_SOURCES = ["paged_kv_cache_device_amd/csrc/gather_kernels.hpp",
                  "paged_kv_cache_device_amd/csrc/indexer_kernels.hpp",
                  "paged_kv_cache_device_amd/csrc/pkvg_capi.hip"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _code_only(text: str) -> str:
    """C++ source without comments and with whitespace collapsed: edits that
    cannot change the compiled code do not change the hash."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash() -> str:
    """Fingerprint of what the kernels are built from: the HIP sources (code
    only) and the compiler flags."""
    from paged_kv_cache_device_amd import build

    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(REPO, rel)) as f:
            h.update(_code_only(f.read()).encode())
    h.update(repr(build.HIPCC_FLAGS).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None."""
    path = os.path.join(TRAFFIC_DIR, f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def summarize_counters(prof_dir: str, workload: str, calib_mib: int, command: str) -> dict:
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE; files
    fetch_counter_collection.csv and write_counter_collection.csv in prof_dir)
    into HBM bytes per gather launch.  Each counter is scaled by what it reads
    for the plain device copies of `calib_mib` MiB that the run ends with (the
    last 10 copy-kernel dispatches), and the result is written to
    profiles/traffic_<workload>.json together with the kernel-source hash."""
    import csv

    import workloads

    def rows(kind):
        with open(os.path.join(prof_dir, f"{kind}_counter_collection.csv")) as f:
            return sorted(csv.DictReader(f), key=lambda r: int(r["Dispatch_Id"]))

    out = {}
    for kind, counter in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
        rs = [r for r in rows(kind) if r["Counter_Name"] == counter]
        gather = [float(r["Counter_Value"]) for r in rs
                  if any(k in r["Kernel_Name"] for k in GATHER_KERNELS)]
        copies = [float(r["Counter_Value"]) for r in rs if "copyBuffer" in r["Kernel_Name"]][-10:]
        known = calib_mib << 20
        factor = known / (statistics.median(copies) * 1024.0)
        out[kind] = {"counter": counter, "gather_kib_median": statistics.median(gather),
                     "launches": len(gather), "calibration_kib_median": statistics.median(copies),
                     "calibration_bytes": known, "scale": round(factor, 5),
                     "bytes_per_launch": statistics.median(gather) * 1024.0 * factor}
    wl = workloads.named(workload)
    total = out["fetch"]["bytes_per_launch"] + out["write"]["bytes_per_launch"]
    res = {"workload": workload, "kernel_source_sha": kernel_source_hash(),
           "hbm_bytes_per_launch": round(total), "algorithmic_bytes": wl.algorithmic_bytes(),
           "traffic_over_algorithmic": round(total / wl.algorithmic_bytes(), 5),
           "fetch": out["fetch"], "write": out["write"], "command": command}
    with open(os.path.join(TRAFFIC_DIR, f"traffic_{workload}.json"), "w") as f:
        json.dump(res, f, indent=1)
    return res


INDEXER_LAYOUT_NAMES = {0: "flat", 1: "tiled"}
# the library's data-moving kernels (the builder kernels of large batches are not counted)
GATHER_KERNELS = ("gather_pages_kernel", "gather_groups_kernel", "indexer_gather_kernel")


def call_for(wl, ws):
    """The library call for workload ``wl`` into workspace ``ws`` (for an
    indexer workload: its own value and scale destinations), marshalled once."""
    import paged_kv_cache_device_amd as pkvg
    import workloads

    if wl.kind == workloads.INDEXER:
        return pkvg.prepare_indexer(wl.cache, wl.dst_values(), wl.dst_scales(), wl.token_to_seq,
                                    wl.cu_seqlen, wl.block_table, wl.block_size,
                                    INDEXER_LAYOUT_NAMES[wl.layout], block_tile=wl.block_tile,
                                    head_tile=wl.head_tile, block_table_width=wl.block_table_width)
    dst = ws[: wl.num_tokens, : wl.entry]
    common = (wl.src_cache(), dst, wl.block_table, wl.cu_seq_lens, wl.num_reqs)
    if wl.kind == workloads.RAW:
        return pkvg.prepare("gather_cache", *common, wl.seq_starts)
    if wl.kind == workloads.UPCONVERT:
        return pkvg.prepare("gather_upconvert_fp8", *common, wl.scale_tensor,
                            seq_starts=wl.seq_starts)
    if wl.kind == workloads.DEQUANT_FP8:
        return pkvg.prepare("gather_maybe_dequant", *common, "fp8", scale=wl.scale_tensor,
                            seq_starts=wl.seq_starts)
    return pkvg.prepare("gather_maybe_dequant", *common, "auto", seq_starts=wl.seq_starts)


def _bulk_fields(wl):
    """The large tensors of a workload: the ones each rotation set copies."""
    import workloads

    if wl.kind == workloads.INDEXER:
        return ("cache", "values", "scales")
    return ("cache_base", "workspace")


def make_sets(wl_dev, min_bytes: int):
    """Copies of a workload's cache and destinations on the device totalling >= min_bytes."""
    import dataclasses

    fields = _bulk_fields(wl_dev)
    per = sum(getattr(wl_dev, f).numel() * getattr(wl_dev, f).element_size() for f in fields)
    n = max(2, -(-min_bytes // per))
    sets = []
    for i in range(n):
        w = dataclasses.replace(wl_dev)
        if i:
            for f in fields:
                setattr(w, f, getattr(wl_dev, f).clone())
        sets.append(w)
    return sets


def time_steps(sets, steps: int, warmup: int):
    """Exactly `steps` back-to-back calls rotating over `sets`, bracketed by
    torch.cuda.synchronize() on both sides.  Returns the wall time (s) and the
    GPU time (ms) between two HIP events recorded on the launch stream right
    before the first and right after the last call."""
    import torch

    runs = [call_for(w, getattr(w, "workspace", None)) for w in sets]
    torch.cuda._sleep(1)  # the spin kernel's first launch loads its code: not in the timed region
    for i in range(warmup):
        runs[i % len(runs)]()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    # a short spin kernel keeps the GPU busy while the host enqueues the first
    # calls, so the event pair times the calls back to back and not the host's
    # first submission (the spin lies before e0 and inside the host clock)
    torch.cuda._sleep(SPACER_CYCLES)
    e0.record()
    for i in range(steps):
        runs[i % len(runs)]()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, e0.elapsed_time(e1)


def cold_latency(wl_dev, reps: int, scrub_bytes: int = 1 << 30, read_scrub: bool = False):
    """Median / p10 / p90 (us) of one call after scrubbing >= 1 GiB (4x the
    Infinity Cache), bracketed by events on the launch stream.  The scrub is a
    fill kernel (the default), or with `read_scrub` a sum over the same bytes:
    it evicts the call's data as well but leaves clean lines behind, so the
    call does not also write back the scrub's dirty lines."""
    import torch

    dev = wl_dev.cache.device if hasattr(wl_dev, "cache") else wl_dev.workspace.device
    scrub = torch.empty(scrub_bytes // 4, dtype=torch.int32, device=dev)
    scrub.fill_(1)
    run = call_for(wl_dev, getattr(wl_dev, "workspace", None))
    out = []
    for i in range(reps + 3):
        if read_scrub:
            scrub.sum()
        else:
            scrub.fill_(i)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        run()
        b.record()
        b.synchronize()
        if i >= 3:
            out.append(a.elapsed_time(b) * 1e3)
    out.sort()
    return {"median_us": statistics.median(out), "p10_us": out[len(out) // 10],
            "p90_us": out[(9 * len(out)) // 10], "reps": reps}


def copy_reference(nbytes_each_way: int, device, steps: int, min_bytes: int):
    """A plain device-to-device copy of the same payload (torch's copy_ of
    contiguous same-dtype tensors, i.e. hipMemcpyAsync device to device), cold
    by rotation: the achievable-copy reference."""
    import torch

    n = max(2, -(-min_bytes // (2 * nbytes_each_way)))
    bufs = [(torch.empty(nbytes_each_way, dtype=torch.uint8, device=device),
             torch.empty(nbytes_each_way, dtype=torch.uint8, device=device)) for _ in range(n)]
    for s, d in bufs:
        d.copy_(s)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        s, d = bufs[i % n]
        d.copy_(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return {"gbs": 2 * nbytes_each_way * steps / wall / 1e9, "ms_per_copy": wall / steps * 1e3,
            "bytes_each_way": nbytes_each_way}


def oracle_row_chunks(wl, parts: int):
    """Cut the workload's output rows into `parts` contiguous ranges.  Each range
    is a list of virtual requests (out_begin, out_end, source start, request),
    so the unchanged oracle can run the ranges on separate threads: by the
    per-token definition, row b of request r reads token start_r + (b - b_r)."""
    cu = wl.cu_seq_lens.tolist()
    T = wl.num_tokens
    ends = wl.request_ends()
    starts = [0] * wl.num_reqs if wl.seq_starts is None else wl.seq_starts.tolist()
    extents = [(min(cu[r], T), min(ends[r], T), starts[r], r) for r in range(wl.num_reqs)]
    extents = [x for x in extents if x[1] > x[0]]
    total = sum(e - b for b, e, _, _ in extents)
    per = max(1, -(-total // parts))
    chunks, cur, budget = [], [], per
    for b, e, s, r in extents:
        while b < e:
            take = min(e - b, budget)
            cur.append((b, b + take, s, r))
            b, s, budget = b + take, s + take, budget - take
            if budget == 0:
                chunks.append(cur)
                cur, budget = [], per
    if cur:
        chunks.append(cur)
    return chunks


def indexer_oracle_threaded(wl, threads: int, values, scales):
    """A callable that runs the oracle's indexer gather once over `threads`
    disjoint row ranges [r0, r1) of `wl`: each range passes token_to_seq and
    the destinations from row r0 on and cu_seqlen shifted down by r0, so row
    r0 + i of the whole gather is row i of the range with the same position in
    its sequence (the oracle's code and arithmetic are unchanged)."""
    import numpy as np

    import oracle

    o = oracle.load()
    T = wl.num_tokens
    per = max(1, -(-T // threads))
    cache = wl.cache.numpy().reshape(-1)
    vflat = values.numpy().reshape(-1)
    sflat = scales.view(__import__("torch").uint8).numpy().reshape(-1)
    vs, ss = values.stride(0), 4 * scales.stride(0)
    t2s = wl.token_to_seq.numpy()
    cu = wl.cu_seqlen.numpy().astype(np.int64)
    bt = wl.block_table.numpy()
    jobs = [(r0, min(r0 + per, T)) for r0 in range(0, T, per)]

    def run(job):
        r0, r1 = job
        return o.indexer_gather(cache, wl.num_blocks, wl.block_size, wl.block_stride, wl.layout,
                                wl.head_dim, wl.block_tile, wl.head_tile, vflat[r0 * vs:], vs,
                                sflat[r0 * ss:], ss, r1 - r0, t2s[r0:r1],
                                (cu - r0).astype(np.int32), wl.num_batches, bt,
                                wl.block_table_width, bt.shape[1])

    return lambda pool: sum(pool.map(run, jobs))


def oracle_threaded(wl, threads: int, ws):
    """A callable that runs the oracle once over `threads` disjoint row ranges of
    `wl` into the workspace `ws` (on a given thread pool) and returns the rows
    written."""
    import torch

    import oracle
    import workloads

    o = oracle.load()
    mode = oracle.MODE_E4M3FN_TO_BF16 if wl.kind in workloads.FP8_KINDS else oracle.MODE_COPY
    dst = ws[: wl.num_tokens, : wl.entry]
    jobs = []
    for chunk in oracle_row_chunks(wl, threads):
        cu = torch.tensor([c[0] for c in chunk] + [chunk[-1][1]], dtype=torch.int32)
        st = torch.tensor([c[2] for c in chunk], dtype=torch.int32)
        bt = wl.block_table[[c[3] for c in chunk]].contiguous()
        jobs.append((bt, cu, st, len(chunk)))

    def run(job):
        bt, cu, st, n = job
        return o.gather_tensors(mode, wl.src_cache(), dst, bt, cu, st, n, wl.scale)

    return lambda pool: sum(pool.map(run, jobs))


def cpu_baseline(wl, seconds: float = 10.0, threads: int = 1):
    """The CPU oracle (test infrastructure, untuned) on the same workload on the
    host, repeated for about `seconds`.  With threads > 1 the output rows are
    cut into that many contiguous ranges run concurrently (the oracle's code and
    arithmetic are unchanged; ctypes releases the GIL during each call)."""
    from concurrent.futures import ThreadPoolExecutor

    import workloads

    if wl.kind == workloads.INDEXER:
        run_once = indexer_oracle_threaded(wl, threads, wl.fresh_values(), wl.fresh_scales())
    else:
        run_once = oracle_threaded(wl, threads, wl.fresh_workspace())
    reps = 0
    with ThreadPoolExecutor(max_workers=threads) as pool:
        t0 = time.perf_counter()
        while True:
            rows = run_once(pool)
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    assert rows == wl.gathered_rows()
    per = el / reps
    return {"value": wl.algorithmic_bytes() / per / 1e9, "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"whole workload ({wl.name}), {reps} repetitions in {el:.1f} s, "
                      f"{per * 1e3:.1f} ms each, {threads} thread(s) over disjoint row ranges, "
                      f"on {cpu_model_name()}"}


def cpu_model_name() -> str:
    """The host CPU's model name from /proc/cpuinfo ("unknown" if absent)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_threads() -> int:
    """Threads for the CPU baseline: the cores this process may use, at most 16
    (the host share of one GPU)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def measure(wl, dev, args) -> dict:
    """Time `args.steps` calls of workload `wl` (cold by rotation), then a warm
    run and single calls after a cache scrub; returns the numbers of one bench
    line (rates from the event-timed region, see the module docstring)."""
    import torch

    import workloads

    g = wl.to(dev)
    alg_bytes = wl.algorithmic_bytes()
    sets = make_sets(g, 3 << 30)  # far above the 256 MB Infinity Cache
    log(f"[bench] {wl.name}: {len(sets)} input/output copies; algorithmic bytes/step {alg_bytes}")
    wall, ev_ms = time_steps(sets, args.steps, args.warmup)
    kern_ms = ev_ms / args.steps
    achieved = alg_bytes / (kern_ms * 1e-3) / 1e9
    log(f"[bench] {wl.name}: {args.steps} steps: {kern_ms * 1e3:.2f} us/launch (events), "
        f"{wall / args.steps * 1e6:.2f} us/step wall, {achieved:.0f} GB/s")
    _, ev_w = time_steps(sets[:1], args.steps, args.warmup)
    warm_us = ev_w / args.steps * 1e3
    del sets
    cold = cold_latency(g, args.cold_reps)
    cold_read = cold_latency(g, args.cold_reps, read_scrub=True)
    log(f"[bench] {wl.name}: cold scrubbed median {cold['median_us']:.2f} us (after a read scrub "
        f"{cold_read['median_us']:.2f} us); warm {warm_us:.2f} us")
    torch.cuda.empty_cache()
    return {
        "value": round(achieved, 2),
        "unit": "GB/s",
        "ms_per_step": round(kern_ms, 6),
        "wall_ms_per_step": round(wall / args.steps * 1e3, 6),
        # raw, 'auto' and indexer gathers copy bytes; the fp8 paths decode and scale in fp32
        "dtype": "u8" if wl.kind in (workloads.RAW, workloads.DEQUANT_AUTO, workloads.INDEXER)
        else "f32",
        "config": workload_config(wl, alg_bytes),
        "pct_of_peak": round(100.0 * achieved / PEAK_HBM_GBS, 2),
        "median_latency_us_cold_scrubbed": round(cold["median_us"], 3),
        # the same algorithmic bytes over the cold single call's median (one launch timed on
        # its own: it carries the launch's own fixed cost)
        "cold_single_call_gbs": round(alg_bytes / (cold["median_us"] * 1e-6) / 1e9, 2),
        "cold_single_call_pct_of_peak": round(100.0 * alg_bytes / (cold["median_us"] * 1e-6) / 1e9 / PEAK_HBM_GBS, 2),
        "per_launch_us": round(kern_ms * 1e3, 3),
        "latency_us": {"cold_scrubbed_single_call": {k: round(v, 3) for k, v in cold.items()},
                       "cold_read_scrubbed_single_call": {k: round(v, 3) for k, v in cold_read.items()},
                       "back_to_back_per_launch_cold": round(kern_ms * 1e3, 3),
                       "back_to_back_per_launch_warm": round(warm_us, 3)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic(wl.name)},
    }


def workload_config(wl, alg_bytes: int) -> dict:
    """The bench line's config object for workload `wl`."""
    import workloads

    if wl.kind == workloads.INDEXER:
        return {"workload": wl.name, "num_batches": wl.num_batches, "num_tokens": wl.num_tokens,
                "block_size": wl.block_size, "head_dim": wl.head_dim,
                "layout": INDEXER_LAYOUT_NAMES[wl.layout], "num_blocks": wl.num_blocks,
                "block_stride": wl.block_stride, "kind": wl.kind,
                "algorithmic_bytes_per_step": alg_bytes, "parallelism": "single GPU"}
    return {"workload": wl.name, "num_reqs": wl.num_reqs, "num_tokens": wl.num_tokens,
            "block_size": wl.block_size, "entry": wl.entry, "num_blocks": wl.num_blocks,
            "kind": wl.kind, "algorithmic_bytes_per_step": alg_bytes, "parallelism": "single GPU"}


# --kind of a custom workload -> the workload kind (entry point and conversion)
CUSTOM_KINDS = {"raw": "raw", "fp8_upconvert": "upconvert", "fp8_dequant": "dequant_fp8",
                "auto": "dequant_auto"}


def custom_workload_name(args) -> str:
    lens = [int(x) for x in args.lens.split(",")]
    return (f"custom_{args.kind}_R{len(lens)}_T{sum(lens)}_bs{args.block_size}_e{args.entry}"
            f"{'_starts' if args.starts else ''}")


def custom_workload(args):
    """A workload from the command line: the given context lengths, block size and
    entry, shuffled physical blocks (5/4 of the pages needed), seeded values."""
    import workloads

    lens = [int(x) for x in args.lens.split(",")]
    pages = sum(-(-n // args.block_size) for n in lens)
    return workloads.make_workload(custom_workload_name(args), CUSTOM_KINDS[args.kind], lens,
                                   args.block_size, args.entry, max(pages * 5 // 4, 1) + 8,
                                   seed=args.seed, draw_starts_quarter=args.starts,
                                   scale=args.scale)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--also", default=",".join(ALSO_WORKLOADS),
                    help="comma-separated named workloads timed in the same run, each reported "
                         "as a nested object under its name ('' for none)")
    ap.add_argument("--only-gather", action="store_true",
                    help="run warmup + steps of the gather and nothing else (for profilers)")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="with --only-gather: then run 10 device copies of this many MiB "
                         "(a plain copy kernel of known size, to scale traffic counters)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--summarize-counters", metavar="PROF_DIR",
                    help="summarize rocprofv3 FETCH_SIZE/WRITE_SIZE runs of --workload into "
                         "profiles/traffic_<workload>.json and exit (no GPU needed)")
    ap.add_argument("--counter-command", default="",
                    help="with --summarize-counters: the profiling command, stored verbatim")
    ap.add_argument("--cold-reps", type=int, default=100)
    custom = ap.add_argument_group(
        "custom workload", "instead of --workload: one built from these flags (seeded, shuffled blocks)")
    custom.add_argument("--lens", help="comma-separated context lengths, one per request")
    custom.add_argument("--kind", default="raw", choices=sorted(CUSTOM_KINDS),
                        help="raw copy, fp8 upconvert, fp8 dequant, or 'auto' (bf16 copy)")
    custom.add_argument("--block-size", type=int, default=64)
    custom.add_argument("--entry", type=int, default=576, help="elements gathered per token")
    custom.add_argument("--starts", action="store_true",
                        help="seq_starts drawn uniformly from [0, len / 4]")
    custom.add_argument("--scale", type=float, default=0.0625, help="fp8 per-tensor scale")
    custom.add_argument("--seed", type=int, default=1)
    args = ap.parse_args()
    if args.lens:
        args.workload = custom_workload_name(args)

    if args.summarize_counters:
        res = summarize_counters(args.summarize_counters, args.workload, args.calibration_copy_mib,
                                 args.counter_command)
        print(json.dumps(res, indent=1))
        return

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the gather "
              "shards by request or page range with no exchange; this benchmark measures "
              "one GPU's share and does not launch several", file=sys.stderr)
        sys.exit(2)

    import torch

    import workloads
    import paged_kv_cache_device_amd as pkvg

    pkvg.library()
    dev = torch.device("cuda:0")
    log(f"[bench] workload {args.workload}: generating")
    wl = custom_workload(args) if args.lens else workloads.named(args.workload)

    if args.only_gather:
        sets = make_sets(wl.to(dev), 3 << 30)  # far above the 256 MB Infinity Cache
        wall, _ = time_steps(sets, args.steps, args.warmup)
        log(f"[bench] only-gather: {args.steps} steps in {wall * 1e3:.2f} ms")
        del sets
        if args.calibration_copy_mib:
            n = args.calibration_copy_mib << 20
            bufs = [(torch.empty(n, dtype=torch.uint8, device=dev),
                      torch.empty(n, dtype=torch.uint8, device=dev)) for _ in range(4)]
            for i in range(10):
                s_, d_ = bufs[i % 4]
                d_.copy_(s_)
            torch.cuda.synchronize()
            log(f"[bench] calibration: 10 copies of {n} bytes")
        return

    head = measure(wl, dev, args)
    payload_each_way = (wl.gathered_rows() * (wl.head_dim + 4) if wl.kind == workloads.INDEXER
                        else wl.gathered_rows() * wl.entry * wl.dst_elem_bytes)
    copy_ref = copy_reference(payload_each_way, dev, args.steps, 3 << 30)
    log(f"[bench] device copy reference {copy_ref['gbs']:.0f} GB/s")
    also = []
    for name in [a for a in args.also.split(",") if a] if not args.lens else []:
        if name == wl.name:
            continue
        log(f"[bench] further workload {name}: generating")
        also.append(measure(workloads.named(name), dev, args))
        torch.cuda.empty_cache()

    result = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic (seeded N(0,1) bf16 / uniform non-NaN e4m3fn codes; shuffled blocks)",
        "config": head["config"],
        "pct_of_peak": head["pct_of_peak"],
        "wall_ms_per_step": head["wall_ms_per_step"],
        "median_latency_us_cold_scrubbed": head["median_latency_us_cold_scrubbed"],
        "cold_single_call_gbs": head["cold_single_call_gbs"],
        "cold_single_call_pct_of_peak": head["cold_single_call_pct_of_peak"],
        "per_launch_us": head["per_launch_us"],
        "latency_us": head["latency_us"],
        "roofline": head["roofline"],
        "copy_reference": copy_ref,
        # the pages' own figures (their page kernel against the prior kernel, kernel latency,
        # on another vendor's GPU): relative context only, nothing here reproduces them
        "context": {"pages_speedup_over_prior_kernel": {"raw_copy_60k": 220.7, "raw_copy_300k": 331.3,
                                                         "fp8_upconvert": "0.99-1.10",
                                                         "maybe_dequant": "1.39-1.77"},
                    "pages_dram_fraction_of_peak": "0.75-0.84"},
    }
    for a in also:
        result[a["config"]["workload"]] = a
    if not args.no_cpu:
        n = host_threads()
        log(f"[bench] timing the CPU oracle: {n} threads, then one (about 8 s each)")
        result["cpu_baseline"] = cpu_baseline(wl, 8.0, n)
        result["cpu_baseline_one_thread"] = cpu_baseline(wl, 8.0, 1)
        log(f"[bench] CPU oracle {result['cpu_baseline']['value']:.2f} GB/s on {n} threads, "
            f"{result['cpu_baseline_one_thread']['value']:.2f} GB/s on one")
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
