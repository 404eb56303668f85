#!/usr/bin/env python3
"""Benchmark of the retrieve-and-inject hot path on one MI355X.

A step is one inject_topk_device call over the whole batch: the retrieved
fact ids, prefixes and block tables (resident in HBM) are resolved to arena
rows, positions and paged slots on the device, every fact's pre-RoPE K/V rows
are gathered from the HBM-resident store, K is rotated to its serving-time
positions, and K and V are scattered into the paged cache, for all layers, KV
heads and requests.  The roofline figures time the dominant kernel alone
(inject_topk on the same, already mapped batch).  The PCIe-inclusive variant
(host build_slot_mapping + H2D of the mapping + inject) is reported separately
under "e2e" and is never `value`.

Timing: the headline step and kernel are K launches with an event after
each (so the line has per-launch percentiles; an event costs a few
microseconds against a 5 ms launch), `ms_per_step` the larger of that mean
and the host's wall clock.  Launches of tens of microseconds (the small
workloads, retrieval, the reference copies and reads) are timed as runs of
back-to-back launches enqueued behind a clock spin with one event before
and one after the run, since an event between launches would add its own
3-5 us to each; cold figures are runs of (MALL-evicting fill, launch) minus
runs of the fills alone.

Prints one JSON line.  Only one GPU: --gpus above 1 exits with a message.
"""

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "injected KV tokens/s (all layers) + achieved HBM GB/s and % of peak, 1 MI355X"
PEAK_HBM_GBPS = 8000.0
PEAK_PCIE_GBPS = 64.0  # PCIe 5.0 x16, one direction
DEFAULT_WORKLOAD = "llama3_8b_batch64_k50"


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="wall-clock budget of the CPU-oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-e2e", action="store_true")
    ap.add_argument("--k-sweep", action="store_true",
                    help="instead of the batch: one request on the 2,000-fact Llama-3-8B store, "
                         "the device step timed for its first k = 5, 10, 20, 50 facts")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step replayed from a captured HIP graph (launch-bound "
                         "small batches)")
    ap.add_argument("--no-permute", action="store_true",
                    help="skip timing the same batch with every request's facts reordered")
    ap.add_argument("--pool-requests", type=int, default=8,
                    help="requests in the sample of the multi-core CPU-oracle baseline (0: skip)")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the step and kernel timings of the other workloads")
    ap.add_argument("--other-workloads-only", default=None, metavar="NAMES",
                    help="(used by the bench itself) time only these comma-separated "
                         "workloads and print their figures as one JSON object")
    ap.add_argument("--no-attend", action="store_true",
                    help="skip timing the query-prefill attention over the injected cache")
    ap.add_argument("--no-retrieve", action="store_true",
                    help="skip timing retrieve_topk and retrieve + inject")
    ap.add_argument("--store", choices=("device", "host"), default="device",
                    help="where the fact store's arenas live: HBM, or pinned host DRAM read "
                         "by the kernel over PCIe (zero-copy)")
    ap.add_argument("--cache-layout", choices=("nhd", "hnd"), default="nhd",
                    help="paged cache block layout: [block_size][H][D] (vLLM's) or "
                         "[H][block_size][D]")
    ap.add_argument("--flush", action="store_true",
                    help="evict the 256 MB Infinity Cache with a 1 GiB fill before every timed "
                         "launch and time launches one by one (for workloads far below 1 GiB)")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the hand-written streaming-copy (inject) and streaming-read "
                         "(retrieval) references of the same bytes")
    ap.add_argument("--placement-probe", action="store_true",
                    help="instead of the bench: the workload's inject kernel and a plain copy "
                         "between the same addresses on successive allocations of its buffers")
    ap.add_argument("--no-host-store", action="store_true",
                    help="skip the host-DRAM store figures (zero-copy and staged)")
    ap.add_argument("--no-slot-check", action="store_true",
                    help="skip timing the step with the device duplicate-slot check on")
    ap.add_argument("--cpu-worker", action="store_true",
                    help="(used by the bench itself) one worker of the multi-core CPU-oracle "
                         "baseline: read a task as JSON on stdin, print the result")
    ap.add_argument("--summarize-profile", nargs=3, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="turn rocprofv3 output of this script into profiles/<kernel>_<workload>.md")
    return ap.parse_args()


# bench.py under rocprofv3: no child processes (the profiler's library has
# initialised the GPU before the program starts) and only the path's kernels
PROFILE_FLAGS = ("--no-cpu-baseline --no-e2e --no-other-workloads --no-ceiling "
                 "--no-slot-check --no-host-store")

# kernels with committed rocprofv3 summaries: name prefix -> source file
PROFILED = {"inject_kernel": "prkv_inject.hip", "attend_kernel": "prkv_attend.hip",
            "score_kernel": "prkv_retrieve.hip"}
ATTN_Q_LEN = 16        # query tokens per request in the attention section
ATTN_GROUP = 4         # query heads per KV head


def kernel_source_sha(kernel="inject_kernel"):
    import hashlib
    path = os.path.join(ROOT, "pre_rope_kv_amd", "csrc", PROFILED[kernel])
    with open(path, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def profile_path(workload, kernel="inject_kernel"):
    return os.path.join(ROOT, "profiles", f"{kernel}_{workload}.md")


def read_profile_traffic(workload, kernel="inject_kernel"):
    """HBM bytes per launch from the committed counter summary, or None when
    there is none or the kernel source changed since it was taken."""
    path = profile_path(workload, kernel)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if line.startswith("- ") and ": " in line:
                k, v = line[2:].split(": ", 1)
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel_source_sha256") != kernel_source_sha(kernel):
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def attention_bytes(w):
    """(cache bytes read, minimal total bytes) of one attend_paged launch over
    every request's whole context: K and V rows once, the queries once, the
    float32 outputs once."""
    sp = w.spec
    ctx = sum(int(w.prefix[r]) + sum(w.length_of(f) for f in ids)
              for r, ids in enumerate(w.retrieved))
    hq = ATTN_GROUP * sp.num_kv_heads
    kv = ctx * sp.num_layers * sp.num_kv_heads * sp.head_dim * 2 * 2
    q = sp.n_requests * ATTN_Q_LEN * hq * sp.head_dim * 2
    out = sp.num_layers * sp.n_requests * ATTN_Q_LEN * hq * sp.head_dim * 4
    return kv, kv + q + out


def algorithmic_bytes(kernel, w):
    if kernel == "inject_kernel":
        return w.n_tokens * w.spec.bytes_per_token, (
            "read K and V rows, write K and V rows: tokens x layers x 4 x H x D x 2 B")
    if kernel == "score_kernel":
        sp = w.spec
        emb = sp.n_requests * sp.facts_per_store * sp.emb_dim * 2
        return emb + sp.n_requests * sp.emb_dim * 2 + sp.n_requests * sp.facts_per_store * 8, (
            "every fact embedding of every request's store once (bf16), the queries once, "
            "one float64 score per fact written")
    return attention_bytes(w)[1], (
        f"K and V rows of every context position once, {ATTN_Q_LEN} bf16 query rows x "
        f"{ATTN_GROUP} heads per KV head, float32 outputs (all layers)")


def summarize_profile(workload, trace_dir, fetch_dir, write_dir, commands):
    """Write the rocprofv3 summaries: one file per profiled kernel plus a
    table of every kernel in the traced run.

    Counter calibration: the 4 GiB device-to-device memcpy of copy_ceiling_gbps
    (__amd_rocclr_copyBuffer, known to read 4 GiB and write 4 GiB) is looked up
    in the same counter runs; FETCH_SIZE and WRITE_SIZE of a kernel are scaled
    by (4 GiB / what the counter reads for that copy).
    """
    import csv
    import glob
    import statistics

    def rows(d, suffix):
        files = glob.glob(os.path.join(d, f"*{suffix}"))
        if not files:
            raise FileNotFoundError(f"no *{suffix} under {d}")
        with open(files[0]) as fh:
            return list(csv.DictReader(fh))

    copy_kib = 4 * 1024 * 1024

    def counter(d, name, kernel):
        rs = rows(d, "counter_collection.csv")
        vals = [float(r["Counter_Value"]) for r in rs if r["Kernel_Name"].startswith(kernel)
                and r["Counter_Name"] == name]
        cal = [float(r["Counter_Value"]) for r in rs
               if r["Kernel_Name"].strip() == "__amd_rocclr_copyBuffer"
               and r["Counter_Name"] == name and float(r["Counter_Value"]) > copy_kib / 4]
        return statistics.mean(vals), statistics.mean(cal), len(vals), len(cal)

    from pre_rope_kv_amd import workloads
    w = workloads.make(workload)
    all_stats = rows(trace_dir, "kernel_stats.csv")
    all_trace = rows(trace_dir, "kernel_trace.csv")
    header = ["rocprofv3 summaries of `bench.py` on one MI355X; raw CSVs stay in the run's",
              "output directory.  Commands (from the repository root):", ""] + \
        [f"    {c}" for c in commands]
    for kernel in PROFILED:
        stats = [r for r in all_stats if r["Name"].startswith(kernel)]
        durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6 for r in all_trace
                if r["Kernel_Name"].startswith(kernel)]
        if not stats:
            continue
        f_k, f_cal, nf, ncf = counter(fetch_dir, "FETCH_SIZE", kernel)
        w_k, w_cal, nw, ncw = counter(write_dir, "WRITE_SIZE", kernel)
        f_scale, w_scale = copy_kib / f_cal, copy_kib / w_cal
        fetch_b = f_k * f_scale * 1024
        write_b = w_k * w_scale * 1024
        alg, alg_what = algorithmic_bytes(kernel, w)
        st = stats[0]
        lines = [f"# {kernel} on {workload} (MI355X, gfx950)", ""] + header + [
            "",
            "## Kernel trace (--kernel-trace --stats)",
            "",
            f"- kernel: {st['Name'][:80]}",
            f"- calls: {st['Calls']}",
            f"- average_ms: {float(st['AverageNs']) / 1e6:.4f}",
            f"- min_ms: {float(st['MinNs']) / 1e6:.4f}",
            f"- max_ms: {float(st['MaxNs']) / 1e6:.4f}",
            f"- median_ms_from_trace: {statistics.median(durs):.4f}",
            f"- share_of_gpu_time_in_run_pct: {float(st['Percentage']):.2f}",
            "",
            "## HBM traffic (--pmc FETCH_SIZE, then --pmc WRITE_SIZE, separate runs)",
            "",
            "Calibration: the 4 GiB device-to-device memcpy (`__amd_rocclr_copyBuffer`)",
            "in the same runs reads 4 GiB and writes 4 GiB by construction.",
            f"Algorithmic bytes: {alg_what}.",
            "",
            f"- fetch_size_kib_per_launch_raw: {f_k:.0f} (mean of {nf} launches)",
            f"- fetch_size_kib_for_4GiB_copy: {f_cal:.0f} (mean of {ncf}); scale {f_scale:.4f}",
            f"- write_size_kib_per_launch_raw: {w_k:.0f} (mean of {nw} launches)",
            f"- write_size_kib_for_4GiB_copy: {w_cal:.0f} (mean of {ncw}); scale {w_scale:.4f}",
            f"- fetch_bytes_per_launch: {fetch_b:.0f}",
            f"- write_bytes_per_launch: {write_b:.0f}",
            f"- traffic_bytes_per_launch: {int(round(fetch_b + write_b))}",
            f"- algorithmic_bytes_per_launch: {alg}",
            f"- traffic_over_algorithmic: {(fetch_b + write_b) / alg:.4f}",
            f"- kernel_source_sha256: `{kernel_source_sha(kernel)}`",
            "",
        ]
        groups = sorted({r["Grid_Size_X"] for r in all_trace if r["Kernel_Name"].startswith(kernel)},
                        key=int)
        if len(groups) > 1:
            # several launch shapes of one kernel (e.g. the fused single-launch
            # step and the kernel alone on a host-built mapping)
            lines += ["## Launch shapes (grouped by grid size)", "",
                      "| grid (workgroups) | calls | median ms | min ms | fetch B/launch | "
                      "write B/launch | traffic / algorithmic |", "|---|---|---|---|---|---|---|"]
            fr = rows(fetch_dir, "counter_collection.csv")
            wr = rows(write_dir, "counter_collection.csv")
            for g in groups:
                d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6 for r in all_trace
                     if r["Kernel_Name"].startswith(kernel) and r["Grid_Size_X"] == g]
                fv = [float(r["Counter_Value"]) for r in fr if r["Kernel_Name"].startswith(kernel)
                      and r["Grid_Size"] == g and r["Counter_Name"] == "FETCH_SIZE"]
                wv = [float(r["Counter_Value"]) for r in wr if r["Kernel_Name"].startswith(kernel)
                      and r["Grid_Size"] == g and r["Counter_Name"] == "WRITE_SIZE"]
                fb = statistics.mean(fv) * f_scale * 1024 if fv else float("nan")
                wb = statistics.mean(wv) * w_scale * 1024 if wv else float("nan")
                lines.append(f"| {int(g) // 256} | {len(d)} | {statistics.median(d):.4f} | "
                             f"{min(d):.4f} | {fb:.0f} | {wb:.0f} | {(fb + wb) / alg:.4f} |")
            lines.append("")
        with open(profile_path(workload, kernel), "w") as fh:
            fh.write("\n".join(lines))
        print(profile_path(workload, kernel))
    table = [f"# Every kernel in the traced bench run on {workload} (MI355X, gfx950)", ""] + \
        header[:2] + ["", f"    {commands[0]}", "",
                      "| kernel | calls | average ms | min ms | max ms | share of GPU time % |",
                      "|---|---|---|---|---|---|"]
    for r in sorted(all_stats, key=lambda r: -float(r["Percentage"])):
        table.append(f"| {r['Name'][:70]} | {r['Calls']} | {float(r['AverageNs']) / 1e6:.4f} | "
                     f"{float(r['MinNs']) / 1e6:.4f} | {float(r['MaxNs']) / 1e6:.4f} | "
                     f"{float(r['Percentage']):.2f} |")
    path = os.path.join(ROOT, "profiles", f"all_kernels_{workload}.md")
    with open(path, "w") as fh:
        fh.write("\n".join(table) + "\n")
    print(path)


def copy_ceiling_gbps(torch, nbytes=4 << 30, reps=10):
    """Read + write bytes / time of two library copies of `nbytes`, for context:
    a device-to-device memcpy, and an elementwise int16 negate kernel (whose
    FETCH_SIZE / WRITE_SIZE counters calibrate the HBM-traffic counters)."""
    src = torch.empty(nbytes // 2, dtype=torch.int16, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    out = {}
    for name, fn in (("memcpy", lambda: dst.copy_(src)),
                     ("elementwise_neg", lambda: torch.neg(src, out=dst))):
        for _ in range(2):
            fn()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        torch.cuda.synchronize()
        out[name] = 2 * nbytes / (s.elapsed_time(e) / reps * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return out


_CEILING = None


def ceiling_lib():
    """libprkv_ceiling.so (built by pre_rope_kv_amd.build): the plain copy the
    inject kernel is measured against, the plain read the retrieval is, and
    the plain gather of the cache rows the attention kernel is."""
    global _CEILING
    if _CEILING is None:
        path = os.path.join(ROOT, "pre_rope_kv_amd", "libprkv_ceiling.so")
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: build with `python -m pre_rope_kv_amd.build`")
        lib = ctypes.CDLL(path)
        vp = ctypes.c_void_p
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        lib.ceiling_gather_scatter.argtypes = [vp, vp, i64, vp, vp, i64, vp, vp, i64, i32, i32,
                                               i32, i32, vp]
        lib.ceiling_gather_scatter.restype = ctypes.c_int
        lib.ceiling_empty.argtypes = [ctypes.c_int32, vp]
        lib.ceiling_empty.restype = ctypes.c_int
        lib.ceiling_read.argtypes = [vp, i64, vp, i32, i32, vp]
        lib.ceiling_read.restype = ctypes.c_int
        lib.ceiling_gather_kv.argtypes = [vp, vp, i64, i32, i32, i32, vp, i32, vp, vp, i32, i32,
                                          i64, i32, vp, i32, i32, vp]
        lib.ceiling_gather_kv.restype = ctypes.c_int
        _CEILING = lib
    return _CEILING


class Flusher:
    """Evicts the 256 MB Infinity Cache (MALL) with a 1 GiB fill on a stream,
    so that the next launch finds none of its data cached."""

    def __init__(self, torch):
        self.buf = torch.empty(1 << 29, dtype=torch.int16, device="cuda")
        self.i = 0

    def __call__(self, torch, stream):
        self.i = (self.i + 1) % 32000      # a new value each time, within int16
        with torch.cuda.stream(stream):
            self.buf.fill_(self.i)


def queue_ahead(torch, stream, ms=2.0):
    """Enqueue ~ms of GPU work that touches no memory (a clock spin) on
    `stream`, so that launches the host enqueues meanwhile are already
    waiting when the GPU reaches them: events around them then time the GPU,
    not the host's launch rate (which bounds back-to-back launches of a few
    microseconds)."""
    spin = getattr(torch.cuda, "_sleep", None)
    if spin is None:        # no spin kernel in this torch build: launches are timed as enqueued
        return
    with torch.cuda.stream(stream):
        spin(int(ms * 1e-3 * 2.0e9))   # cycles at ~2 GHz (bounded spin)


def time_launches(torch, fn, stream, steps, warmup, flusher=None, queued=False, reps=3):
    """Mean and median ms per launch of fn() on `stream`.  Warm: `steps`
    back-to-back launches split into `reps` runs, each enqueued behind a
    clock spin (queue_ahead) and timed by two events around the run, so the
    figures are GPU time even for launches shorter than the host's launch
    cost, and no event sits between launches (an event after every launch
    adds 3-5 us to each); mean = all runs' time / all launches, median = the
    median of the runs' means.  Cold (a flusher): every launch follows a
    MALL-evicting fill; `reps` runs of `steps` (fill, launch) pairs and as
    many runs of the fills alone, each between two events behind a clock
    spin; a launch's cold time = (pairs - fills) / steps (the fills' jitter
    averages out over the run), mean over the runs and their median.
    `queued` is kept for callers: runs are always queued."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    if flusher is None:
        per_run = max(1, steps // reps)
        means, total = [], 0.0
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            queue_ahead(torch, stream)
            e0.record(stream)
            for _ in range(per_run):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            total += ms
            means.append(ms / per_run)
        means.sort()
        return total / (per_run * reps), means[len(means) // 2]
    def run(with_launch):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        queue_ahead(torch, stream)
        e0.record(stream)
        for _ in range(steps):
            flusher(torch, stream)
            if with_launch:
                fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    diffs = []
    for _ in range(reps):
        diffs.append((run(True) - run(False)) / steps)
    diffs.sort()
    return sum(diffs) / len(diffs), diffs[len(diffs) // 2]


def time_span(torch, fn, stream, steps, warmup):
    """Mean ms per launch of fn() on `stream` over `steps` back-to-back
    launches between two events, enqueued behind a clock spin: for launches of
    tens of microseconds, where an event after every launch would add its own
    time to each."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    queue_ahead(torch, stream)
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def gather_scatter_ceiling(torch, dw, steps, warmup, flusher=None):
    """Read + write GB/s of a plain copy that moves exactly the bytes of the
    workload's inject launch (libprkv_ceiling.so): every token's K and V row
    of every layer from its arena row to a cache row, with no rotation.
    "mapped": the batch's own arena rows and cache slots (the inject launch's
    addresses); "contiguous": rows t -> t of the same arena and cache.  Each
    is the best of token- and layer-major wave orders x 64 / 256 / 1024-lane
    workgroups; with a flusher the best shape is also timed cold.  It
    overwrites cache rows, so the cache is reset and the batch re-injected
    afterwards.  None when the layout has no such copy (HND cache, host
    store, rows other than 256 B - 4 KiB in powers of two)."""
    sp, w = dw.w.spec, dw.w
    if dw.hnd or dw.store_location != "device" or \
            sp.row_bytes not in (256, 512, 1024, 2048, 4096):
        return None
    lib = ceiling_lib()
    stream = dw.stream
    n, L = dw.n_tokens, sp.num_layers
    num_slots = w.num_blocks * sp.block_size
    src, _, slot = dw.d_map
    # every row index inside its buffer (the copy trusts them)
    assert 0 <= int(src[:n].min()) and int(src[:n].max()) < w.capacity_rows
    assert 0 <= int(slot[:n].min()) and int(slot[:n].max()) < num_slots
    assert n <= w.capacity_rows and n <= num_slots
    nbytes = n * sp.bytes_per_token
    queued = nbytes < COLD_BELOW_BYTES
    out = {"bytes_per_launch": nbytes}
    for name, rows in (("mapped", (src.data_ptr(), slot.data_ptr())), ("contiguous", (None, None))):
        best = None
        for order in (0, 1):
            for threads in (64, 256, 1024):
                args = (dw.k_arena.data_ptr(), dw.v_arena.data_ptr(), w.capacity_rows * sp.row_bytes,
                        dw.k_cache.data_ptr(), dw.v_cache.data_ptr(), num_slots * sp.row_bytes,
                        rows[0], rows[1], n, L, sp.row_bytes, order, threads, stream.cuda_stream)

                def fn(a=args):
                    rc = lib.ceiling_gather_scatter(*a)
                    if rc != 0:
                        raise RuntimeError(f"ceiling_gather_scatter failed ({rc})")

                ms, _ = time_launches(torch, fn, stream, steps, warmup, queued=queued)
                if best is None or ms < best[0]:
                    best = (ms, order, threads, fn)
        ms, order, threads, fn = best
        row = {"gbps": nbytes / (ms * 1e-3) / 1e9, "ms": ms,
               "order": "token-major" if order == 0 else "layer-major", "threads": threads}
        if flusher is not None:
            c_ms, c_med = time_launches(torch, fn, stream, steps, 2, flusher)
            row.update({"cold_ms": c_ms, "cold_median_ms": c_med,
                        "cold_gbps": nbytes / (c_ms * 1e-3) / 1e9})
        out[name] = row
    out["gbps"] = max(out["mapped"]["gbps"], out["contiguous"]["gbps"])
    if flusher is not None:
        out["cold_gbps"] = max(out["mapped"]["cold_gbps"], out["contiguous"]["cold_gbps"])
    dw.reset_cache()
    dw.inject()
    torch.cuda.synchronize()
    return out


def host_store_figures(torch, lib, w, dw_hbm, steps, warmup, hbm_kernel_ms):
    """The workload with its store in pinned host DRAM (the pages' capacity
    lever), injected into the HBM workload's cache two ways, each step timed
    by wall clock between synchronizations: zero-copy (the inject kernel
    reads the retrieved rows over PCIe), and staged (store_stage_facts copies
    the batch's facts into HBM in chunks on a second stream, each chunk
    injected as soon as it has landed; the staging store reuses the HBM
    workload's arenas, into which it writes the same rows it already holds).
    added_ms = step - the HBM-resident inject kernel."""
    from pre_rope_kv_amd import harness, prkv

    t_setup = time.perf_counter()
    hw = harness.DeviceWorkload(w, store_location="host", cache_from=dw_hbm)
    setup_s = time.perf_counter() - t_setup
    n = hw.n_tokens
    pcie_bytes = n * w.spec.bytes_per_token // 2     # the reads cross PCIe, the writes do not

    def wall(step):
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        assert int(hw.status.item()) == 0, "host-store inject reported skipped tokens"
        return (time.perf_counter() - t0) * 1e3 / steps

    kargs = hw.inject_args()

    def zero_copy():
        rc = lib.inject_topk(*kargs)
        if rc != 0:
            raise prkv.PrkvError(rc, "inject_topk", lib.last_error_string().decode())

    zc_ms = wall(zero_copy)
    # The link's attainable rate: the copy engine moving a contiguous run of
    # the same pinned arena into HBM (the batch's byte count, at most 1 GiB per
    # copy: the rate does not depend on size beyond that).
    n_copy = min(pcie_bytes, 1 << 30) // 2
    src = hw.k_arena.view(-1)[:n_copy]
    h2d_gbps = None
    try:
        dst = torch.empty(n_copy, dtype=torch.int16, device="cuda")
    except torch.cuda.OutOfMemoryError:
        dst = None      # no room beside the workload: reported as null
    if dst is not None:
        n_h2d = max(3, min(30, int(8e9 // (2 * n_copy))))     # about 8 GB in all
        dst.copy_(src, non_blocking=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n_h2d):
            dst.copy_(src, non_blocking=True)
        torch.cuda.synchronize()
        h2d_gbps = n_h2d * 2 * n_copy / (time.perf_counter() - t0) / 1e9
        del dst
    zc_gbps = pcie_bytes / (zc_ms * 1e-3) / 1e9
    out = {"setup_s": setup_s, "pcie_read_bytes": pcie_bytes,
           "zero_copy": {"ms": zc_ms, "added_ms": zc_ms - hbm_kernel_ms, "pcie_gbps": zc_gbps},
           "h2d_copy_engine_gbps": h2d_gbps,
           "zero_copy_frac_of_h2d_copy": zc_gbps / h2d_gbps if h2d_gbps else None}
    staged = {}
    for chunks in (1, 4, 16):
        st = harness.StagedInjector(hw, dw_hbm.k_arena, dw_hbm.v_arena, chunks=chunks)
        ms = wall(st.step)
        staged[str(len(st.pieces))] = {"ms": ms, "added_ms": ms - hbm_kernel_ms,
                                       "pcie_gbps": pcie_bytes / (ms * 1e-3) / 1e9}
        del st
    out["staged_by_chunks"] = staged
    best_chunks = min(staged, key=lambda c: staged[c]["ms"])
    out["staged_best"] = dict(staged[best_chunks], chunks=int(best_chunks))
    out["faster"] = "zero_copy" if zc_ms <= staged[best_chunks]["ms"] else "staged"
    out["what"] = ("store in pinned host DRAM: zero-copy = inject_topk reading host memory; "
                   "staged = store_stage_facts into HBM in chunks on a second stream + "
                   "inject_topk per chunk; ms per step by wall clock")
    del hw
    return out


def launch_floor(torch, stream, steps=200):
    """ms per launch of an empty kernel, back to back behind a clock spin (so
    the GPU, not the host, sets the pace): one workgroup, and 2,048 workgroups
    (the shortest time any launch can take here)."""
    lib = ceiling_lib()
    out = {}
    for grid in (1, 2048):
        ms, med = time_launches(torch, lambda g=grid: lib.ceiling_empty(g, stream.cuda_stream),
                                stream, steps, 10, queued=True)
        out[f"grid_{grid}_ms"] = ms
    # the same launches with an event recorded after each one: what an event
    # between launches adds to each
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    queue_ahead(torch, stream)
    evs[0].record(stream)
    for i in range(steps):
        lib.ceiling_empty(1, stream.cuda_stream)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    out["grid_1_event_per_launch_ms"] = evs[0].elapsed_time(evs[steps]) / steps
    return out


def device_info(torch):
    import socket
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "gcn_arch": getattr(p, "gcnArchName", ""),
            "cus": p.multi_processor_count, "hbm_gib": round(p.total_memory / 2**30, 1),
            "host": socket.gethostname()}


def cpu_baseline(w, budget_s):
    """The CPU oracle, as it stands, on a bounded sample of the same workload:
    facts of the requests in order, all layers, until the budget is spent."""
    import numpy as np

    from oracle import inject as oinject

    sp = w.spec
    done_tokens, done_facts, elapsed = 0, 0, 0.0
    reqs = w.requests()
    r_used = 0
    for r, (ids, prefix, bt) in enumerate(reqs):
        rows, ks, vs, row = {}, [], [], 0
        for f in sorted(set(ids)):
            k, v = w.fact_kv(f, device="cuda")
            ks.append(k.cpu().numpy().view(np.uint16))
            vs.append(v.cpu().numpy().view(np.uint16))
            rows[f] = (row, w.length_of(f))
            row += w.length_of(f)
        k_ar, v_ar = np.concatenate(ks, 1), np.concatenate(vs, 1)
        img_k = oinject.PagedImage(sp.num_layers, bt, sp.block_size, sp.num_kv_heads,
                                   sp.head_dim, 0x7F7F)
        img_v = oinject.PagedImage(sp.num_layers, bt, sp.block_size, sp.num_kv_heads,
                                   sp.head_dim, 0x7F7F)
        # one fact at a time so the sample can stop inside a request
        p = prefix
        for f in ids:
            t0 = time.perf_counter()
            n = oinject.inject(k_ar, v_ar, rows, [([f], p, bt)], sp.block_size, sp.rope_theta,
                               img_k, img_v)
            elapsed += time.perf_counter() - t0
            p += w.length_of(f)
            done_tokens += n
            done_facts += 1
            if elapsed >= budget_s:
                break
        r_used = r + 1
        if elapsed >= budget_s:
            break
    return {
        "value": done_tokens / elapsed,
        "unit": "injected KV tokens/s",
        "cores": 1,
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": (f"{done_tokens} tokens ({done_facts} facts of the first {r_used} "
                   f"request(s)), all {sp.num_layers} layers, rotate + scatter only, "
                   f"{elapsed:.1f} s on 1 host core (NumPy float64, single-threaded)"),
    }


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo (None if unreadable)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _pool_worker(task):
    """One worker of the multi-core oracle baseline: the oracle's inject for a
    range of layers of every sampled request.  Returns (token-layers, seconds)."""
    import numpy as np

    from oracle import inject as oinject

    folder, layers, reqs, spec_vals = task
    block_size, num_kv_heads, head_dim, theta = spec_vals
    done, spent = 0, 0.0
    for r, (ids, prefix, bt, rows) in enumerate(reqs):
        rows = {int(f): tuple(v) for f, v in rows.items()}
        k_ar = np.load(os.path.join(folder, f"k{r}.npy"), mmap_mode="r")[layers[0]:layers[1]]
        v_ar = np.load(os.path.join(folder, f"v{r}.npy"), mmap_mode="r")[layers[0]:layers[1]]
        k_ar, v_ar = np.ascontiguousarray(k_ar), np.ascontiguousarray(v_ar)
        nl = layers[1] - layers[0]
        img_k = oinject.PagedImage(nl, bt, block_size, num_kv_heads, head_dim, 0x7F7F)
        img_v = oinject.PagedImage(nl, bt, block_size, num_kv_heads, head_dim, 0x7F7F)
        t0 = time.perf_counter()
        n = oinject.inject(k_ar, v_ar, rows, [(ids, prefix, bt)], block_size, theta, img_k, img_v)
        spent += time.perf_counter() - t0
        done += n * nl
    return done, spent


def cpu_worker_main():
    """--cpu-worker: wait for one task (JSON on stdin), run it, print the result."""
    os.environ.setdefault("OMP_NUM_THREADS", "1")
    line = sys.stdin.readline()
    if not line.strip():
        return            # the bench ended without using this worker
    done, spent = _pool_worker(json.loads(line))
    print(json.dumps({"done": done, "spent": spent}), flush=True)


# the host CPU share that comes with one GPU here; more workers than that
# would compete with each other, not add cores
CPU_WORKER_CAP = 16


def start_cpu_workers():
    """Start the multi-core baseline's worker processes, idle until fed.  Called
    before this process makes any GPU call, so no child is ever started by a
    process that has initialised the GPU."""
    import subprocess
    visible = len(os.sched_getaffinity(0))
    n = min(visible, CPU_WORKER_CAP)
    env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1")
    procs = [subprocess.Popen([sys.executable, "-u", os.path.abspath(__file__), "--cpu-worker"],
                              stdin=subprocess.PIPE, stdout=subprocess.PIPE, text=True, env=env)
             for _ in range(n)]
    return {"procs": procs, "visible_cores": visible}


def stop_cpu_workers(workers):
    """End every worker: close its input (an idle worker then exits) and wait;
    kill the exact PID only if it does not exit."""
    if not workers:
        return
    for p in workers["procs"]:
        try:
            if p.stdin and not p.stdin.closed:
                p.stdin.close()
        except OSError:
            pass
    for p in workers["procs"]:
        try:
            p.wait(timeout=60)
        except Exception:
            p.kill()
            p.wait()


def cpu_baseline_pool(w, n_requests, workers, gen_device="cuda"):
    """The same oracle spread over the host's cores (the started worker
    processes, split by layer, as the work is independent per layer) on the
    first n_requests requests: tokens/s = sampled tokens / the slowest
    worker's compute time."""
    import shutil
    import tempfile

    import numpy as np

    sp = w.spec
    procs = workers["procs"]
    cores = min(len(procs), sp.num_layers)
    folder = tempfile.mkdtemp(prefix="prkv_pool_")
    try:
        reqs = []
        n_tok = 0
        for r, (ids, prefix, bt) in enumerate(w.requests()[:n_requests]):
            rows, ks, vs, row = {}, [], [], 0
            for f in sorted(set(ids)):
                k, v = w.fact_kv(f, device=gen_device)
                ks.append(k.cpu().numpy().view(np.uint16))
                vs.append(v.cpu().numpy().view(np.uint16))
                rows[int(f)] = (row, w.length_of(f))
                row += w.length_of(f)
            np.save(os.path.join(folder, f"k{r}.npy"), np.concatenate(ks, 1))
            np.save(os.path.join(folder, f"v{r}.npy"), np.concatenate(vs, 1))
            reqs.append(([int(f) for f in ids], int(prefix), [int(b) for b in bt], rows))
            n_tok += sum(w.length_of(f) for f in ids)
        edges = np.linspace(0, sp.num_layers, cores + 1).round().astype(int)
        vals = (sp.block_size, sp.num_kv_heads, sp.head_dim, sp.rope_theta)
        for i, p in enumerate(procs[:cores]):
            task = (folder, (int(edges[i]), int(edges[i + 1])), reqs, vals)
            p.stdin.write(json.dumps(task) + "\n")
            p.stdin.flush()
            p.stdin.close()
        res = []
        for p in procs[:cores]:
            out = json.loads(p.stdout.readline())
            res.append((out["done"], out["spent"]))
    finally:
        stop_cpu_workers(workers)
        shutil.rmtree(folder, ignore_errors=True)
    token_layers = sum(d for d, _ in res)
    assert token_layers == n_tok * sp.num_layers
    slowest = max(t for _, t in res)
    return {
        "value": n_tok / slowest,
        "unit": "injected KV tokens/s",
        "cores": cores,
        "cores_visible": workers["visible_cores"],
        "cores_cap": CPU_WORKER_CAP,
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": (f"{n_tok} tokens of the first {len(reqs)} request(s), all {sp.num_layers} "
                   f"layers split over {cores} worker processes (one per core, "
                   f"{workers['visible_cores']} cores visible, at most {CPU_WORKER_CAP} used: "
                   f"the host share of one GPU); rotate + scatter only; "
                   f"slowest worker {slowest:.1f} s, {sum(t for _, t in res):.1f} core-s in all"),
    }


def k_sweep_rows(args, torch, lib, w, dw, flusher):
    """The pages' retrieval-budget sweep (k = 5, 10, 20, 50) on one request:
    the device step (mapping + inject) for the first k facts of the drawn
    request of the 2,000-fact store, with the fused mapping (one launch) and
    with the separate plan and mapping kernels (forced by a max_facts bound
    above the fused limit), back to back (warm) and one launch at a time after
    a 1 GiB fill that evicts the MALL (cold)."""
    from pre_rope_kv_amd import prkv

    stream = dw.stream
    rows = []
    ptr_cap = 257        # a max_facts bound above the fused mapping's limit (256)
    big_ws = torch.zeros(prkv.inject_device_workspace_bytes(ptr_cap, dw.max_tokens),
                         dtype=torch.uint8, device=dw.device)

    def step_fn(k, max_facts, workspace):
        ptr = torch.tensor([0, k], dtype=torch.int32, device=dw.device)
        batch = prkv.device_batch(1, dw.d_bt.shape[1], max_facts, dw.max_tokens, ptr, dw.d_ids,
                                  dw.d_start, dw.d_bt, dw.d_bt_len)
        a = list(dw.inject_device_args())
        a[2] = ctypes.byref(batch)
        a[7], a[8] = workspace.data_ptr(), workspace.numel()

        def step(keep=(ptr, batch)):
            rc = lib.inject_topk_device(*a)
            if rc != 0:
                raise prkv.PrkvError(rc, "inject_topk_device", lib.last_error_string().decode())
        return step

    for k in (5, 10, 20, 50):
        fused = step_fn(k, k, dw.workspace)
        three = step_fn(k, ptr_cap, big_ws)
        ms, _ = time_launches(torch, fused, stream, args.steps, args.warmup, queued=True)
        ms3, _ = time_launches(torch, three, stream, args.steps, args.warmup, queued=True)
        ms_cold, med_cold = time_launches(torch, fused, stream, args.steps, args.warmup, flusher)
        assert int(dw.status.item()) == 0
        n_tok = sum(w.length_of(f) for f in w.retrieved[0][:k])
        nb = n_tok * w.spec.bytes_per_token
        rows.append({"k": k, "tokens": n_tok, "bytes_per_launch": nb,
                     "step_ms": ms, "tokens_per_s": n_tok / (ms * 1e-3),
                     "hbm_gbps": nb / (ms * 1e-3) / 1e9,
                     "step_ms_three_kernels": ms3,
                     "step_ms_cold": ms_cold, "step_median_ms_cold": med_cold,
                     "tokens_per_s_cold": n_tok / (ms_cold * 1e-3),
                     "hbm_gbps_cold": nb / (ms_cold * 1e-3) / 1e9})
    del big_ws
    return rows


def k_sweep(args):
    """--k-sweep: only the retrieval-budget sweep, as one JSON line."""
    import torch

    from pre_rope_kv_amd import harness, prkv, workloads

    lib = prkv.lib()
    torch.cuda.set_device(0)
    w = workloads.make("llama3_8b_k50")
    dw = harness.DeviceWorkload(w)
    dw.setup_device_batch()
    rows = k_sweep_rows(args, torch, lib, w, dw, Flusher(torch))
    print(json.dumps({"metric": "device step time vs retrieval budget k, 1 request, 1 MI355X",
                      "unit": "ms", "higher_is_better": False, "n_gpus": 1,
                      "steps": args.steps, "warmup": args.warmup, "dtype": "f32",
                      "data": "synthetic", "config": {"workload": "llama3_8b_k50 (first k facts)"},
                      "sweep": rows}), flush=True)


def single_user_step(args, torch, lib, w, dw, time_fn):
    """One request's GPU part of the time to first token: retrieve_topk over
    its store (ids written into the device batch), inject_topk_device, then
    attend_paged for 16 query tokens (the context's last positions) x 4
    query heads per KV head; the three calls back to back per step."""
    import math

    from pre_rope_kv_amd import prkv

    spec = w.spec
    # the prefix slots hold zeros (they are never injected), as in the
    # attention figure of the main workload
    with torch.cuda.stream(dw.stream):
        dw.k_cache.zero_()
        dw.v_cache.zero_()
    torch.cuda.synchronize()
    embs = [w.store_embeddings(si, "cuda") for si in range(spec.n_requests)]
    emb = torch.cat(embs, 0).contiguous()
    q_emb = w.query_embeddings("cuda", emb=embs)
    ws_b = prkv.retrieve_workspace_bytes(spec.n_requests, spec.facts_per_store)
    rws = torch.empty(ws_b, dtype=torch.uint8, device="cuda")
    d_rs = torch.as_tensor(w.req_store(), device="cuda")
    rargs = (emb.data_ptr(), spec.n_requests, spec.facts_per_store, spec.emb_dim,
             q_emb.data_ptr(), d_rs.data_ptr(), spec.n_requests, spec.k, dw.d_ids.data_ptr(),
             None, rws.data_ptr(), ws_b, dw.status.data_ptr(), dw.stream.cuda_stream)
    q_len, hq, D, L = ATTN_Q_LEN, ATTN_GROUP * spec.num_kv_heads, spec.head_dim, spec.num_layers
    ctxs = [int(w.prefix[r]) + sum(w.length_of(f) for f in ids)
            for r, ids in enumerate(w.retrieved)]
    g = torch.Generator(device="cuda")
    g.manual_seed(13)
    qt = torch.randn((spec.n_requests, q_len, hq, D), generator=g,
                     device="cuda").to(torch.bfloat16).view(torch.int16)
    q_start = torch.as_tensor([c - q_len for c in ctxs], dtype=torch.int32, device="cuda")
    out = torch.empty((L, spec.n_requests, q_len, hq, D), dtype=torch.float32, device="cuda")
    ab = prkv.attn_batch(spec.n_requests, q_len, hq, dw.d_bt.shape[1], qt, q_start, dw.d_bt,
                         dw.d_bt_len, out)
    kp = (ctypes.c_void_p * L)(*[t.data_ptr() for t in dw.k_layers()])
    vp = (ctypes.c_void_p * L)(*[t.data_ptr() for t in dw.v_layers()])
    aargs = (dw.store.handle, ctypes.byref(ab), kp, vp, spec.block_size, w.num_blocks,
             1.0 / math.sqrt(D), dw.status.data_ptr(), dw.stream.cuda_stream)
    dargs = dw.inject_device_args()

    def calls(*fa):
        for f, a in fa:
            rc = f(*a)
            if rc != 0:
                raise prkv.PrkvError(rc, f.__name__, lib.last_error_string().decode())
        return 0

    retrieve_ms = time_fn(lambda *a: calls((lib.retrieve_topk, rargs)), ())
    attend_ms = time_fn(lambda *a: calls((lib.attend_paged, aargs)), ())
    step_ms = time_fn(lambda *a: calls((lib.retrieve_topk, rargs),
                                       (lib.inject_topk_device, dargs),
                                       (lib.attend_paged, aargs)), ())
    assert bool(torch.isfinite(out).all()), "attention produced non-finite values"
    return {"what": "retrieve_topk + inject_topk_device + attend_paged (16 query tokens), "
                    "back to back, one request",
            "ms": step_ms, "retrieve_ms": retrieve_ms, "attend_ms": attend_ms}


# workloads far below the 256 MB MALL's reach are also timed cold
COLD_BELOW_BYTES = 1 << 30


def other_workloads(args, torch, lib, names):
    """Device step and inject kernel alone on each of `names`, each workload
    set up and released in turn: tokens/s of the step, algorithmic GB/s of
    the kernel, warm (back-to-back launches, events around args.steps of
    them) and, for workloads below 1 GiB per launch, cold (each launch after a
    1 GiB fill that evicts the MALL, so none of its data is cached); next to
    them the hand-written streaming copy of the same bytes, the step with the
    duplicate-slot check, and on the 2,000-fact store the k sweep."""
    import gc

    from pre_rope_kv_amd import harness, prkv, workloads

    flusher = Flusher(torch)
    rows = {"launch_floor": launch_floor(torch, torch.cuda.current_stream())}
    for name in names:
        spec = workloads.SPECS[name]
        if args.cache_layout == "hnd":
            spec = workloads.dataclasses.replace(spec, cache_layout=prkv.CACHE_HND)
        w0 = workloads.make(spec)
        nb = harness.fit_num_blocks(spec, 2 * w0.capacity_rows * spec.num_layers *
                                    spec.row_bytes + (1 << 30))
        w = w0 if nb == spec.num_blocks else workloads.make(spec, num_blocks=nb)
        dw = harness.DeviceWorkload(w)
        dw.setup_device_batch()
        stream = dw.stream

        def caller(fn, a):
            def call():
                rc = fn(*a)
                if rc != 0:
                    raise prkv.PrkvError(rc, fn.__name__, lib.last_error_string().decode())
            return call

        def time_fn(fn, a):       # the single-user step's signature
            ms, _ = time_launches(torch, caller(fn, a), stream, args.steps, args.warmup)
            assert int(dw.status.item()) == 0, f"{name}: skipped tokens"
            return ms

        step = caller(lib.inject_topk_device, dw.inject_device_args())
        kernel = caller(lib.inject_topk, dw.inject_args())
        alg = dw.n_tokens * spec.bytes_per_token
        cold = alg < COLD_BELOW_BYTES
        step_ms, step_med = time_launches(torch, step, stream, args.steps, args.warmup,
                                          queued=cold)
        kernel_ms, kernel_med = time_launches(torch, kernel, stream, args.steps, args.warmup,
                                              queued=cold)
        assert int(dw.status.item()) == 0, f"{name}: skipped tokens"
        profiled = w is w0 and args.cache_layout == "nhd"
        row = {
            "tokens": dw.n_tokens, "layers": spec.num_layers, "kv_heads": spec.num_kv_heads,
            "requests": spec.n_requests, "k": spec.k, "block_size": spec.block_size,
            "num_blocks": w.num_blocks, "bytes_per_launch": alg,
            "warm": {"timing": "back to back in 3 runs, each enqueued behind a clock spin and "
                               "timed by two events around it (none between launches)",
                     "step_ms": step_ms, "step_median_ms": step_med,
                     "tokens_per_s": dw.n_tokens / (step_ms * 1e-3),
                     "kernel_ms": kernel_ms, "kernel_median_ms": kernel_med,
                     "hbm_gbps": alg / (kernel_ms * 1e-3) / 1e9,
                     "frac_of_peak": alg / (kernel_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS},
            "traffic": read_profile_traffic(name) if profiled else None,
        }
        if cold:
            c_step, c_step_med = time_launches(torch, step, stream, args.steps, args.warmup,
                                               flusher)
            c_kern, c_kern_med = time_launches(torch, kernel, stream, args.steps, args.warmup,
                                               flusher)
            assert int(dw.status.item()) == 0, f"{name}: skipped tokens"
            row["cold"] = {"timing": "every launch after a 1 GiB fill that evicts the MALL: "
                                     "runs of (fill, launch) minus runs of fills alone, each "
                                     "between two events",
                           "step_ms": c_step, "step_median_ms": c_step_med,
                           "tokens_per_s": dw.n_tokens / (c_step * 1e-3),
                           "kernel_ms": c_kern, "kernel_median_ms": c_kern_med,
                           "hbm_gbps": alg / (c_kern * 1e-3) / 1e9,
                           "frac_of_peak": alg / (c_kern * 1e-3) / 1e9 / PEAK_HBM_GBPS}
        ceil = None if args.no_ceiling else \
            gather_scatter_ceiling(torch, dw, args.steps, args.warmup, flusher if cold else None)
        if ceil is not None:
            row["ceiling_copy"] = ceil
            row["warm"]["frac_of_ceiling"] = row["warm"]["hbm_gbps"] / ceil["gbps"]
            if cold:
                row["cold"]["frac_of_ceiling"] = row["cold"]["hbm_gbps"] / ceil["cold_gbps"]
        if not args.no_slot_check:
            dw.setup_device_batch(flags=prkv.BATCH_CHECK_SLOTS)
            chk = caller(lib.inject_topk_device, dw.inject_device_args())
            chk_ms, _ = time_launches(torch, chk, stream, args.steps, args.warmup)
            assert int(dw.status.item()) == 0, f"{name}: slot check flagged a valid batch"
            row["slot_check"] = {"step_ms": chk_ms, "added_ms": chk_ms - step_ms}
            dw.setup_device_batch()
        if name == "llama3_8b_k50":
            row["k_sweep"] = k_sweep_rows(args, torch, lib, w, dw, flusher)
        if name in ("llama3_8b_k5", "llama3_8b_k50") and not args.no_host_store:
            row["host_store"] = host_store_figures(torch, lib, w, dw, min(args.steps, 20),
                                                   2, kernel_ms)
        if spec.n_requests == 1 and spec.head_dim in (64, 128) and not args.no_retrieve \
                and not args.no_attend:
            row["serving_step"] = single_user_step(args, torch, lib, w, dw, time_fn)
        rows[name] = row
        del dw, w, w0
        gc.collect()
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return rows


def placement_probe(args):
    """--placement-probe: one workload's inject kernel and a plain copy
    between the same addresses (gather_scatter_ceiling), each timed on four
    successive allocations of its store and cache in one process: the first,
    the same freed and allocated again, one made after the 64-request batch
    (256 GiB of cache) was allocated, injected and freed, and that one freed
    and allocated again.  Prints one JSON line.  Shows whether a change of
    rate follows the kernel or the buffers."""
    import gc

    import torch

    from pre_rope_kv_amd import harness, prkv, workloads

    lib = prkv.lib()
    torch.cuda.set_device(0)
    spec = workloads.SPECS[args.workload]
    phases = []

    def measure(tag):
        w = workloads.make(spec)
        dw = harness.DeviceWorkload(w)
        kargs = dw.inject_args()

        def kernel():
            rc = lib.inject_topk(*kargs)
            if rc != 0:
                raise prkv.PrkvError(rc, "inject_topk", lib.last_error_string().decode())

        ms, _ = time_launches(torch, kernel, dw.stream, args.steps, args.warmup)
        ceil = gather_scatter_ceiling(torch, dw, args.steps, args.warmup)
        nb = dw.n_tokens * spec.bytes_per_token
        phases.append({"phase": tag, "kernel_ms": ms, "kernel_gbps": nb / (ms * 1e-3) / 1e9,
                       "copy_mapped_gbps": ceil["mapped"]["gbps"],
                       "copy_contiguous_gbps": ceil["contiguous"]["gbps"],
                       "kernel_over_copy": nb / (ms * 1e-3) / 1e9 / ceil["mapped"]["gbps"],
                       "k_cache_va": hex(dw.k_cache.data_ptr()),
                       "v_cache_va": hex(dw.v_cache.data_ptr())})
        print(json.dumps(phases[-1]), file=sys.stderr, flush=True)
        del dw
        gc.collect()
        torch.cuda.synchronize()
        torch.cuda.empty_cache()

    measure("allocation 1")
    measure("allocation 2: freed and allocated again")
    big = harness.DeviceWorkload(workloads.make("llama3_8b_batch64_k50"))
    big.inject()
    torch.cuda.synchronize()
    del big
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    measure("allocation 3: after the 64-request batch was allocated, injected and freed")
    measure("allocation 4: freed and allocated again")
    print(json.dumps({"what": "placement probe: inject kernel vs a plain copy between the same "
                              "addresses on successive allocations", "workload": spec.name,
                      "steps": args.steps, "phases": phases}), flush=True)


def other_workloads_child(args, names):
    """other_workloads() in a child process of its own (started, not exec'd),
    so that its allocations see the device as a fresh process would."""
    import subprocess
    cmd = [sys.executable, "-u", os.path.abspath(__file__), "--other-workloads-only",
           ",".join(names), "--steps", str(args.steps), "--warmup", str(args.warmup),
           "--cache-layout", args.cache_layout]
    for flag in ("no_ceiling", "no_slot_check", "no_host_store", "no_retrieve", "no_attend"):
        if getattr(args, flag):
            cmd.append("--" + flag.replace("_", "-"))
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
    if res.returncode != 0:
        raise RuntimeError(f"other-workload timing failed (exit {res.returncode}):\n"
                           f"{res.stderr[-3000:]}")
    return json.loads(res.stdout.strip().splitlines()[-1])


def main():
    args = parse()
    if args.cpu_worker:
        cpu_worker_main()
        return
    if args.other_workloads_only:
        import torch

        from pre_rope_kv_amd import prkv
        lib = prkv.lib()
        torch.cuda.set_device(0)
        print(json.dumps(other_workloads(args, torch, lib, args.other_workloads_only.split(","))),
              flush=True)
        return
    if args.summarize_profile:
        trace_dir, fetch_dir, write_dir = args.summarize_profile
        regex = "|".join(list(PROFILED) + ["copyBuffer"])
        wl = "" if args.workload == DEFAULT_WORKLOAD else f"--workload {args.workload} "
        cmds = [
            f"rocprofv3 --kernel-trace --stats -T -d {trace_dir} -o inject -f csv -- "
            f"python -u bench.py {wl}--steps 20 --warmup 5 {PROFILE_FLAGS}",
            f"rocprofv3 --pmc FETCH_SIZE --kernel-include-regex \"{regex}\" "
            f"-T -d {fetch_dir} -o fetch -f csv -- python -u bench.py {wl}--steps 3 --warmup 1 "
            f"{PROFILE_FLAGS}",
            f"rocprofv3 --pmc WRITE_SIZE --kernel-include-regex \"{regex}\" "
            f"-T -d {write_dir} -o write -f csv -- python -u bench.py {wl}--steps 3 --warmup 1 "
            f"{PROFILE_FLAGS}",
            f"python bench.py --workload {args.workload} --summarize-profile {trace_dir} "
            f"{fetch_dir} {write_dir}",
        ]
        summarize_profile(args.workload, trace_dir, fetch_dir, write_dir, cmds)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.k_sweep and args.gpus == 1 and world == 1:
        k_sweep(args)
        return
    if args.placement_probe and args.gpus == 1 and world == 1:
        placement_probe(args)
        return
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}); the inject path needs no collective and shards by "
              "request, KV head or layer range with no exchange step.", file=sys.stderr)
        sys.exit(2)
    # Every child process is started here, before this process makes any GPU
    # call: the CPU-baseline workers (idle until fed) and, run to completion,
    # the other-workloads child.
    workers = None
    if not args.no_cpu_baseline and args.pool_requests > 0:
        workers = start_cpu_workers()
    try:
        run(args, workers)
    finally:
        stop_cpu_workers(workers)


def run(args, workers):
    # The other workloads first, in a child process, while this process has
    # not touched the GPU: timed after this process had allocated and freed
    # the 64-request batch, the 80-layer batch ran 7 % slower than on a fresh
    # device (5.61 vs 5.24 ms on one box).
    others = None
    if not args.no_other_workloads and args.store == "device" and not args.flush:
        names = [n for n in ("tiny_L1_H2_D64", "llama3_8b_k5", "llama3_8b_k50",
                             "llama3_8b_batch64_k50", "llama3_70b_batch16_k50",
                             "llama3_8b_batch64_k50_h1")
                 if n != args.workload]
        others = other_workloads_child(args, names)

    import torch

    from pre_rope_kv_amd import harness, prkv, workloads

    lib = prkv.lib()
    torch.cuda.set_device(0)

    ceiling = copy_ceiling_gbps(torch)

    spec = workloads.SPECS[args.workload]
    if args.cache_layout == "hnd":
        spec = workloads.dataclasses.replace(spec, cache_layout=prkv.CACHE_HND)
    w0 = workloads.make(spec)
    reserve = (2 * w0.capacity_rows * spec.num_layers * spec.row_bytes
               if args.store == "device" else 0) + (1 << 30)
    nb = harness.fit_num_blocks(spec, reserve)
    w = w0 if nb == spec.num_blocks else workloads.make(spec, num_blocks=nb)
    # the committed counter summaries were taken on the default configuration
    profiled_config = w is w0 and args.store == "device" and args.cache_layout == "nhd"
    t_setup = time.perf_counter()
    dw = harness.DeviceWorkload(w, store_location=args.store)
    dw.setup_device_batch()
    setup_s = time.perf_counter() - t_setup
    stream = dw.stream
    kargs = dw.inject_args()
    dargs = dw.inject_device_args()

    def call(fn, a, name):
        rc = fn(*a)
        if rc != 0:
            raise prkv.PrkvError(rc, name, lib.last_error_string().decode())

    def step_device():
        call(lib.inject_topk_device, dargs, "inject_topk_device")

    def step_kernel():
        call(lib.inject_topk, kargs, "inject_topk")

    flusher = Flusher(torch) if args.flush else None

    def timed(step):
        """(wall seconds, sorted per-launch ms, mean ms) of args.steps launches."""
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        if flusher is not None:
            # launches timed one by one, each after a 1 GiB fill that evicts the MALL
            starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
            ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(args.steps):
                flusher(torch, stream)
                starts[i].record(stream)
                step()
                ends[i].record(stream)
            torch.cuda.synchronize()
            wall = time.perf_counter() - t0
            per = sorted(starts[i].elapsed_time(ends[i]) for i in range(args.steps))
            return wall, per, sum(per) / len(per)
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        evs[0].record(stream)
        for i in range(args.steps):
            step()
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        per = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
        return wall, per, evs[0].elapsed_time(evs[args.steps]) / args.steps

    # the step: the whole path on the device from the HBM-resident batch
    wall_s, step_per_ms, step_ms = timed(step_device)
    assert int(dw.status.item()) == 0, "device path reported skipped tokens"
    ms_per_step = step_ms if flusher is not None else max(wall_s * 1e3 / args.steps, step_ms)
    # the dominant kernel alone (same kernel, mapping already resident)
    _, per_ms, kernel_ms = timed(step_kernel)
    assert int(dw.status.item()) == 0

    # the plain copy of the same bytes between the same addresses (and a
    # contiguous one), for the attainable-bandwidth reference
    own_ceiling = None if args.no_ceiling else \
        gather_scatter_ceiling(torch, dw, args.steps, args.warmup, flusher)

    graph = None
    if args.graph:
        # the step captured once and replayed: kernels only, no host work
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        torch.cuda.synchronize()
        gargs = list(dargs)
        gargs[-1] = side.cuda_stream
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            call(lib.inject_topk_device, gargs, "inject_topk_device")
        torch.cuda.synchronize()
        _, g_per, g_ms = timed(g.replay)
        assert int(dw.status.item()) == 0
        graph = {"what": "inject_topk_device captured in a HIP graph, replayed",
                 "ms": g_ms, "median_ms": g_per[len(g_per) // 2],
                 "tokens_per_s": dw.n_tokens / (g_ms * 1e-3)}

    perm = None
    if not args.no_permute:
        # the same facts of every request in another order: other positions
        # and slots for the same token count (assembly order is free)
        import numpy as np
        rng = np.random.default_rng(2024)
        req_ptr, ids, _, _, _ = w.csr()
        pids = ids.copy()
        for r in range(len(req_ptr) - 1):
            pids[req_ptr[r]:req_ptr[r + 1]] = rng.permutation(ids[req_ptr[r]:req_ptr[r + 1]])
        d_pids = torch.from_numpy(pids).to(dw.device)
        pbatch = prkv.device_batch(len(req_ptr) - 1, dw.d_bt.shape[1], dw.max_facts,
                                   dw.max_tokens, dw.d_req_ptr, d_pids, dw.d_start, dw.d_bt,
                                   dw.d_bt_len)
        pargs = list(dargs)
        pargs[2] = ctypes.byref(pbatch)

        def step_perm():
            call(lib.inject_topk_device, pargs, "inject_topk_device")

        _, _, p_ms = timed(step_perm)
        assert int(dw.status.item()) == 0
        perm = {"what": "the step with every request's facts in a shuffled order",
                "ms": p_ms, "ratio_to_step": p_ms / step_ms}
        step_device()   # facts back in drawn order

    slot_check = None
    if not args.no_slot_check:
        # the same step with the device duplicate-slot check on
        dw.setup_device_batch(flags=prkv.BATCH_CHECK_SLOTS)
        cargs = dw.inject_device_args()

        def step_checked():
            call(lib.inject_topk_device, cargs, "inject_topk_device")

        _, _, c_ms = timed(step_checked)
        assert int(dw.status.item()) == 0, "the slot check flagged a valid batch"
        slot_check = {"what": "the step with PRKV_BATCH_CHECK_SLOTS (slot set cleared, "
                              "filled by the mapping kernel, colliding tokens marked)",
                      "ms": c_ms, "added_ms": c_ms - step_ms}
        dw.setup_device_batch()
        dargs = dw.inject_device_args()

    n_tok = dw.n_tokens
    alg_bytes = n_tok * spec.bytes_per_token
    achieved = alg_bytes / (kernel_ms * 1e-3) / 1e9
    traffic = read_profile_traffic(spec.name) if profiled_config else None

    e2e = None
    if not args.no_e2e:
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(args.steps):
            dw.map_and_copy()
            step_kernel()
        torch.cuda.synchronize()
        e2e_ms = (time.perf_counter() - t1) * 1e3 / args.steps
        e2e = {"ms_per_step": e2e_ms, "tokens_per_s": n_tok / (e2e_ms * 1e-3),
               "what": "host build_slot_mapping + pinned H2D of the mapping + inject_topk"}

    retrieval = None
    if not args.no_retrieve:
        # retrieval embeddings per store, queries built around the drawn facts
        embs = [w.store_embeddings(si, "cuda") for si in range(spec.n_requests)]
        emb = torch.cat(embs, 0).contiguous()
        q = w.query_embeddings("cuda", emb=embs)
        del embs
        ws_b = prkv.retrieve_workspace_bytes(spec.n_requests, spec.facts_per_store)
        rws = torch.empty(ws_b, dtype=torch.uint8, device="cuda")
        d_rs = torch.as_tensor(w.req_store(), device="cuda")
        rargs = (emb.data_ptr(), spec.n_requests, spec.facts_per_store, spec.emb_dim,
                 q.data_ptr(), d_rs.data_ptr(), spec.n_requests, spec.k, dw.d_ids.data_ptr(),
                 None, rws.data_ptr(), ws_b, dw.status.data_ptr(), stream.cuda_stream)

        def step_retrieve():
            call(lib.retrieve_topk, rargs, "retrieve_topk")

        def step_both():
            step_retrieve()
            step_device()

        r_ms = time_span(torch, step_retrieve, stream, args.steps, args.warmup)
        _, _, b_ms = timed(step_both)
        assert int(dw.status.item()) == 0, "retrieve + inject reported skipped tokens"
        emb_bytes = spec.n_requests * spec.facts_per_store * spec.emb_dim * 2
        read_ceiling = None
        if not args.no_ceiling:
            # the same embedding bytes read once by a plain streaming kernel (16-byte
            # nontemporal loads, slices per workgroup), fastest of 16 launch shapes
            clib = ceiling_lib()
            sink = torch.zeros(256, dtype=torch.int32, device="cuda")
            for per_lane in (1, 2, 4, 8):
                for grid in (1024, 2048, 4096, 8192):
                    def step_read(pl=per_lane, g=grid):
                        rc = clib.ceiling_read(emb.data_ptr(), emb_bytes, sink.data_ptr(), pl, g,
                                               stream.cuda_stream)
                        if rc != 0:
                            raise RuntimeError(f"ceiling_read failed ({rc})")
                    c_ms = time_span(torch, step_read, stream, args.steps, args.warmup)
                    if read_ceiling is None or c_ms < read_ceiling["ms"]:
                        read_ceiling = {"ms": c_ms, "gbps": emb_bytes / (c_ms * 1e-3) / 1e9,
                                        "per_lane": per_lane, "grid": grid}
            del sink
        retrieval = {
            "what": "retrieve_topk: exact inner-product top-k over each request's store "
                    f"({spec.facts_per_store} facts x {spec.emb_dim} bf16), then "
                    "inject_topk_device on the retrieved ids",
            "retrieve_ms": r_ms,
            "retrieve_embedding_gbps": emb_bytes / (r_ms * 1e-3) / 1e9,
            "read_ceiling": read_ceiling,
            "retrieve_pct_of_read_ceiling": (100.0 * read_ceiling["ms"] / r_ms
                                             if read_ceiling else None),
            "retrieve_and_inject_ms": b_ms,
            "retrieve_and_inject_tokens_per_s": n_tok / (b_ms * 1e-3),
            "score_kernel_bytes_per_launch": algorithmic_bytes("score_kernel", w)[0],
            "score_kernel_traffic": (read_profile_traffic(spec.name, "score_kernel")
                                     if profiled_config else None),
        }
        del emb, q, rws

    attn = None
    if not args.no_attend and spec.head_dim in (64, 128):
        # query prefill over the injected cache: the last q_len positions of each
        # request's context act as its query (16 tokens, 4 query heads per KV head)
        import math
        q_len, hq = ATTN_Q_LEN, ATTN_GROUP * spec.num_kv_heads
        with torch.cuda.stream(stream):
            dw.k_cache.zero_()
            dw.v_cache.zero_()
        step_kernel()   # facts back in the (otherwise zero) cache
        ctxs = [int(w.prefix[r]) + sum(w.length_of(f) for f in ids)
                for r, ids in enumerate(w.retrieved)]
        g = torch.Generator(device="cuda")
        g.manual_seed(11)
        qt = torch.randn((spec.n_requests, q_len, hq, spec.head_dim), generator=g,
                         device="cuda").to(torch.bfloat16).view(torch.int16)
        q_start = torch.as_tensor([c - q_len for c in ctxs], dtype=torch.int32, device="cuda")
        out = torch.empty((spec.num_layers, spec.n_requests, q_len, hq, spec.head_dim),
                          dtype=torch.float32, device="cuda")
        ab = prkv.attn_batch(spec.n_requests, q_len, hq, dw.d_bt.shape[1], qt, q_start, dw.d_bt,
                             dw.d_bt_len, out)
        akp = (ctypes.c_void_p * spec.num_layers)(*[t.data_ptr() for t in dw.k_layers()])
        avp = (ctypes.c_void_p * spec.num_layers)(*[t.data_ptr() for t in dw.v_layers()])
        aargs = (dw.store.handle, ctypes.byref(ab), akp, avp, spec.block_size, w.num_blocks,
                 1.0 / math.sqrt(spec.head_dim), dw.status.data_ptr(), stream.cuda_stream)

        def step_attend():
            call(lib.attend_paged, aargs, "attend_paged")

        _, a_per, a_ms = timed(step_attend)
        assert int(dw.status.item()) == 0
        assert bool(torch.isfinite(out).all()), "attention produced non-finite values"
        kv_bytes, a_alg = attention_bytes(w)
        assert kv_bytes == sum(ctxs) * spec.num_layers * spec.num_kv_heads * spec.head_dim * 4
        flops = sum(ctxs) * spec.num_layers * hq * q_len * spec.head_dim * 4
        a_traffic = read_profile_traffic(spec.name, "attend_kernel") if profiled_config else None
        gather_ceiling = gather_by_heads = None
        if not args.no_ceiling and not dw.hnd:
            # the same cache rows (every context position's K and V rows, through the
            # same block tables, in the same XCD-aware workgroup order) read by a plain
            # gather with no arithmetic, fastest of 1-8 passes in flight x plain /
            # nontemporal loads; one workgroup per (layer, request, KV head) as the
            # attention kernel splits the work, and for comparison per 2, 4, 8 adjacent
            # heads (longer contiguous pieces of each cache row)
            clib = ceiling_lib()
            sink = torch.zeros(256, dtype=torch.int32, device="cuda")
            d_ctx = torch.as_tensor(ctxs, dtype=torch.int32, device="cuda")
            layer_bytes = dw.k_cache.stride(0) * dw.k_cache.element_size()
            gather_by_heads = {}
            for hg in (1, 2, 4, 8):
                if spec.num_kv_heads % hg or 256 % (hg * spec.head_dim // 8):
                    continue
                best = None
                for nt in (0, 1):
                    for passes in (1, 2, 4, 8):
                        def step_gather(ps=passes, n=nt, h=hg):
                            rc = clib.ceiling_gather_kv(
                                dw.k_cache.data_ptr(), dw.v_cache.data_ptr(), layer_bytes,
                                spec.num_layers, spec.num_kv_heads, spec.head_dim,
                                dw.d_bt.data_ptr(), dw.d_bt.shape[1], dw.d_bt_len.data_ptr(),
                                d_ctx.data_ptr(), spec.n_requests, spec.block_size,
                                w.num_blocks, h, sink.data_ptr(), ps, n, stream.cuda_stream)
                            if rc != 0:
                                raise RuntimeError(f"ceiling_gather_kv failed ({rc})")
                        c_ms = time_span(torch, step_gather, stream, args.steps, args.warmup)
                        if best is None or c_ms < best["ms"]:
                            best = {"ms": c_ms, "gbps": kv_bytes / (c_ms * 1e-3) / 1e9,
                                    "passes": passes, "nontemporal": bool(nt)}
                gather_by_heads[str(hg)] = best
            gather_ceiling = gather_by_heads["1"]
            del sink, d_ctx
        attn = {
            "what": f"attend_paged: {q_len} query tokens x {hq} query heads per request over "
                    "its whole context in the paged cache, all layers, one launch",
            "ms": a_ms,
            "kv_bytes": kv_bytes,
            "hbm_gbps": kv_bytes / (a_ms * 1e-3) / 1e9,
            "pct_of_hbm_peak": 100.0 * kv_bytes / (a_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
            "tflops": flops / (a_ms * 1e-3) / 1e12,
            "pct_of_bf16_mfma_peak": 100.0 * flops / (a_ms * 1e-3) / 1e12 / 2500.0,
            "roofline": {"bound": "hbm", "achieved": a_alg / (a_ms * 1e-3) / 1e9,
                         "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                         "frac": a_alg / (a_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                         "traffic": a_traffic, "kernel": f"attend_kernel<{spec.head_dim}>",
                         "bytes_per_launch": a_alg},
            "bound": "hbm (about 64 flop per byte of cache read, below the MFMA ridge)",
            "gather_ceiling": gather_ceiling,
            "pct_of_gather_ceiling": (100.0 * gather_ceiling["ms"] / a_ms
                                      if gather_ceiling else None),
            "gather_ceiling_by_heads_per_workgroup": gather_by_heads,
        }
        del out, qt

    host_store = None
    if not args.no_host_store and args.store == "device" and not dw.hnd:
        host_store = host_store_figures(torch, lib, w, dw, min(args.steps, 5), 1, kernel_ms)

    cpu = cpu_pool = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_seconds)
        if workers is not None:
            cpu_pool = cpu_baseline_pool(w, args.pool_requests, workers)


    out = {
        "metric": METRIC,
        "value": n_tok * args.steps / (ms_per_step * args.steps * 1e-3),
        "unit": "injected KV tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": spec.name, "storage": "bf16",
            "store": "HBM" if args.store == "device" else "host DRAM, pinned, read over PCIe",
            "layers": spec.num_layers,
            "kv_heads": spec.num_kv_heads, "head_dim": spec.head_dim,
            "requests": spec.n_requests, "k": spec.k, "tokens": n_tok,
            "block_size": spec.block_size, "num_blocks": w.num_blocks,
            "cache_layout": args.cache_layout.upper(),
            "num_blocks_spec": spec.num_blocks, "parallelism": "single GPU",
        },
        "hbm_gbps": achieved,
        "pct_of_peak": 100.0 * achieved / PEAK_HBM_GBPS,
        "pct_of_copy_ceiling": (100.0 * achieved / own_ceiling["gbps"]) if own_ceiling else None,
        "copy_ceiling": {
            "what": "plain copy of the launch's bytes (libprkv_ceiling.so): every token's K "
                    "and V row of every layer from arena to cache, no rotation, 16-byte "
                    "nontemporal loads and stores; mapped = the batch's own arena rows and "
                    "cache slots, contiguous = rows t -> t; best of two wave orders x three "
                    "workgroup sizes",
            "hand_written": own_ceiling, "library_copies_gbps": ceiling},
        "step": "inject_topk_device: plan + per-token mapping + inject kernels, batch "
                "(fact ids, prefixes, block tables) resident in HBM",
        "step_ms": {"mean": step_ms, "median": step_per_ms[len(step_per_ms) // 2]},
        "kernel_ms": {"mean": kernel_ms, "p10": per_ms[len(per_ms) // 10],
                      "median": per_ms[len(per_ms) // 2], "p90": per_ms[(9 * len(per_ms)) // 10]},
        "roofline": ({
            "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBPS, "traffic": traffic,
            "kernel": f"inject_kernel<{spec.head_dim}>",
            "bytes_per_launch": alg_bytes,
        } if args.store == "device" else {
            # reads of the retrieved rows cross PCIe (host -> device); writes stay in HBM
            "bound": "pcie", "achieved": (alg_bytes / 2) / (kernel_ms * 1e-3) / 1e9,
            "peak": PEAK_PCIE_GBPS, "unit": "GB/s",
            "frac": (alg_bytes / 2) / (kernel_ms * 1e-3) / 1e9 / PEAK_PCIE_GBPS,
            "traffic": None, "kernel": f"inject_kernel<{spec.head_dim}>",
            "bytes_per_launch": alg_bytes // 2,
        }),
        "cpu_baseline": cpu,
        "cpu_baseline_all_cores": cpu_pool,
        "permuted_order": perm,
        "slot_check": slot_check,
        "host_store": host_store,
        "graph_replay": graph,
        "retrieval": retrieval,
        "attention": attn,
        "other_workloads": others,
        "e2e": e2e,
        "setup_s": setup_s,
        "timing": "per-launch events after a 1 GiB MALL flush" if args.flush
                  else "back-to-back launches, events around the batch",
        "device": device_info(torch),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
