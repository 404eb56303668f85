#!/usr/bin/env python3
"""Benchmark of the retrieve-and-inject hot path on one MI355X.

A step is one inject_topk launch over the whole batch: every retrieved fact's
pre-RoPE K/V rows are gathered from the HBM-resident store, K is rotated to
its serving-time positions, and K and V are scattered into the paged cache,
for all layers, KV heads and requests.  The store, the cache and the slot
mapping are resident in HBM before the timed region.  The PCIe-inclusive
variant (host build_slot_mapping + H2D of the mapping + inject) is reported
separately under "e2e" and is never `value`.

Prints one JSON line.  Only one GPU: --gpus above 1 exits with a message.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "injected KV tokens/s (all layers) + achieved HBM GB/s and % of peak, 1 MI355X"
PEAK_HBM_GBPS = 8000.0
DEFAULT_WORKLOAD = "llama3_8b_batch64_k50"


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="wall-clock budget of the CPU-oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-e2e", action="store_true")
    return ap.parse_args()


def copy_ceiling_gbps(torch, nbytes=4 << 30, reps=10):
    """Device-to-device copy rate (read + write bytes / time) for context."""
    src = torch.empty(nbytes // 2, dtype=torch.int16, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(2):
        dst.copy_(src)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(reps):
        dst.copy_(src)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    del src, dst
    torch.cuda.empty_cache()
    return 2 * nbytes / (ms * 1e-3) / 1e9


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
        "kind": "oracle",
        "sample": (f"{done_tokens} tokens ({done_facts} facts of the first {r_used} "
                   f"request(s)), all {sp.num_layers} layers, rotate + scatter only, "
                   f"{elapsed:.1f} s on 1 host core (NumPy float64, single-threaded)"),
    }


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}); the inject path needs no collective and shards by "
              "request, KV head or layer range with no exchange step.", file=sys.stderr)
        sys.exit(2)

    import torch

    from pre_rope_kv_amd import harness, prkv, workloads

    lib = prkv.lib()
    torch.cuda.set_device(0)
    ceiling = copy_ceiling_gbps(torch)

    spec = workloads.SPECS[args.workload]
    w0 = workloads.make(args.workload)
    reserve = 2 * w0.capacity_rows * spec.num_layers * spec.row_bytes + (1 << 30)
    nb = harness.fit_num_blocks(spec, reserve)
    w = w0 if nb == spec.num_blocks else workloads.make(args.workload, num_blocks=nb)
    t_setup = time.perf_counter()
    dw = harness.DeviceWorkload(w)
    setup_s = time.perf_counter() - t_setup
    a = dw.inject_args()
    stream = dw.stream

    def step():
        rc = lib.inject_topk(*a)
        if rc != 0:
            raise prkv.PrkvError(rc, "inject_topk", lib.last_error_string().decode())

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert int(dw.status.item()) == 0

    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(args.steps):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t0
    per_ms = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    kernel_ms = evs[0].elapsed_time(evs[args.steps]) / args.steps
    ms_per_step = max(wall_s * 1e3 / args.steps, kernel_ms)

    n_tok = dw.n_tokens
    alg_bytes = n_tok * spec.bytes_per_token
    achieved = alg_bytes / (kernel_ms * 1e-3) / 1e9

    e2e = None
    if not args.no_e2e:
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(args.steps):
            dw.map_and_copy()
            step()
        torch.cuda.synchronize()
        e2e_ms = (time.perf_counter() - t1) * 1e3 / args.steps
        e2e = {"ms_per_step": e2e_ms, "tokens_per_s": n_tok / (e2e_ms * 1e-3),
               "what": "host build_slot_mapping + pinned H2D of the mapping + inject_topk"}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_seconds)

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
            "workload": spec.name, "storage": "bf16", "layers": spec.num_layers,
            "kv_heads": spec.num_kv_heads, "head_dim": spec.head_dim,
            "requests": spec.n_requests, "k": spec.k, "tokens": n_tok,
            "block_size": spec.block_size, "num_blocks": w.num_blocks,
            "num_blocks_spec": spec.num_blocks, "parallelism": "single GPU",
        },
        "hbm_gbps": achieved,
        "pct_of_peak": 100.0 * achieved / PEAK_HBM_GBPS,
        "pct_of_copy_ceiling": 100.0 * achieved / ceiling,
        "copy_ceiling_gbps": ceiling,
        "kernel_ms": {"mean": kernel_ms, "p10": per_ms[len(per_ms) // 10],
                      "median": per_ms[len(per_ms) // 2], "p90": per_ms[(9 * len(per_ms)) // 10]},
        "roofline": {
            "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBPS, "traffic": None,
            "kernel": "inject_kernel<128>",
            "bytes_per_launch": alg_bytes,
        },
        "cpu_baseline": cpu,
        "e2e": e2e,
        "setup_s": setup_s,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
