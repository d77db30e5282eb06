#!/usr/bin/env python3
"""Benchmark of one absorbed-MLA decode step on one MI355X.

Workload: the DeepSeek-V3-shaped single-layer decode, bf16 with fp32
accumulation: B=32 sequences, H=128 heads, Q=1 new token, Dn=128, Dr=64,
Vd=128, Ckv=512, 4096 cached tokens per sequence in a contiguous
[B, Lk, 512+64] cache; seeded synthetic inputs (seed 1).

One step = the whole path: mla_cache_append (the new token's row),
mla_absorb_q, mla_decode_attn (token-split attention + log-sum-exp merge) and
mla_up_proj_v. Inputs are resident in HBM before timing starts; every step
reads a different one of several cache copies so that the 256 MB Infinity
Cache cannot serve the 151 MB cache from the previous step.

Prints one JSON line (see the keys below). --gpus N with N > 1 is refused:
this build runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0       # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
WORKLOAD = "dsv3_bf16"
METRIC = "MLA decode tokens/s + KV GB/s & MFMA TFLOP/s as % of MI355X roofline"
ATTN_KERNEL_SOURCES = ("attn_mfma.hip", "device_common.h", "internal.h")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in ATTN_KERNEL_SOURCES:
        with open(os.path.join(ROOT, "mla_latent_kv_08_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(bytes_alg: float):
    """HBM bytes per launch measured with rocprofv3 counters, if taken on this kernel source."""
    path = os.path.join(ROOT, "profiles", "attn_decode_dsv3_bf16_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


COPY_BYTES = 256 << 20  # size of the calibration copy (read and written once each)
TRAFFIC_PATH = os.path.join(ROOT, "profiles", "attn_decode_dsv3_bf16_traffic.json")


def _counter_values(run_dir: str, counter: str) -> dict:
    """Values (KiB) of one rocprofv3 counter per kernel name, one per dispatch."""
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    per = {}
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                key = (r["Kernel_Name"], r["Dispatch_Id"])
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    values = {}
    for (name, _), v in per.items():
        values.setdefault(name, []).append(v)
    return values


def summarize_counters(fetch_dir: str, write_dir: str):
    """Scale FETCH_SIZE / WRITE_SIZE of the attention call by what the same counters
    read for the calibration copy, and store the HBM bytes per launch."""
    fetch = _counter_values(fetch_dir, "FETCH_SIZE")
    write = _counter_values(write_dir, "WRITE_SIZE")

    def values(d, key):
        hits = [v for k, vs in d.items() if key in k for v in vs]
        if not hits:
            raise SystemExit(f"no dispatch matching {key!r}")
        return hits

    def pick(d, key):  # mean over the dispatches of a kernel
        v = values(d, key)
        return sum(v) / len(v)

    # The calibration copy is the largest copy dispatch of the run (smaller
    # ones upload the inputs).
    copy_kib = COPY_BYTES / 1024.0
    f_factor = copy_kib / max(values(fetch, "copyBuffer"))
    w_factor = copy_kib / max(values(write, "copyBuffer"))
    attn_f = pick(fetch, "attn_mfma_kernel<false>") * 1024.0 * f_factor
    attn_w = pick(write, "attn_mfma_kernel<false>") * 1024.0 * w_factor
    comb_f = pick(fetch, "attn_combine_kernel") * 1024.0 * f_factor
    comb_w = pick(write, "attn_combine_kernel") * 1024.0 * w_factor
    rec = {
        "kernel_source_hash": kernel_source_hash(),
        "hbm_bytes_per_launch": attn_f + attn_w + comb_f + comb_w,
        "attention_kernel": {"fetch_bytes": attn_f, "write_bytes": attn_w},
        "merge_kernel": {"fetch_bytes": comb_f, "write_bytes": comb_w},
        "fetch_scale": f_factor, "write_scale": w_factor,
        "calibration": f"one {COPY_BYTES} B device-to-device copy in the same process",
    }
    with open(TRAFFIC_PATH, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec))


def cpu_baseline(w, inp, budget_s: float = 15.0):
    """Time the fp64 oracle (as it stands) on a bounded sample of the same workload."""
    from oracle import mla_ref
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    done = 0
    t0 = time.perf_counter()
    while done < w.B:
        b = done
        mla_ref.decode_nonabsorbed(inp.q_nope[b:b + 1], inp.q_pe[b:b + 1], [inp.seq_latent(b)],
                                   [inp.seq_rope(b)], inp.wkv_b, [int(inp.seq_lens[b])],
                                   w.softmax_scale)
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": done * w.Q / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{done} of {w.B} sequences (all {w.H} heads, {int(inp.seq_lens[0])} cached tokens "
                      f"each), fp64 non-absorbed oracle, {dt:.1f} s wall"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--copies", type=int, default=4, help="rotated cache copies (>= 3 defeats the MALL)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workgroups", type=int, default=0)
    ap.add_argument("--graph", action="store_true",
                    help="replay each step (and the timed attention calls) from captured HIP "
                         "graphs instead of launching the calls one by one")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run one device-to-device copy of COPY_BYTES (counter calibration)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc outputs (FETCH_SIZE, WRITE_SIZE) of a "
                         "--calibrate-copy run into the traffic record under profiles/, then exit")
    args = ap.parse_args()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the multi-GPU form of this "
              "path is a design note, not part of this build.", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as W
    from mla_latent_kv_08_amd import ops

    w = W.WORKLOADS[WORKLOAD]
    inp = W.generate(w)
    pl = W.place(inp)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    B, H, Q = w.B, w.H, w.Q
    phys = W.combined_rows(inp.latent, inp.rope, pl, fill=0.0)
    caches = []
    bufs = []
    for _ in range(max(1, args.copies)):
        buf = phys.to(dev)
        bufs.append(buf)
        caches.append(ops.LatentCache.combined(buf, w.Ckv, pl.capacity))
    del phys
    q_nope = inp.q_nope.to(dev)
    q_pe = inp.q_pe.to(dev)
    wkv_b = inp.wkv_b.to(dev)
    seq_lens = inp.seq_lens.to(dev)
    max_len = int(inp.seq_lens.max())
    # The newest token of every sequence, written again by the append each step.
    last = (inp.seq_offsets[1:] - 1)
    c_new = inp.latent[last].reshape(B, 1, w.Ckv).contiguous().to(dev)
    r_new = inp.rope[last].reshape(B, 1, w.Dr).contiguous().to(dev)
    q_lat = torch.empty(B, H, Q, w.Ckv, dtype=torch.bfloat16, device=dev)
    x = torch.empty_like(q_lat)
    lse = torch.empty(B, H, Q, dtype=torch.float32, device=dev)
    out = torch.empty(B, H, Q, w.Vd, dtype=torch.bfloat16, device=dev)
    ws_bytes = ops.mla_decode_workspace_size(B, H, Q, ops.MLA_BF16, max_len, args.workgroups)
    workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    if args.calibrate_copy:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    ncopy = len(caches)

    def attend(c, st):
        ops.mla_decode_attn(q_lat, q_pe, caches[c], seq_lens, max_len, w.softmax_scale, x, lse,
                            workspace=workspace, workgroups=args.workgroups, stream=st)

    def step_calls(c, st):
        ops.mla_cache_append(c_new, r_new, caches[c], seq_lens, stream=st)
        ops.mla_absorb_q(q_nope, wkv_b, q_lat, stream=st)
        attend(c, st)
        ops.mla_up_proj_v(x, wkv_b, out, stream=st)

    # A decode step is the same four library calls every time. By default they
    # are launched one by one; with --graph they are captured once per cache
    # copy into HIP graphs and replayed (measured no faster on this stack: a
    # graph launch costs about what the separate launches do).
    step_graphs, attn_graphs = [], []
    if args.graph:
        for c in range(ncopy):  # first calls run eagerly (one-time library set-up)
            step_calls(c, stream)
        torch.cuda.synchronize()
        for c in range(ncopy):
            gs, ga = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
            with torch.cuda.graph(gs):
                step_calls(c, torch.cuda.current_stream())
            with torch.cuda.graph(ga):
                attend(c, torch.cuda.current_stream())
            step_graphs.append(gs)
            attn_graphs.append(ga)
        torch.cuda.synchronize()

    def step(i):
        if not args.graph:
            step_calls(i % ncopy, stream)
        else:
            step_graphs[i % ncopy].replay()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for i in range(args.steps):
        step(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_total = t_start.elapsed_time(t_end)
    ms_step = ms_total / args.steps

    # The attention call alone (attention kernel + merge), over the cache
    # copies in turn, on its stream: one pair of HIP events around `steps`
    # back-to-back calls gives the average (the host enqueues ahead, so no
    # launch latency enters); a pair around each call of a second pass gives
    # the spread (those include the per-call launch gap when the GPU waits
    # for the host).
    def attn_call(i):
        if not args.graph:
            attend(i % ncopy, stream)
        else:
            attn_graphs[i % ncopy].replay()

    attn_call(0)
    torch.cuda.synchronize()
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    h0 = time.perf_counter()
    a0.record(stream)
    for i in range(args.steps):
        attn_call(i)
    a1.record(stream)
    host_us = (time.perf_counter() - h0) / args.steps * 1e6
    torch.cuda.synchronize()
    attn_avg_ms = a0.elapsed_time(a1) / args.steps
    ev_attn = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
    for i in range(args.steps):
        ev_attn[i][0].record(stream)
        attn_call(i)
        ev_attn[i][1].record(stream)
    torch.cuda.synchronize()
    attn_ms = sorted(a.elapsed_time(b) for a, b in ev_attn)
    pct = lambda p: attn_ms[min(len(attn_ms) - 1, int(p * len(attn_ms)))]  # noqa: E731
    if not torch.isfinite(out.float()).all():
        print("non-finite output", file=sys.stderr)
        sys.exit(3)

    lens = [int(v) for v in inp.seq_lens]
    cache_bytes = sum(lens) * (w.Ckv + w.Dr) * 2
    io_bytes = B * H * Q * (w.Ckv * 2 + w.Dr * 2 + w.Ckv * 2 + 4)
    bytes_alg = cache_bytes + io_bytes
    flops = sum(H * min(L, L - Q + q + 1) * 2 * (2 * w.Ckv + w.Dr) for L in lens for q in range(Q))
    attn_s = attn_avg_ms / 1e3
    achieved_gbps = bytes_alg / attn_s / 1e9
    tflops = flops / attn_s / 1e12
    traffic = load_traffic(bytes_alg)
    cpu = None if args.no_cpu_baseline else cpu_baseline(w, inp)
    rec = {
        "metric": METRIC,
        "value": B * Q / (ms_step / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "DeepSeek-V3-shaped MLA decode, one layer: B=32, H=128, Q=1, Dn=128, "
                               "Dr=64, Vd=128, Ckv=512, Lk=4096, contiguous [B,Lk,576] bf16 cache",
                   "global_batch": B, "seq_len": max_len, "parallelism": "none (1 GPU)",
                   "cache_copies": len(caches), "launch": "hip graph replay" if args.graph else "eager"},
        "roofline": {"bound": "hbm", "achieved": achieved_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved_gbps / HBM_PEAK_GBPS,
                     "traffic": traffic},
        "attn": {"kernel": "mla_decode_attn (token-split attention + merge)",
                 "avg_ms": attn_avg_ms, "host_us_per_call": host_us,
                 "per_call_p50_ms": pct(0.5), "per_call_p95_ms": pct(0.95), "per_call_p99_ms": pct(0.99),
                 "alg_bytes": bytes_alg, "alg_flops": flops, "kv_GBps": cache_bytes / attn_s / 1e9,
                 "mfma_TFLOPs": tflops, "mfma_frac": tflops / MFMA_BF16_PEAK_TFLOPS,
                 "kernel_source_hash": kernel_source_hash()},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
