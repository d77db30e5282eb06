#!/usr/bin/env python3
"""Benchmark of one absorbed-MLA decode step on one MI355X.

Workload: the DeepSeek-V3-shaped single-layer decode, bf16 with fp32
accumulation: B=32 sequences, H=128 heads, Q=1 new token, Dn=128, Dr=64,
Vd=128, Ckv=512, 4096 cached tokens per sequence in a contiguous
[B, Lk, 512+64] cache; seeded synthetic inputs (seed 1).

One step = the whole path: the cache append of the new token's row and the
query absorption (mla_append_absorb: mla_cache_append and mla_absorb_q in one
launch; --separate-append calls the two), then attention and the value
up-projection (mla_decode_attn_up: token-split attention, then the
log-sum-exp merge and W_UV in one kernel; --separate-up calls mla_decode_attn
and mla_up_proj_v). Inputs are resident in HBM before timing starts; every step
reads a different one of several cache copies so that the 256 MB Infinity
Cache cannot serve the 151 MB cache from the previous step.

Prints one JSON line (see the keys below). --gpus N with N > 1 is refused:
the benchmark measures one GPU's share.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
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


def summarize_counters(fetch_dir: str, write_dir: str, workload: str = WORKLOAD):
    """Scale FETCH_SIZE / WRITE_SIZE of the attention call by what the same counters
    read for the calibration copy, and store the HBM bytes per launch (per workload:
    profiles/attn_decode_<workload>_traffic.json)."""
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
    # the attention kernel of the workload's latent dtype (first template argument: FP4)
    key = "attn_mfma_kernel<true" if workload == "mtp_fp4" else "attn_mfma_kernel<false"
    attn_f = pick(fetch, key) * 1024.0 * f_factor
    attn_w = pick(write, key) * 1024.0 * w_factor
    comb_f = pick(fetch, "attn_combine_kernel") * 1024.0 * f_factor
    comb_w = pick(write, "attn_combine_kernel") * 1024.0 * w_factor
    rec = {
        "workload": workload,
        "kernel_source_hash": kernel_source_hash(),
        "hbm_bytes_per_launch": attn_f + attn_w + comb_f + comb_w,
        "attention_kernel": {"fetch_bytes": attn_f, "write_bytes": attn_w},
        "merge_kernel": {"fetch_bytes": comb_f, "write_bytes": comb_w},
        "fetch_scale": f_factor, "write_scale": w_factor,
        "calibration": f"one {COPY_BYTES} B device-to-device copy in the same process",
    }
    path = TRAFFIC_PATH if workload == WORKLOAD else os.path.join(ROOT, "profiles",
                                                                 f"attn_decode_{workload}_traffic.json")
    with open(path, "w") as fh:
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
            "cpu": cpu_model(),
            "sample": f"{done} of {w.B} sequences (all {w.H} heads, {int(inp.seq_lens[0])} cached tokens "
                      f"each), fp64 non-absorbed oracle, {dt:.1f} s wall"}



def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cache_row_bytes(w) -> int:
    """Bytes of one cached token: [latent | rope] in the storage dtype, or FP4 codes + scales + bf16 rope."""
    if w.dtype == "fp4":
        return w.Ckv // 2 + w.Ckv // 16 + 2 * w.Dr
    return (w.Ckv + w.Dr) * (4 if w.dtype == "f32" else 2)


def attn_cost(w, lens):
    """Algorithmic bytes and flops of one attention call: every visible cache row read once,
    q_lat / q_pe read and x / lse written once; 2*(Ckv + Dr + Ckv) flop per (head, query,
    visible token), with query q of Q seeing the first len - Q + q + 1 tokens."""
    es = 4 if w.dtype == "f32" else 2
    cache_bytes = sum(lens) * cache_row_bytes(w)
    io_bytes = w.B * w.H * w.Q * (w.Ckv * es + w.Dr * es + w.Ckv * es + 4)
    flops = sum(w.H * max(0, min(L, L - w.Q + q + 1)) * 2 * (2 * w.Ckv + w.Dr)
                for L in lens for q in range(w.Q))
    return cache_bytes, io_bytes, flops


def time_back_to_back(fn, n: int, stream) -> float:
    """Average ms of fn(i) over n calls enqueued back to back between one pair of HIP events."""
    import torch
    fn(0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(n):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def setup_attn_case(w, dev, copies: int, lo: bool = True):
    """Seeded inputs of workload w on the GPU: q_lat from mla_absorb_q, the cache in the
    workload's layout (paged ones with NaN in every unused row), outputs and workspace."""
    import torch
    import workloads as W
    from mla_latent_kv_08_amd import ops
    inp = W.generate(w)
    pl = W.place(inp)
    pt = pl.page_table.to(dev) if pl.page_table is not None else None
    lens = [int(v) for v in inp.seq_lens]
    seq_lens = inp.seq_lens.to(dev)
    max_len = max(lens)
    caches = []
    if w.dtype != "fp4":
        phys = W.combined_rows(inp.latent, inp.rope, pl, fill=float("nan"))
        for _ in range(copies):
            caches.append(ops.LatentCache.combined(phys.to(dev), w.Ckv, pl.capacity, page_table=pt))
        del phys
    else:
        # FP4 rows are written by the library's own append (fp32 latent in, codes + scales out).
        row = ops.LatentCache.fp4_row_bytes(w.Ckv, w.Dr)
        buf = torch.full((pl.n_rows, row), 0xFF, dtype=torch.uint8, device=dev)
        first = ops.LatentCache.fp4(buf, w.Ckv, pl.capacity, page_table=pt)
        c = torch.zeros(w.B, max_len, w.Ckv, dtype=torch.float32)
        r = torch.zeros(w.B, max_len, w.Dr, dtype=inp.rope.dtype)
        for b, L in enumerate(lens):
            if L:
                c[b, max_len - L:] = inp.seq_latent(b)
                r[b, max_len - L:] = inp.seq_rope(b)
        c, r = c.to(dev), r.to(dev)
        ops.mla_cache_append(c, r, first, seq_lens)
        caches.append(first)
        # Further copies written by the same append (a device-to-device copy of
        # the cache would be mistaken for the counter-calibration copy).
        for _ in range(copies - 1):
            more = ops.LatentCache.fp4(torch.full_like(buf, 0xFF), w.Ckv, pl.capacity, page_table=pt)
            ops.mla_cache_append(c, r, more, seq_lens)
            caches.append(more)
        del c, r
    dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    q_lat = torch.empty(w.B, w.H, w.Q, w.Ckv, dtype=dt, device=dev)
    q_lo = torch.empty_like(q_lat) if (lo and w.dtype != "f32") else None
    ops.mla_absorb_q(inp.q_nope.to(dev), inp.wkv_b.to(dev), q_lat, q_lat_lo=q_lo)
    code = ops.MLA_F32 if w.dtype == "f32" else ops.MLA_BF16
    ws = ops.mla_decode_workspace_size(w.B, w.H, w.Q, code, max_len)
    torch.cuda.synchronize()
    return {"lens": lens, "caches": caches, "seq_lens": seq_lens, "max_len": max_len, "inputs_sha256": inp.sha256(),
            "q_lat": q_lat, "q_lat_lo": q_lo, "q_pe": inp.q_pe.to(dev), "x": torch.empty_like(q_lat),
            "lse": torch.empty(w.B, w.H, w.Q, dtype=torch.float32, device=dev),
            "workspace": torch.empty(max(ws, 16), dtype=torch.uint8, device=dev)}


# The other workloads of the method's measurement table: the attention call
# alone, with its own roofline. Caches of 436 MB and more exceed the 256 MB
# Infinity Cache; the FP4 one is still rotated over two copies.
OTHER_WORKLOADS = {"tiny_f32": 1, "ragged_paged_bf16": 1, "long_splitkv_bf16": 1, "mtp_fp4": 2}


def measure_other_workloads(dev, stream, reps: int, lo=None, names=None) -> dict:
    """The attention call alone on each named workload; `lo` None takes the workload's own q_lat_lo setting."""
    import torch
    import workloads as W
    from mla_latent_kv_08_amd import ops
    out = {}
    for name, copies in OTHER_WORKLOADS.items():
        if names is not None and name not in names:
            continue
        w = W.WORKLOADS[name]
        print(f"bench: workload {name}", file=sys.stderr, flush=True)
        case = setup_attn_case(w, dev, copies, w.q_lat_lo if lo is None else lo)
        inputs_sha = case["inputs_sha256"]

        def call(i, case=case, w=w):
            ops.mla_decode_attn(case["q_lat"], case["q_pe"], case["caches"][i % len(case["caches"])],
                                case["seq_lens"], case["max_len"], w.softmax_scale, case["x"],
                                case["lse"], workspace=case["workspace"], q_lat_lo=case["q_lat_lo"],
                                stream=stream)

        ms = time_back_to_back(call, reps, stream)
        if not torch.isfinite(case["x"].float()).all():
            raise SystemExit(f"{name}: non-finite attention output")
        cache_b, io_b, flops = attn_cost(w, case["lens"])
        t = ms / 1e3
        t_hbm = (cache_b + io_b) / (HBM_PEAK_GBPS * 1e9)
        t_mfma = flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
        rec = {"attn_avg_ms": ms, "B": w.B, "H": w.H, "Q": w.Q, "tokens": sum(case["lens"]),
               "q_lat_lo": case["q_lat_lo"] is not None, "inputs_sha256": inputs_sha,
               "cache": ("paged 64-token pages" if w.paged else "contiguous") + f", {w.dtype} latent",
               "cache_bytes": cache_b, "io_bytes": io_b, "alg_flops": flops,
               "kv_GBps": cache_b / t / 1e9, "mfma_TFLOPs": flops / t / 1e12}
        if w.dtype == "f32":
            rec["bound"] = "launch latency"
        else:
            rec["bound"] = "hbm" if t_hbm >= t_mfma else "mfma"
            rec["t_roofline_us"] = max(t_hbm, t_mfma) * 1e6
            rec["roofline_frac"] = max(t_hbm, t_mfma) / t
        out[name] = rec
        del case
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return out


def measure_prefill(dev, stream, reps: int) -> dict:
    """mla_prefill_attn (non-absorbed) at DeepSeek-V3 dimensions (H=128, Dn=Vd=128, Dr=64, Ckv=512, bf16):
    chunked prefill, 64 new tokens on a 4096-token cache, B=8 (fused path: every chunk's K and V formed once,
    in LDS); and a full prefill of 4096 tokens, B=1, on the two-kernel path (K and V formed once into a
    workspace, then flash attention), with the fused path timed beside it. alg_flops counts each head's K and
    V made once per token plus the causal score and value products; exec_flops what the path issues (the
    fused path forms the chunks again for every 64-query tile; the two-kernel path forms them once and its
    attention runs whole 32-token tiles, masked). Each case is timed after an untimed pass of the same calls."""
    import torch
    from mla_latent_kv_08_amd import ops
    out = {}
    for name, B, Q, L, n, two in (("chunked_q64_lk4096_b8", 8, 64, 4096, reps, False),
                                  ("full_q4096_b1", 1, 4096, 4096, 10, True),
                                  ("full_q4096_b1_fused", 1, 4096, 4096, 3, False)):
        print(f"bench: prefill {name}", file=sys.stderr, flush=True)
        H, C, R, D = 128, 512, 64, 128
        g = torch.Generator().manual_seed(11)
        buf = torch.randn(B * L, C + R, generator=g).to(torch.bfloat16).to(dev)
        cache = ops.LatentCache.combined(buf, C, L)
        sl = torch.full((B,), L, dtype=torch.int32, device=dev)
        qn = torch.randn(B, H, Q, D, generator=g).to(torch.bfloat16).to(dev)
        qp = torch.randn(B, H, Q, R, generator=g).to(torch.bfloat16).to(dev)
        wkv = (torch.randn(H, 2 * D, C, generator=g) / math.sqrt(C)).to(torch.bfloat16).to(dev)
        o = torch.empty(B, H, Q, D, dtype=torch.bfloat16, device=dev)
        lse = torch.empty(B, H, Q, dtype=torch.float32, device=dev)
        scale = 1.0 / math.sqrt(D + R)
        ws_bytes = ops.mla_prefill_workspace_size(B, H, Q, L) if two else 0
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if two else None
        call = lambda i: ops.mla_prefill_attn(qn, qp, cache, sl, wkv, scale, o, lse, workspace=ws, stream=stream)
        time_back_to_back(call, n, stream)  # untimed pass: the clocks ramp up during the first calls
        ms = time_back_to_back(call, n, stream)
        if not torch.isfinite(o.float()).all():
            raise SystemExit(f"prefill {name}: non-finite output")
        pairs = sum(L - Q + q + 1 for q in range(Q))
        alg = B * H * (L * 2 * D * C * 2 + pairs * (D + R + D) * 2)
        qt = 128 if two else 64
        tiles = 0
        for q0 in range(0, Q, qt):
            last = L - Q + min(q0 + qt - 1, Q - 1)
            tiles += last // 32 + 1
        attn = B * H * tiles * qt * 32 * (D + R + D) * 2
        execf = attn + (B * H * ((L + 31) // 32) * 32 * 2 * D * C * 2 if two else B * H * tiles * 32 * 2 * D * C * 2)
        t = ms / 1e3
        out[name] = {"B": B, "H": H, "Q": Q, "Lk": L, "ms": ms,
                     "path": "two kernels (K, V formed once into a workspace; flash attention)" if two
                     else "fused (K, V formed per 64-query tile in LDS)",
                     "workspace_bytes": ws_bytes, "alg_flops": alg, "exec_flops": execf,
                     "alg_TFLOPs": alg / t / 1e12, "exec_TFLOPs": execf / t / 1e12,
                     "mfma_frac_alg": alg / t / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                     "mfma_frac_exec": execf / t / 1e12 / MFMA_BF16_PEAK_TFLOPS}
        del buf, cache, qn, qp, wkv, o, lse, ws
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return out


def measure_v4_form(dev, stream, reps: int) -> dict:
    """The DeepSeek-V4.1-Flash form at the headline's cache size: 64 query heads over one latent whose last
    64 dims carry the rotation, B=32, Lk=4096, Q=1, on the form's own rows (no RoPE section): bf16 1024-byte
    rows (3 rotated copies, 403 MB) and FP4 288-byte rows of codes and scales (8 copies, 302 MB), both past
    the MALL; and, for comparison, DeepSeek-V3 rows with a zero 64-dim RoPE slot (1152 B, 2 copies). Each
    attention call alone, and the chain on the bf16 own rows, back to back: mla_rope_append in latent-tail
    mode (the step's new token and its 64 query rows), mla_decode_attn, mla_sink_inverse_rope (sink
    column, x's tail turned back), mla_grouped_out_proj (8 groups x 1024, random bf16 W_O, 67 MB)."""
    import torch
    import workloads as W
    from mla_latent_kv_08_amd import ops
    print("bench: workload v4_form_bf16", file=sys.stderr, flush=True)
    B, H, Q, L, C, R = 32, 64, 1, 4096, 512, 64
    g = torch.Generator().manual_seed(5)
    hist = torch.randn(B, L, C, generator=g).to(torch.bfloat16).to(dev)
    sl = torch.full((B,), L, dtype=torch.int32, device=dev)
    table = W.rope_table(L, R).to(dev)

    def fill(cache):
        ops.mla_rope_append(hist, None, cache, sl, table, latent_tail=True, stream=stream)
        return cache
    own = [fill(ops.LatentCache.latent_only(torch.zeros(B * L, C, dtype=torch.bfloat16, device=dev), C, L))
           for _ in range(3)]
    fp4_row = ops.LatentCache.fp4_row_bytes(C, 0)
    fp4 = [fill(ops.LatentCache.fp4(torch.zeros(B * L, fp4_row, dtype=torch.uint8, device=dev), C, L, rope=False))
           for _ in range(8)]
    v3rows = [fill(ops.LatentCache.combined(torch.zeros(B * L, C + R, dtype=torch.bfloat16, device=dev), C, L))
              for _ in range(2)]
    new = hist[:, L - Q:].contiguous()
    del hist
    q = torch.randn(B, H, Q, C, generator=g).to(torch.bfloat16).to(dev)
    zero_pe = torch.zeros(B, H, Q, R, dtype=torch.bfloat16, device=dev)
    sinks = torch.randn(H, generator=g).to(dev)
    x = torch.empty(B, H, Q, C, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(B, H, Q, dtype=torch.float32, device=dev)
    ws = torch.empty(max(16, ops.mla_decode_workspace_size(B, H, Q, ops.MLA_BF16, L)), dtype=torch.uint8, device=dev)
    scale = 1.0 / math.sqrt(C)

    def rope(i):
        ops.mla_rope_append(new, None, own[i % len(own)], sl, table, q_pe=q, latent_tail=True, stream=stream)

    def attn(i):
        ops.mla_decode_attn(q, None, own[i % len(own)], sl, L, scale, x, lse, workspace=ws, stream=stream)

    def attn_fp4(i):
        ops.mla_decode_attn(q, None, fp4[i % len(fp4)], sl, L, scale, x, lse, workspace=ws, stream=stream)

    def attn_v3rows(i):
        ops.mla_decode_attn(q, zero_pe, v3rows[i % len(v3rows)], sl, L, scale, x, lse, workspace=ws, stream=stream)

    def sink(i):
        ops.mla_sink_inverse_rope(x, lse, sl, sinks, table, stream=stream)

    G, N = 8, 1024
    w_o = (torch.randn(G, N, (H // G) * C, generator=g) / 64.0).to(torch.bfloat16).to(dev)
    hidden = torch.empty(B, Q, G * N, dtype=torch.bfloat16, device=dev)

    def out_proj(i):
        ops.mla_grouped_out_proj(x, w_o, hidden, stream=stream)

    def chain(i):
        rope(i)
        attn(i)
        sink(i)
        out_proj(i)

    rec = {"B": B, "H": H, "Q": Q, "Lk": L,
           "cache": "contiguous, the form's own rows: bf16 latent (tail rotated), no RoPE section, 1024 B"}
    for name, fn in (("attn_fp4_ms", attn_fp4), ("attn_v3_rows_ms", attn_v3rows), ("rope_append_ms", rope),
                     ("attn_ms", attn), ("sink_inverse_rope_ms", sink), ("grouped_out_proj_ms", out_proj),
                     ("chain_ms", chain)):
        rec[name] = time_back_to_back(fn, reps, stream)
    if not torch.isfinite(x.float()).all():
        raise SystemExit("v4_form_bf16: non-finite output")
    io_b = B * H * Q * (C * 2 + C * 2 + 4)
    flops = B * H * Q * L * 2 * (C + C)
    mfma_t = flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)

    def roof(cache_b, ms):
        t = ms / 1e3
        t_hbm = (cache_b + io_b) / (HBM_PEAK_GBPS * 1e9)
        bound = "hbm" if t_hbm >= mfma_t else "mfma"
        return {"cache_bytes": cache_b, "io_bytes": io_b, "alg_flops": flops, "ms": ms,
                "kv_GBps": cache_b / t / 1e9, "bound": bound, "t_roofline_us": max(t_hbm, mfma_t) * 1e6,
                "roofline_frac": max(t_hbm, mfma_t) / t}
    rec["own_rows_bf16"] = roof(B * L * C * 2, rec["attn_ms"])
    rec["own_rows_fp4"] = roof(B * L * fp4_row, rec["attn_fp4_ms"])
    # V3 rows: the zero RoPE slot is read but carries nothing, so the fraction counts the latent bytes only.
    rec["v3_rows_zero_rope_slot"] = roof(B * L * C * 2, rec["attn_v3_rows_ms"])
    rec.update({"bound": "hbm", "t_roofline_us": rec["own_rows_bf16"]["t_roofline_us"],
                "roofline_frac": rec["own_rows_bf16"]["roofline_frac"],
                "tokens_per_s": B * Q / (rec["chain_ms"] / 1e3),
                "grouped_out_proj": {"groups": G, "group_out": N, "weight_bytes": G * N * (H // G) * C * 2,
                                     "GBps": G * N * (H // G) * C * 2 / (rec["grouped_out_proj_ms"] / 1e3) / 1e9}})
    del own, fp4, v3rows, x, q, w_o, hidden
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


def copy_gbps(dev, stream, nbytes: int = 1 << 30, reps: int = 10) -> float:
    """Device-to-device copy rate (bytes read + written per second) as context for the roofline."""
    import torch
    src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    ms = time_back_to_back(lambda i: dst.copy_(src), reps, stream)
    del src, dst
    return 2 * nbytes / (ms / 1e3) / 1e9


def gpu_context(dev) -> dict:
    import subprocess
    import torch
    info = {"device": torch.cuda.get_device_name(dev), "hip": torch.version.hip, "torch": torch.__version__}
    try:
        r = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=30)
        info["clocks"] = [ln.split(":", 2)[-1].strip() for ln in r.stdout.splitlines()
                          if "sclk" in ln or "mclk" in ln or "fclk" in ln][:6]
    except Exception as e:  # pragma: no cover - tool missing or slow
        info["clocks"] = f"unavailable ({type(e).__name__})"
    return info


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--copies", type=int, default=4, help="rotated cache copies (>= 3 defeats the MALL)")
    ap.add_argument("--settle-s", type=float, default=0.25,
                    help="seconds of untimed steps before the warmup steps, so that the timed steps run at "
                         "steady clocks (0: none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workgroups", type=int, default=0)
    ap.add_argument("--lo", choices=("auto", "on", "off"), default="auto",
                    help="pass the query's low part q_lat_lo to the scores: auto = as each workload is "
                         "configured (spiked long context and FP4: on; headline and ragged: off)")
    ap.add_argument("--graph", action="store_true",
                    help="replay each step (and the timed attention calls) from captured HIP "
                         "graphs instead of launching the calls one by one")
    ap.add_argument("--separate-append", action="store_true",
                    help="call mla_cache_append and mla_absorb_q separately instead of mla_append_absorb")
    ap.add_argument("--separate-up", action="store_true",
                    help="call mla_decode_attn and mla_up_proj_v separately instead of mla_decode_attn_up")
    ap.add_argument("--headline-only", action="store_true",
                    help="skip the other workloads (ragged paged, long context, FP4 MTP, tiny fp32) "
                         "and the context figures (copy rate, clocks)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only time mla_prefill_attn (chunked and full prefill) and print that record")
    ap.add_argument("--workload", choices=sorted(OTHER_WORKLOADS) + ["v4_form_bf16"],
                    help="only time the attention call of this workload (--steps back-to-back calls) and "
                         "print its record: for profiling runs")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run one device-to-device copy of COPY_BYTES (counter calibration)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc outputs (FETCH_SIZE, WRITE_SIZE) of a "
                         "--calibrate-copy run (of --workload, else the headline) into the traffic "
                         "record under profiles/, then exit")
    args = ap.parse_args()
    lo_flag = {"auto": None, "on": True, "off": False}[args.lo]
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, workload=args.workload or WORKLOAD)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the library has no "
              "multi-GPU path; it measures one GPU's share of a sharded decode.", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as W
    from mla_latent_kv_08_amd import ops

    dev = torch.device("cuda", 0)
    if args.workload == "v4_form_bf16":
        torch.cuda.set_device(dev)
        rec = measure_v4_form(dev, torch.cuda.current_stream(dev), max(1, args.steps))
        print(json.dumps({"workload": args.workload, **rec}))
        return
    if args.workload:
        torch.cuda.set_device(dev)
        if args.calibrate_copy:
            src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
            dst = torch.empty_like(src)
            torch.cuda.synchronize()
            dst.copy_(src)
            torch.cuda.synchronize()
            del src, dst
        rec = measure_other_workloads(dev, torch.cuda.current_stream(dev), max(1, args.steps), lo=lo_flag,
                                      names=(args.workload,))
        print(json.dumps({"workload": args.workload, **rec[args.workload]}))
        return
    w = W.WORKLOADS[WORKLOAD]
    inp = W.generate(w)
    pl = W.place(inp)
    if args.prefill_only:
        print(json.dumps({"prefill_bf16": measure_prefill(dev, torch.cuda.current_stream(dev), 20)}))
        return
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
    use_lo = w.q_lat_lo if lo_flag is None else lo_flag
    q_lo = torch.empty_like(q_lat) if use_lo else None
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
                            workspace=workspace, workgroups=args.workgroups, q_lat_lo=q_lo, stream=st)

    def append_absorb(c, st):
        if args.separate_append:
            ops.mla_cache_append(c_new, r_new, caches[c], seq_lens, stream=st)
            ops.mla_absorb_q(q_nope, wkv_b, q_lat, q_lat_lo=q_lo, stream=st)
        else:
            ops.mla_append_absorb(c_new, r_new, caches[c], seq_lens, q_nope, wkv_b, q_lat, q_lat_lo=q_lo, stream=st)

    def up_proj(c, st):
        ops.mla_up_proj_v(x, wkv_b, out, stream=st)

    def attend_up(c, st):
        ops.mla_decode_attn_up(q_lat, q_pe, caches[c], seq_lens, max_len, w.softmax_scale, x, lse, wkv_b, out,
                               workspace=workspace, workgroups=args.workgroups, q_lat_lo=q_lo, stream=st)

    if args.separate_up:
        parts = (("append_absorb", append_absorb), ("attn", attend), ("up_proj", up_proj))
    else:
        parts = (("append_absorb", append_absorb), ("attn_up", attend_up))

    def step_calls(c, st):
        for _, fn in parts:
            fn(c, st)

    # A decode step is the same library calls every time. By default they
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

    # Clock settling: the GPU's clocks ramp up over the first tens of
    # milliseconds of sustained load, and a few warmup steps take well under a
    # millisecond. A fixed period of the same step, untimed and before the
    # warmup steps, lets the timed steps run at steady clocks whatever the
    # warmup count.
    settle_steps = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < args.settle_s:
        for _ in range(64):
            step(settle_steps)
            settle_steps += 1
        torch.cuda.synchronize()
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

    # Each call's share of a step: a second eager pass with an event between
    # consecutive calls (so each call sees the cache state of a real step).
    names = tuple(k for k, _ in parts)
    in_step = {k: 0.0 for k in names}
    if not args.graph:
        evs = []
        for i in range(args.steps):
            c = i % ncopy
            e = [torch.cuda.Event(enable_timing=True) for _ in range(len(parts) + 1)]
            e[0].record(stream)
            for j, (_, fn) in enumerate(parts):
                fn(c, stream)
                e[j + 1].record(stream)
            evs.append(e)
        torch.cuda.synchronize()
        for e in evs:
            for j, k in enumerate(names):
                in_step[k] += e[j].elapsed_time(e[j + 1]) / args.steps

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
    # (Timed after the attention passes: 400 short launches before them would
    # leave the clocks low for the batched attention timing.)
    # The append with the rotary embedding on the way in (mla_rope_append:
    # the new RoPE keys turned to their positions and stored, the step's 128
    # heads of q_pe turned in place, one pass) against the plain append
    # (mla_cache_append); each as `steps` back-to-back calls between one pair
    # of HIP events. The cos/sin table is input data (the usual 10000-base
    # schedule, fp32); the rotation runs on a copy of q_pe.
    rope_table = W.rope_table(max_len + 1, w.Dr).to(dev)
    q_pe_rot = q_pe.clone()

    rope_ms = time_back_to_back(lambda i: ops.mla_rope_append(c_new, r_new, caches[i % ncopy], seq_lens, rope_table,
                                                              q_pe=q_pe_rot, stream=stream), args.steps, stream)
    plain_append_ms = time_back_to_back(lambda i: ops.mla_cache_append(c_new, r_new, caches[i % ncopy], seq_lens,
                                                                       stream=stream), args.steps, stream)

    if not torch.isfinite(out.float()).all():
        print("non-finite output", file=sys.stderr)
        sys.exit(3)

    lens = [int(v) for v in inp.seq_lens]
    cache_bytes, io_bytes, flops = attn_cost(w, lens)
    bytes_alg = cache_bytes + io_bytes
    # The projections against their own weight-bandwidth roofline (bf16 weights
    # read once, activations in and out once).
    wt = H * w.Dn * w.Ckv * 2
    proj_bytes = {"append_absorb": wt + B * H * Q * (w.Dn + (2 if use_lo else 1) * w.Ckv) * 2
                  + 2 * B * Q * (w.Ckv + w.Dr) * 2,
                  "up_proj": H * w.Vd * w.Ckv * 2 + B * H * Q * (w.Ckv + w.Vd) * 2}
    attn_s = attn_avg_ms / 1e3
    achieved_gbps = bytes_alg / attn_s / 1e9
    tflops = flops / attn_s / 1e12
    traffic = load_traffic(bytes_alg)
    calls = {}
    for k in names:
        if args.graph:
            break
        calls[k] = {"ms": in_step[k]}
        if k in proj_bytes and in_step[k] > 0:
            gbps = proj_bytes[k] / (in_step[k] / 1e3) / 1e9
            calls[k].update({"alg_bytes": proj_bytes[k], "GBps": gbps, "hbm_frac": gbps / HBM_PEAK_GBPS})
    others, context = None, None
    if not args.headline_only:
        others = measure_other_workloads(dev, stream, max(10, args.steps), lo=lo_flag)
        others["v4_form_bf16"] = measure_v4_form(dev, stream, max(10, args.steps))
        others["prefill_bf16"] = measure_prefill(dev, stream, 20)
        context = gpu_context(dev)
        context["copy_GBps"] = copy_gbps(dev, stream)
    cpu = None if args.no_cpu_baseline else cpu_baseline(w, inp)
    rec = {
        "metric": METRIC,
        "value": B * Q / (ms_step / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"seconds": args.settle_s, "steps": settle_steps,
                   "why": "untimed steps before the warmup steps: the clocks ramp over the first tens of ms"},
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "DeepSeek-V3-shaped MLA decode, one layer: B=32, H=128, Q=1, Dn=128, "
                               "Dr=64, Vd=128, Ckv=512, Lk=4096, contiguous [B,Lk,576] bf16 cache",
                   "global_batch": B, "seq_len": max_len, "parallelism": "none (1 GPU)",
                   "cache_copies": len(caches),
                   "launch": ("hip graph replay" if args.graph else "eager")
                             + (", append and absorption as two calls" if args.separate_append
                                else ", append fused into the absorption launch")
                             + (", attention and up-projection as two calls" if args.separate_up
                                else ", split merge fused with the up-projection"),
                   "scores": ("q_lat + q_lat_lo (bf16 high and low parts of the fp32 absorption)" if use_lo
                              else "q_lat (bf16, the absorption rounded once)"),
                   "inputs_sha256": inp.sha256()},
        "roofline": {"bound": "hbm", "achieved": achieved_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved_gbps / HBM_PEAK_GBPS,
                     "traffic": traffic},
        "attn": {"kernel": "mla_decode_attn (token-split attention + merge)",
                 "avg_ms": attn_avg_ms, "host_us_per_call": host_us,
                 "per_call_p50_ms": pct(0.5), "per_call_p95_ms": pct(0.95), "per_call_p99_ms": pct(0.99),
                 "alg_bytes": bytes_alg, "alg_flops": flops, "kv_GBps": cache_bytes / attn_s / 1e9,
                 "mfma_TFLOPs": tflops, "mfma_frac": tflops / MFMA_BF16_PEAK_TFLOPS,
                 "kernel_source_hash": kernel_source_hash()},
        "calls_in_step": calls or None,
        "rope_append": {"call": "mla_rope_append (k_pe rotated and appended, q_pe [B,128,1,64] rotated in place)",
                        "ms": rope_ms, "plain_append_ms": plain_append_ms,
                        "bytes": B * Q * (w.Ckv + w.Dr) * 2 * 2 + B * w.H * Q * w.Dr * 2 * 2 + B * Q * w.Dr * 4,
                        "bound": "launch latency"},
        "workloads": others,
        "context": context,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
