"""Shared helpers of the parity tests: GPU inputs, the GPU path, the oracle side.

The GPU side goes only through the C ABI (mla_latent_kv_08_amd.ops); the oracle
side only through oracle/. Both are fed from workloads.py.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np
import torch

import workloads as W
from oracle import fp4_ref, mla_ref

TOL = {"f32": 1e-4, "bf16": 1e-2, "fp4": 1e-2}
# q_lat + q_lat_lo against the fp64 absorption: the two bf16 parts hold the
# fp32 sum to about 2^-17 of each element, plus the fp32 accumulation error.
Q_SPLIT_TOL = 1e-4


def ops():
    from mla_latent_kv_08_amd import ops as _ops
    return _ops


def say(msg: str) -> None:
    print(msg, flush=True)


# ---------------------------------------------------------------------------
# GPU side
# ---------------------------------------------------------------------------

class GpuCase:
    def __init__(self, inp: W.Inputs, poison: bool = True, capacity: Optional[int] = None,
                 page_perm_override=None):
        o = ops()
        self.inp = inp
        w = inp.w
        self.w = w
        dev = "cuda"
        self.pl = W.place(inp, capacity)
        self.q_nope = inp.q_nope.to(dev)
        self.q_pe = inp.q_pe.to(dev)
        self.wkv_b = inp.wkv_b.to(dev)
        self.seq_lens = inp.seq_lens.to(dev)
        self.max_len = int(inp.seq_lens.max()) if w.B else 0
        pt = self.pl.page_table.to(dev) if self.pl.page_table is not None else None
        if w.dtype in ("f32", "bf16"):
            fill = float("nan") if poison else 0.0
            buf = W.combined_rows(inp.latent, inp.rope, self.pl, fill).to(dev)
            self.cache = o.LatentCache.combined(buf, w.Ckv, self.pl.capacity, page_table=pt)
        else:
            row = o.LatentCache.fp4_row_bytes(w.Ckv, w.Dr)
            fillb = 0xFF if poison else 0
            buf = torch.full((self.pl.n_rows, row), fillb, dtype=torch.uint8, device=dev)
            self.cache = o.LatentCache.fp4(buf, w.Ckv, self.pl.capacity, page_table=pt)
            self.append_all(inp.latent)
        self.buf = buf

    def append_all(self, latent_rows: torch.Tensor, src_dtype=torch.float32):
        """Write every logical token through mla_cache_append (one call, right-aligned)."""
        o = ops()
        w, inp = self.w, self.inp
        n = self.max_len
        if n == 0:
            return
        c = torch.zeros(w.B, n, w.Ckv, dtype=src_dtype)
        r = torch.zeros(w.B, n, w.Dr, dtype=inp.rope.dtype)
        for b in range(w.B):
            L = int(inp.seq_lens[b])
            if L:
                c[b, n - L:] = latent_rows[inp.seq_offsets[b]:inp.seq_offsets[b + 1]].to(src_dtype)
                r[b, n - L:] = inp.seq_rope(b)
        o.mla_cache_append(c.cuda(), r.cuda(), self.cache, self.seq_lens)

    def run(self, workgroups: int = 0, lo: bool = True):
        """One decode step through the C ABI. bf16 / FP4: with `lo` the query's low
        part (q_lat_lo) is formed by mla_absorb_q and used by the scores."""
        o = ops()
        w = self.w
        dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
        B, H, Q = w.B, w.H, w.Q
        q_lat = torch.empty(B, H, Q, w.Ckv, dtype=dt, device="cuda")
        q_lo = torch.empty_like(q_lat) if (lo and w.dtype != "f32") else None
        x = torch.empty(B, H, Q, w.Ckv, dtype=dt, device="cuda")
        lse = torch.empty(B, H, Q, dtype=torch.float32, device="cuda")
        out = torch.empty(B, H, Q, w.Vd, dtype=dt, device="cuda")
        o.mla_absorb_q(self.q_nope, self.wkv_b, q_lat, q_lat_lo=q_lo)
        o.mla_decode_attn(q_lat, self.q_pe, self.cache, self.seq_lens, self.max_len, w.softmax_scale,
                          x, lse, workgroups=workgroups, q_lat_lo=q_lo)
        o.mla_up_proj_v(x, self.wkv_b, out)
        torch.cuda.synchronize()
        res = {"q_lat": q_lat, "x": x, "lse": lse, "out": out}
        if q_lo is not None:
            res["q_lat_lo"] = q_lo
        return res


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


# ---------------------------------------------------------------------------
# Oracle side
# ---------------------------------------------------------------------------

def oracle_latent_rows(inp: W.Inputs, b: int):
    """Latent rows of sequence b as the oracle sees them (FP4: quantised by the oracle's codec)."""
    rows = inp.seq_latent(b)
    if inp.w.dtype == "fp4":
        codes, scales = fp4_ref.quantize_rows_fast(rows.numpy())
        return fp4_ref.dequantize_rows(codes, scales)
    return rows


def oracle(inp: W.Inputs, heads: Optional[Sequence[int]] = None, batch: Optional[Sequence[int]] = None):
    w = inp.w
    bs = list(range(w.B)) if batch is None else list(batch)
    kv = [oracle_latent_rows(inp, b) for b in bs]
    pe = [inp.seq_rope(b) for b in bs]
    lens = [int(inp.seq_lens[b]) for b in bs]
    res = mla_ref.decode_nonabsorbed(inp.q_nope[bs], inp.q_pe[bs], kv, pe, inp.wkv_b, lens,
                                     w.softmax_scale, heads=heads)
    hs = list(range(w.H)) if heads is None else list(heads)
    res["q_lat"] = mla_ref.absorb_q(inp.q_nope[bs][:, hs], inp.wkv_b[hs])
    return res


def assert_close(gpu: np.ndarray, ref: np.ndarray, tol: float, name: str):
    ref = np.asarray(ref)
    gpu = np.asarray(gpu)
    assert gpu.shape == ref.shape, (name, gpu.shape, ref.shape)
    assert np.isfinite(gpu).all(), f"{name}: non-finite GPU values"
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    err = float(np.max(np.abs(gpu - ref))) if ref.size else 0.0
    say(f"  {name}: max|err| = {err:.3e}, max|ref| = {scale:.3e}, ratio = {err / max(scale, 1e-300):.3e}")
    assert err <= tol * scale, f"{name}: max|err| {err:.3e} > {tol} * {scale:.3e}"


def assert_lse_close(gpu: np.ndarray, ref: np.ndarray, tol: float, name: str = "lse"):
    fin = np.isfinite(ref)
    assert np.array_equal(np.isneginf(gpu), np.isneginf(ref)), f"{name}: -inf pattern differs"
    if fin.any():
        err = float(np.max(np.abs(gpu[fin] - ref[fin])))
        lim = tol * (1.0 + float(np.max(np.abs(ref[fin]))))
        say(f"  {name}: max|err| = {err:.3e} (limit {lim:.3e})")
        assert err <= lim


def compare(gpu: dict, ref: dict, w: W.Workload, heads=None, batch=None, tol=None):
    """x, out (and q_lat) within tol * max|ref| (default: the dtype's bar); lse within tol * (1 + max|lse|)."""
    tol = TOL[w.dtype] if tol is None else tol
    sel = lambda t: t if batch is None else t[list(batch)]  # noqa: E731
    hsel = lambda t: t if heads is None else t[:, list(heads)]  # noqa: E731
    assert_close(to64(hsel(sel(gpu["q_lat"]))), ref["q_lat"], tol, "q_lat")
    if "q_lat_lo" in gpu:
        # hi + lo keeps about 16 significant bits of the fp32 sum.
        both = to64(hsel(sel(gpu["q_lat"]))) + to64(hsel(sel(gpu["q_lat_lo"])))
        assert_close(both, ref["q_lat"], Q_SPLIT_TOL, "q_lat + q_lat_lo")
    assert_close(to64(hsel(sel(gpu["x"]))), ref["x"], tol, "x")
    assert_lse_close(to64(hsel(sel(gpu["lse"]))), ref["lse"], tol)
    assert_close(to64(hsel(sel(gpu["out"]))), ref["out"], tol, "out")
