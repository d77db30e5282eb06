"""Seeded synthetic inputs for MLA decode workloads.

This module holds only random draws, dtype rounding and data placement (which
physical cache row or page a logical token lands in). It contains none of the
attention arithmetic, so that the HIP path and the CPU oracle can both be fed
from it without sharing any of the method's computation.

Shapes follow the DeepSeek-V3 MLA layer used throughout the pages: 128 heads,
a 128-wide non-RoPE query/key part, a 64-wide decoupled RoPE part, a 128-wide
value head and a 512-wide compressed latent (page "DeepSeek-V3/R1 architecture
deep dive", the MultiHeadLatentAttention sketch; page "MLA decode step"
exercise, the argument shape comments of mla_decode_step).

Draw order for one workload (a single CPU torch.Generator seeded with the
workload seed): [per-sequence lengths], q_nope, q_pe, latent rows (logical
order: sequence 0 tokens 0..len-1, then sequence 1, ...), RoPE rows, wkv_b,
then extras (page permutation, spiked token indices). Normal draws are fp32
and are rounded once (RNE) to the storage dtype.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Optional, Sequence

import torch

PAGE_TOKENS = 64


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Q: int
    Dn: int
    Dr: int
    Vd: int
    Ckv: int
    dtype: str  # "f32", "bf16" or "fp4" (FP4 latent, bf16 everything else)
    seed: int
    lk: Optional[int] = None  # every sequence has this length
    lk_range: Optional[tuple] = None  # inclusive integer-uniform draw per sequence
    lens: Optional[tuple] = None  # explicit lengths (reduced parity cases)
    paged: bool = False  # 64-token pages dealt from a shuffled shared pool
    spike_frac: float = 0.0  # fraction of tokens per sequence whose latent is scaled
    spike_mult: float = 1.0
    # Run configuration, not data: whether the timed launch passes the query's
    # low part (q_lat_lo) to the scores. Spiked logits need it to stay within
    # the bf16 bar; over an FP4 latent it only sharpens the query's one
    # rounding to fp16, at no matrix-op cost.
    q_lat_lo: bool = False

    @property
    def softmax_scale(self) -> float:
        # 1/sqrt(Dn + Dr): the demo of the decode-step exercise page.
        return 1.0 / math.sqrt(self.Dn + self.Dr)

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads. Names describe what each one is.
WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", B=1, H=16, Q=1, Dn=128, Dr=64, Vd=128, Ckv=512,
                         dtype="f32", seed=0, lk=256),
    "dsv3_bf16": Workload("dsv3_bf16", B=32, H=128, Q=1, Dn=128, Dr=64, Vd=128, Ckv=512,
                          dtype="bf16", seed=1, lk=4096),
    "ragged_paged_bf16": Workload("ragged_paged_bf16", B=64, H=128, Q=1, Dn=128, Dr=64, Vd=128,
                                  Ckv=512, dtype="bf16", seed=2, lk_range=(512, 32768),
                                  paged=True),
    "long_splitkv_bf16": Workload("long_splitkv_bf16", B=4, H=128, Q=1, Dn=128, Dr=64, Vd=128,
                                  Ckv=512, dtype="bf16", seed=3, lk=131072,
                                  spike_frac=0.01, spike_mult=8.0, q_lat_lo=True),
    "mtp_fp4": Workload("mtp_fp4", B=128, H=128, Q=2, Dn=128, Dr=64, Vd=128, Ckv=512,
                        dtype="fp4", seed=4, lk=8192, q_lat_lo=True),
}
WORKLOAD_ORDER = ["tiny_f32", "dsv3_bf16", "ragged_paged_bf16", "long_splitkv_bf16", "mtp_fp4"]


def storage_dtype(w: Workload) -> torch.dtype:
    return torch.float32 if w.dtype == "f32" else torch.bfloat16


@dataclasses.dataclass
class Inputs:
    """Logical inputs of one workload (CPU tensors).

    latent/rope hold the rows of all sequences back to back in logical order;
    seq_offsets[b] is where sequence b starts. For the FP4 workload `latent` is
    the fp32 latent before quantisation; every other tensor is in storage dtype.
    """
    w: Workload
    seq_lens: torch.Tensor  # int32 [B], includes the Q new tokens
    seq_offsets: torch.Tensor  # int64 [B+1]
    q_nope: torch.Tensor  # [B,H,Q,Dn]
    q_pe: torch.Tensor  # [B,H,Q,Dr]
    latent: torch.Tensor  # [T,Ckv]
    rope: torch.Tensor  # [T,Dr]
    wkv_b: torch.Tensor  # [H,Dn+Vd,Ckv]
    page_perm: Optional[torch.Tensor] = None  # int64 [pool] physical page of the k-th logical page
    spike_rows: Optional[torch.Tensor] = None  # int64 global logical rows that were scaled

    def seq_latent(self, b: int) -> torch.Tensor:
        return self.latent[self.seq_offsets[b]:self.seq_offsets[b + 1]]

    def seq_rope(self, b: int) -> torch.Tensor:
        return self.rope[self.seq_offsets[b]:self.seq_offsets[b + 1]]

    def sha256(self) -> dict:
        out = {}
        for k in ("seq_lens", "q_nope", "q_pe", "latent", "rope", "wkv_b", "page_perm", "spike_rows"):
            t = getattr(self, k)
            if t is None:
                continue
            t = t.contiguous()
            if t.dtype == torch.bfloat16:
                t = t.view(torch.int16)
            out[k] = hashlib.sha256(t.numpy().tobytes()).hexdigest()
        return out


def _lengths(w: Workload, g: torch.Generator) -> torch.Tensor:
    if w.lens is not None:
        assert len(w.lens) == w.B
        return torch.tensor(w.lens, dtype=torch.int32)
    if w.lk_range is not None:
        lo, hi = w.lk_range
        return torch.randint(lo, hi + 1, (w.B,), generator=g, dtype=torch.int64).to(torch.int32)
    return torch.full((w.B,), int(w.lk), dtype=torch.int32)


def generate(w: Workload) -> Inputs:
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed)
    lens = _lengths(w, g)
    offs = torch.zeros(w.B + 1, dtype=torch.int64)
    offs[1:] = torch.cumsum(lens.to(torch.int64), 0)
    T = int(offs[-1])
    q_nope = torch.randn(w.B, w.H, w.Q, w.Dn, generator=g)
    q_pe = torch.randn(w.B, w.H, w.Q, w.Dr, generator=g)
    latent = torch.randn(T, w.Ckv, generator=g)
    rope = torch.randn(T, w.Dr, generator=g)
    # wkv_b ~ N(0, 1/Ckv): variance 1/512 for the 512-wide latent.
    wkv_b = torch.randn(w.H, w.Dn + w.Vd, w.Ckv, generator=g) * (1.0 / math.sqrt(w.Ckv))
    page_perm = None
    if w.paged:
        pages = int(sum((int(l) + PAGE_TOKENS - 1) // PAGE_TOKENS for l in lens))
        page_perm = torch.randperm(pages, generator=g)
    spike_rows = None
    if w.spike_frac > 0:
        rows = []
        for b in range(w.B):
            L = int(lens[b])
            k = int(math.floor(w.spike_frac * L))
            idx = torch.randperm(L, generator=g)[:k]
            rows.append(idx.to(torch.int64) + int(offs[b]))
        spike_rows = torch.sort(torch.cat(rows)).values
        latent[spike_rows] *= w.spike_mult
    sd = storage_dtype(w)
    q_nope = q_nope.to(sd)
    q_pe = q_pe.to(sd)
    rope = rope.to(sd)
    wkv_b = wkv_b.to(sd)
    if w.dtype != "fp4":
        latent = latent.to(sd)
    return Inputs(w, lens, offs, q_nope, q_pe, latent, rope, wkv_b, page_perm, spike_rows)


# ---------------------------------------------------------------------------
# Physical placement of cache rows (layout only).
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class Placement:
    """Where each logical token row lives in the physical cache.

    Contiguous caches reserve `capacity` rows per sequence: row = b*capacity + t.
    Paged caches hold 64-token pages; page_table[b, j] is the physical page of
    the sequence's j-th logical page and row = page*64 + t%64.
    """
    n_rows: int
    capacity: int
    page_size: int  # 0 = contiguous
    page_table: Optional[torch.Tensor]  # int32 [B, max_pages]
    rows: torch.Tensor  # int64 [T] physical row of each logical row


def place(inp: Inputs, capacity: Optional[int] = None) -> Placement:
    w = inp.w
    lens = [int(l) for l in inp.seq_lens]
    if not w.paged:
        cap = capacity if capacity is not None else max(max(lens), 1)
        rows = torch.cat([torch.arange(L, dtype=torch.int64) + b * cap for b, L in enumerate(lens)]) \
            if sum(lens) else torch.zeros(0, dtype=torch.int64)
        return Placement(w.B * cap, cap, 0, None, rows)
    npages = [(L + PAGE_TOKENS - 1) // PAGE_TOKENS for L in lens]
    max_pages = max(max(npages), 1)
    table = torch.zeros(w.B, max_pages, dtype=torch.int32)
    perm = inp.page_perm
    rows = []
    k = 0
    for b, L in enumerate(lens):
        for j in range(npages[b]):
            table[b, j] = int(perm[k])
            k += 1
        t = torch.arange(L, dtype=torch.int64)
        rows.append(table[b, (t // PAGE_TOKENS)].to(torch.int64) * PAGE_TOKENS + t % PAGE_TOKENS)
    rows = torch.cat(rows) if rows else torch.zeros(0, dtype=torch.int64)
    n_pages = int(perm.numel())
    return Placement(n_pages * PAGE_TOKENS, max_pages * PAGE_TOKENS, PAGE_TOKENS, table, rows)


def scatter_rows(src: torch.Tensor, placement: Placement, fill: float = float("nan")) -> torch.Tensor:
    """Physical [n_rows, D] array holding src's logical rows; unused rows are `fill`."""
    out = torch.full((placement.n_rows, src.shape[1]), fill, dtype=src.dtype)
    if src.shape[0]:
        out[placement.rows] = src
    return out


def combined_rows(latent: torch.Tensor, rope: torch.Tensor, placement: Placement,
                  fill: float = float("nan")) -> torch.Tensor:
    """Physical [n_rows, Ckv+Dr] cache with each row = [latent | rope]."""
    return torch.cat([scatter_rows(latent, placement, fill), scatter_rows(rope, placement, fill)], 1)


def reduced(w: Workload, B: int, lens: Sequence[int], seed: Optional[int] = None) -> Workload:
    """A smaller workload with the same structure (for parity at oracle-friendly sizes)."""
    return w.with_(B=B, lens=tuple(int(x) for x in lens), lk=None, lk_range=None,
                   seed=w.seed if seed is None else seed)


def rope_table(n_pos: int, d: int, base: float = 10000.0) -> torch.Tensor:
    """A caller's cosine/sine table for the rotary embedding: fp32 [n_pos, d],
    row p = [cos(p w_0) .. cos(p w_{d/2-1}), sin(p w_0) .. sin(p w_{d/2-1})]
    with the usual schedule w_i = base^(-2i/d). The angles are formed in fp64
    and the values rounded once to fp32; the library applies whatever table
    it is given, so this is input data like any other."""
    i = torch.arange(d // 2, dtype=torch.float64)
    w = base ** (-2.0 * i / d)
    ang = torch.arange(n_pos, dtype=torch.float64)[:, None] * w[None, :]
    return torch.cat([torch.cos(ang), torch.sin(ang)], 1).to(torch.float32)
