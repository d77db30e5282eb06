"""Plain fp64 CPU oracle for MLA decode with weight absorption.

TEST INFRASTRUCTURE. Only tests/, the smoke check of the package entry file and
the CPU-baseline leg of bench.py may import this module. The product path (the
HIP library and its Python binding) never calls it and shares no code with it.

What it computes (notation of the "MLA decode step" exercise page: q_nope
[B,H,Q,Dn], q_pe [B,H,Q,Dr], kv_cache [B,Lk,Ckv], pe_cache [B,Lk,Dr], wkv_b
[H,Dn+Vd,Ckv] whose first Dn rows per head are W_UK and last Vd rows are W_UV):

The main entry, `decode_nonabsorbed`, is the "restore first" evaluation the
CacheCompressed discussion page describes: per head it decompresses the key and
value of every visible token from the latent, then runs ordinary attention:

  1. K_nope[t,h,:] = W_UK[h] c_t and V[t,h,:] = W_UV[h] c_t    (decompression)
  2. s_t = softmax_scale * (q_nope . K_nope[t] + q_pe . k_pe[t]) (two score
     streams merged, then scaled: exercise page, prose and step 3)
  3. only positions up to the query's own position are visible (exercise page,
     prose: future positions are masked; step 4 sets them to -inf)
  4. p = softmax over the visible positions (exercise page, torch.softmax)
  5. out = sum_t p_t V[t]; x = sum_t p_t c_t (exercise page: x is the weighted
     sum over kv_cache; out maps it to the value space)

Readings taken where the pages are silent (each is listed with its reason in
the design notes of the repository):
  * visibility: query q of Q new tokens of a sequence whose cache holds `len`
    rows (the Q new rows included) sees positions 0..len-Q+q;
  * a query with no visible position yields out = 0, x = 0, lse = -inf;
  * lse is the natural-log log-sum-exp of the scaled logits.

Visible rows are taken by slicing, never by multiplying with a mask, so values
in hidden rows (NaN, huge numbers) cannot reach any result.
"""
from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence

import numpy as np


def _f64(a) -> np.ndarray:
    """fp64 copy of a numpy array or CPU torch tensor (bf16 converts exactly)."""
    if hasattr(a, "detach"):
        import torch
        t = a.detach()
        if t.dtype in (torch.bfloat16, torch.float16):
            t = t.to(torch.float32)
        return t.to(torch.float64).numpy()
    return np.asarray(a, dtype=np.float64)


def visible_count(seq_len: int, q_len: int, q: int) -> int:
    """Number of cache positions query q (0-based among q_len new tokens) may see."""
    return int(max(0, min(seq_len, seq_len - q_len + q + 1)))


def absorb_q(q_nope, wkv_b, Dn: Optional[int] = None) -> np.ndarray:
    """q_lat[b,h,q,c] = sum_d q_nope[b,h,q,d] * W_UK[h,d,c] by direct summation.

    The absorption of W_UK into the query: the DeepSeek-V3 deep-dive page
    (comment in forward_inference: pre-multiply Q by W_UK before the score) and
    the exercise page, step 1 (project q_nope into the latent space).
    """
    qn = _f64(q_nope)
    w = _f64(wkv_b)
    Dn = qn.shape[-1] if Dn is None else Dn
    return np.einsum("bhqd,hdc->bhqc", qn, w[:, :Dn, :])


def up_proj_v(x, wkv_b, Dn: int) -> np.ndarray:
    """out[b,h,q,v] = sum_c W_UV[h,v,c] * x[b,h,q,c] (exercise page, step 5)."""
    xx = _f64(x)
    w = _f64(wkv_b)
    return np.einsum("bhqc,hvc->bhqv", xx, w[:, Dn:, :])


def _softmax_stats(s: np.ndarray):
    """max, exp(s-max), sum and lse along the last axis of a non-empty score row."""
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    l = np.sum(e, axis=-1, keepdims=True)
    return m, e, l, (m + np.log(l))[..., 0]


def decode_nonabsorbed(q_nope, q_pe, kv_rows: Sequence, pe_rows: Sequence, wkv_b,
                       seq_lens: Iterable[int], softmax_scale: float,
                       heads: Optional[Sequence[int]] = None, token_block: int = 2048,
                       return_probs: bool = False):
    """Non-absorbed fp64 MLA decode (the oracle's definition of the path).

    kv_rows[b] / pe_rows[b]: the sequence's latent rows [>=len, Ckv] and RoPE
    rows [>=len, Dr] in logical token order (arrays or CPU tensors).
    heads: subset of heads to evaluate (all by default); outputs are indexed by
    position in that list.
    Returns dict(out [B,Hs,Q,Vd], x [B,Hs,Q,Ckv], lse [B,Hs,Q]) and, with
    return_probs, p[b][h][q] = probability vector over the visible positions.
    """
    qn = _f64(q_nope)
    qp = _f64(q_pe)
    w = _f64(wkv_b)
    B, H, Q, Dn = qn.shape
    Vd = w.shape[1] - Dn
    Ckv = w.shape[2]
    heads = list(range(H)) if heads is None else list(heads)
    Hs = len(heads)
    w_uk = w[heads, :Dn, :]  # [Hs, Dn, Ckv]
    w_uv = w[heads, Dn:, :]  # [Hs, Vd, Ckv]
    out = np.zeros((B, Hs, Q, Vd))
    x = np.zeros((B, Hs, Q, Ckv))
    lse = np.full((B, Hs, Q), -np.inf)
    probs = [] if return_probs else None
    lens = [int(v) for v in seq_lens]
    for b in range(B):
        L = lens[b]
        nvis = [visible_count(L, Q, q) for q in range(Q)]
        n_all = max(nvis) if nvis else 0
        pb = [[None] * Q for _ in range(Hs)] if return_probs else None
        if n_all == 0:
            if return_probs:
                probs.append(pb)
            continue
        qn_b = qn[b, heads]  # [Hs, Q, Dn]
        qp_b = qp[b, heads]  # [Hs, Q, Dr]
        # Pass 1: decompress K per token block, score every visible position.
        scores = np.empty((Hs, Q, n_all))
        for t0 in range(0, n_all, token_block):
            t1 = min(n_all, t0 + token_block)
            c = _f64(kv_rows[b][t0:t1])  # [T, Ckv]
            kpe = _f64(pe_rows[b][t0:t1])  # [T, Dr]
            k_nope = np.matmul(w_uk, c.T)  # [Hs, Dn, T]: K_nope[t,h,:] = W_UK[h] c_t
            s_nope = np.matmul(qn_b, k_nope)  # [Hs, Q, T]
            s_pe = np.matmul(qp_b, kpe.T)  # [Hs, Q, T]
            scores[:, :, t0:t1] = softmax_scale * (s_nope + s_pe)
        # Softmax over each query's own visible prefix.
        p_full = np.zeros((Hs, Q, n_all))
        for q in range(Q):
            n = nvis[q]
            if n == 0:
                continue
            _, e, l, lse_q = _softmax_stats(scores[:, q, :n])
            p_full[:, q, :n] = e / l
            lse[b, :, q] = lse_q
            if return_probs:
                for i in range(Hs):
                    pb[i][q] = p_full[i, q, :n].copy()
        # Pass 2: decompress V per token block and take the weighted sums.
        for t0 in range(0, n_all, token_block):
            t1 = min(n_all, t0 + token_block)
            c = _f64(kv_rows[b][t0:t1])
            v = np.matmul(w_uv, c.T)  # [Hs, Vd, T]: V[t,h,:] = W_UV[h] c_t
            pblk = p_full[:, :, t0:t1]  # [Hs, Q, T]
            out[b] += np.matmul(pblk, v.transpose(0, 2, 1))
            x[b] += np.matmul(pblk, c)
        if return_probs:
            probs.append(pb)
    res = {"out": out, "x": x, "lse": lse}
    if return_probs:
        res["p"] = probs
    return res


def decode_absorbed(q_nope, q_pe, kv_rows: Sequence, pe_rows: Sequence, wkv_b,
                    seq_lens: Iterable[int], softmax_scale: float):
    """Absorbed fp64 form, used only to check the oracle (the two must agree).

    q_lat = W_UK^T q_nope; s_t = scale*(q_lat . c_t + q_pe . k_pe_t); x = sum p c;
    out = W_UV x (DeepSeek-V3 deep-dive page, absorption comment; exercise page).
    """
    qn = _f64(q_nope)
    qp = _f64(q_pe)
    w = _f64(wkv_b)
    B, H, Q, Dn = qn.shape
    Ckv = w.shape[2]
    q_lat = absorb_q(qn, w, Dn)
    x = np.zeros((B, H, Q, Ckv))
    lse = np.full((B, H, Q), -np.inf)
    lens = [int(v) for v in seq_lens]
    for b in range(B):
        L = lens[b]
        for q in range(Q):
            n = visible_count(L, Q, q)
            if n == 0:
                continue
            c = _f64(kv_rows[b][:n])
            kpe = _f64(pe_rows[b][:n])
            s = softmax_scale * (q_lat[b, :, q] @ c.T + qp[b, :, q] @ kpe.T)  # [H, n]
            _, e, l, lse_q = _softmax_stats(s)
            x[b, :, q] = (e / l) @ c
            lse[b, :, q] = lse_q
    out = up_proj_v(x, w, Dn)
    return {"out": out, "x": x, "lse": lse, "q_lat": q_lat}


def decode_bruteforce(q_nope, q_pe, kv_rows, pe_rows, wkv_b, seq_lens, softmax_scale):
    """Scalar Python loops over every index; tiny inputs only.

    Every product and sum is written out one element at a time, so it checks
    the array code of the other two forms.
    """
    qn = _f64(q_nope).tolist()
    qp = _f64(q_pe).tolist()
    w = _f64(wkv_b).tolist()
    B, H, Q, Dn = len(qn), len(qn[0]), len(qn[0][0]), len(qn[0][0][0])
    Dr = len(qp[0][0][0])
    Ckv = len(w[0][0])
    Vd = len(w[0]) - Dn
    lens = [int(v) for v in seq_lens]
    out = [[[[0.0] * Vd for _ in range(Q)] for _ in range(H)] for _ in range(B)]
    x = [[[[0.0] * Ckv for _ in range(Q)] for _ in range(H)] for _ in range(B)]
    lse = [[[-math.inf] * Q for _ in range(H)] for _ in range(B)]
    for b in range(B):
        c = _f64(kv_rows[b]).tolist()
        kpe = _f64(pe_rows[b]).tolist()
        for h in range(H):
            for q in range(Q):
                n = visible_count(lens[b], Q, q)
                if n == 0:
                    continue
                s = []
                for t in range(n):
                    acc = 0.0
                    for d in range(Dn):
                        k = 0.0
                        for cc in range(Ckv):
                            k += w[h][d][cc] * c[t][cc]
                        acc += qn[b][h][q][d] * k
                    for r in range(Dr):
                        acc += qp[b][h][q][r] * kpe[t][r]
                    s.append(softmax_scale * acc)
                m = max(s)
                e = [math.exp(v - m) for v in s]
                l = sum(e)
                lse[b][h][q] = m + math.log(l)
                for t in range(n):
                    p = e[t] / l
                    for v in range(Vd):
                        val = 0.0
                        for cc in range(Ckv):
                            val += w[h][Dn + v][cc] * c[t][cc]
                        out[b][h][q][v] += p * val
                    for cc in range(Ckv):
                        x[b][h][q][cc] += p * c[t][cc]
    return {"out": np.array(out), "x": np.array(x), "lse": np.array(lse)}


def attend_subset(q_lat_row, q_pe_row, c, kpe, softmax_scale, idx):
    """(x, lse) of one query row over the token subset idx (empty -> (0, -inf)).

    Used to check the split-KV merge rule: attention over a partition of the
    visible positions, merged, must equal attention over all of them.
    """
    idx = list(idx)
    ql = _f64(q_lat_row)
    qp = _f64(q_pe_row)
    cc = _f64(c)
    kp = _f64(kpe)
    if not idx:
        return np.zeros(cc.shape[1]), -np.inf
    s = softmax_scale * (cc[idx] @ ql + kp[idx] @ qp)
    m = np.max(s)
    e = np.exp(s - m)
    l = np.sum(e)
    return (e / l) @ cc[idx], float(m + np.log(l))


def lse_combine(x_parts, lse_parts):
    """Merge split partial results: lse = log sum_s exp(lse_s); x = sum_s exp(lse_s - lse) x_s.

    Parts with lse_s = -inf (empty splits) contribute nothing; if every part is
    empty the result is (0, -inf).
    """
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    x_parts = np.asarray(x_parts, dtype=np.float64)
    finite = np.isfinite(lse_parts)
    if not finite.any():
        return np.zeros(x_parts.shape[1:]), -np.inf
    m = np.max(lse_parts[finite])
    wts = np.where(finite, np.exp(np.where(finite, lse_parts, 0.0) - m), 0.0)
    tot = np.sum(wts)
    lse = m + math.log(tot)
    x = np.tensordot(wts / tot, x_parts, axes=(0, 0))
    return x, lse


def physical_row(b: int, pos: int, capacity: int, page_size: int, page_table=None) -> int:
    """Physical cache row of logical token `pos` of sequence b.

    Contiguous caches: b*capacity + pos. Paged caches: page_table[b][pos//page]
    * page + pos % page (the slot address arithmetic of the latent cache pool on
    the DeepSeek-V3 deep-dive page, with 64-token pages).
    """
    if page_size == 0:
        return b * capacity + pos
    return int(page_table[b][pos // page_size]) * page_size + pos % page_size


def cache_bytes(seq_lens: Iterable[int], bytes_per_row: int) -> int:
    """Bytes a latent cache holds: one shared row per token, whatever the head count."""
    return int(sum(int(l) for l in seq_lens)) * bytes_per_row
