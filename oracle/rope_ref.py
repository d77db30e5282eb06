"""Plain fp64 reference of the rotary position embedding applied on the way
into the latent cache.

TEST INFRASTRUCTURE. Only tests/, the smoke check of the package entry file and
the CPU-baseline leg of bench.py may import this module. The product path (the
HIP library and its Python binding) never calls it and shares no code with it.

What the pages fix: the position part of the key is rotated before it is
stored beside the latent (DeepSeek-V3 architecture deep-dive page,
`forward_inference`: the RoPE key of the new token is `apply_rope` of its
projection, then cached), and a rotation is checked by hand on a few elements,
cosine and sine of the position's angle, with the unrotated part unchanged and
the inverse rotation restoring the vector (DeepSeek-V4.1-Flash course page,
block 4A, the parity checklist). What they leave open, with the reading taken:

  * the angles: the caller supplies them as a table, row p = [cos(a_{p,0}),
    ..., cos(a_{p,d/2-1}), sin(a_{p,0}), ..., sin(a_{p,d/2-1})] for position p
    (d = Dr). The usual schedule a_{p,i} = p * base^(-2i/d) is one such table;
    the reference applies whatever table it is given;
  * which elements form a rotated pair: style INTERLEAVED pairs (2i, 2i+1),
    style HALVES pairs (i, i + d/2); pair i turns by angle a_{p,i};
  * the rotation of a pair (x, y) by a: (x cos a - y sin a, x sin a + y cos a);
  * the position of new token j of a sequence whose length (new tokens
    included) is len: len - Q + j, the row the append writes; the queries of
    a decode step are its new tokens, so query j takes the same position;
  * a position outside the table (or negative) has no angle: its rotated
    values are NaN.
"""
from __future__ import annotations

import numpy as np

INTERLEAVED = 0
HALVES = 1


def pair_index(d: int, style: int):
    """(first, second) element indices of the d/2 rotated pairs."""
    if d % 2:
        raise ValueError("RoPE dimension must be even")
    i = np.arange(d // 2)
    if style == INTERLEAVED:
        return 2 * i, 2 * i + 1
    if style == HALVES:
        return i, i + d // 2
    raise ValueError(f"unknown RoPE style {style}")


def rotate(x, cos_sin_row, style: int) -> np.ndarray:
    """x [..., d] rotated by one table row [d] (cosines, then sines), in fp64."""
    x = np.asarray(x, dtype=np.float64)
    row = np.asarray(cos_sin_row, dtype=np.float64)
    d = x.shape[-1]
    c, s = row[: d // 2], row[d // 2:]
    i0, i1 = pair_index(d, style)
    out = np.empty_like(x)
    xa, xb = x[..., i0], x[..., i1]
    out[..., i0] = xa * c - xb * s
    out[..., i1] = xa * s + xb * c
    return out


def positions(seq_lens, q_len: int) -> np.ndarray:
    """[B, Q] positions len_b - Q + j of the new tokens (and of the queries)."""
    lens = np.asarray(seq_lens, dtype=np.int64)
    return lens[:, None] - q_len + np.arange(q_len)[None, :]


def rope_step(k_pe_new, q_pe, cos_sin, seq_lens, style: int):
    """Rotated new keys [B, Q, d] and queries [B, H, Q, d] of one decode step.

    k_pe_new [B, Q, d]; q_pe [B, H, Q, d] or None; cos_sin [n_pos, d]. A token
    whose position lies outside [0, n_pos) gets NaN.
    """
    k = np.asarray(k_pe_new, dtype=np.float64)
    table = np.asarray(cos_sin, dtype=np.float64)
    B, Q, d = k.shape
    pos = positions(seq_lens, Q)
    k_out = np.full_like(k, np.nan)
    q_out = None
    if q_pe is not None:
        q = np.asarray(q_pe, dtype=np.float64)
        q_out = np.full_like(q, np.nan)
    for b in range(B):
        for j in range(Q):
            p = int(pos[b, j])
            if not 0 <= p < table.shape[0]:
                continue
            k_out[b, j] = rotate(k[b, j], table[p], style)
            if q_out is not None:
                q_out[b, :, j] = rotate(q[b, :, j], table[p], style)
    return k_out, q_out
