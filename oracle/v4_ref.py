"""Plain fp64 reference of the DeepSeek-V4.1-Flash form of latent attention:
RoPE on the tail of the latent, a per-head sink score column, and the inverse
rotation of the output's tail.

TEST INFRASTRUCTURE. Only tests/, the smoke check of the package entry file and
the CPU-baseline leg of bench.py may import this module. The product path (the
HIP library and its Python binding) never calls it and shares no code with it.

What the course page (DeepSeek-V4.1-Flash, block 4A) fixes: one 512-wide latent
per cached entry serves every head as key and value; only the tail of the
latent carries the rotary position (the figure caption and the walkthrough say
the last 64 dims); attention runs with an attention-sink score column; the
output's rotated part is turned back (inverse RoPE) before the grouped output
projection, so that position does not leak into the hidden state. Readings
taken where it is silent:

  * the rotated dims are the last r = 64 of the 512; pairs and angles are those
    of `rope_ref` (a caller's cos/sin table and a pairing style);
  * key t is the latent of token t with its tail turned to position t; the
    query of head h (512 wide) has its tail turned to the query's position
    len - Q + q; the value of token t is the same rotated latent;
  * s_t = scale * (q . k_t) over the 512 dims; position t is visible to query
    q iff t <= len - Q + q;
  * the sink of head h is one more logit, in the units of the scaled scores,
    that enters the softmax normaliser and carries no value:
      p_t = exp(s_t) / (sum_{t' visible} exp(s_t') + exp(sink_h));
  * x = sum_t p_t v_t, then the last r dims of x are turned back by the
    query's position (rotation by the negated angles);
  * lse = log(sum_t exp(s_t) + exp(sink_h)) (the sink included); a query with
    no visible token gets x = 0 and lse = sink_h (-inf without a sink).
"""
from __future__ import annotations

import numpy as np

from oracle import rope_ref as RR


def rotate_tail(x, cos_sin_row, style: int, r: int, inverse: bool = False) -> np.ndarray:
    """x [..., C] with its last r dims turned by one table row (negated angles if inverse)."""
    x = np.asarray(x, dtype=np.float64)
    row = np.asarray(cos_sin_row, dtype=np.float64)
    if inverse:
        row = np.concatenate([row[: r // 2], -row[r // 2:]])
    out = x.copy()
    out[..., -r:] = RR.rotate(x[..., -r:], row, style)
    return out


def decode_v4(q, latent_rows, seq_lens, cos_sin, style: int, softmax_scale: float, sinks=None, r: int = 64):
    """q [B, H, Q, C] (tails not yet rotated); latent_rows: per sequence [len, C]
    unrotated latents; cos_sin [n_pos, r]; sinks [H] or None.
    Returns {"x": [B,H,Q,C], "lse": [B,H,Q]}."""
    q = np.asarray(q, dtype=np.float64)
    table = np.asarray(cos_sin, dtype=np.float64)
    B, H, Q, C = q.shape
    x = np.zeros((B, H, Q, C))
    lse = np.zeros((B, H, Q))
    sk = np.full(H, -np.inf) if sinks is None else np.asarray(sinks, dtype=np.float64)
    for b in range(B):
        n = int(seq_lens[b])
        lat = np.asarray(latent_rows[b], dtype=np.float64)[:n]
        keys = np.stack([rotate_tail(lat[t], table[t], style, r) for t in range(n)]) if n else np.zeros((0, C))
        for j in range(Q):
            pos = n - Q + j
            vis = max(0, min(n, pos + 1))
            for h in range(H):
                if vis == 0:
                    lse[b, h, j] = sk[h]
                    continue
                qh = rotate_tail(q[b, h, j], table[pos], style, r)
                s = softmax_scale * (keys[:vis] @ qh)
                m = max(np.max(s), sk[h])
                e = np.exp(s - m)
                den = np.sum(e) + np.exp(sk[h] - m)
                xv = (e / den) @ keys[:vis]
                x[b, h, j] = rotate_tail(xv, table[pos], style, r, inverse=True)
                lse[b, h, j] = m + np.log(den)
    return {"x": x, "lse": lse}


def grouped_out_proj(x, w_o) -> np.ndarray:
    """The grouped output projection that follows the V4.1-Flash form (course
    page, block 4A: the head outputs go through W_O by groups, each group with
    its own small matrix, the results joined into the hidden dimension; the
    figure gives 8 groups x 1024). Readings: with G groups of H/G heads, group
    g holds heads g*H/G .. (g+1)*H/G - 1; their rows (after the inverse
    rotation) are joined head after head into one vector of (H/G)*C; W_O[g]
    [N, (H/G)*C] maps it to hidden columns g*N .. g*N + N - 1.

    x [B, H, Q, C]; w_o [G, N, (H/G)*C] -> out [B, Q, G*N], in fp64.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w_o, dtype=np.float64)
    B, H, Q, C = x.shape
    G, N, K = w.shape
    if H % G or K != (H // G) * C:
        raise ValueError("w_o must be [G, N, (H/G)*C] with G dividing H")
    hg = H // G
    out = np.zeros((B, Q, G * N))
    for g in range(G):
        # [B, Q, hg*C]: the group's heads joined, head after head.
        xg = x[:, g * hg:(g + 1) * hg].transpose(0, 2, 1, 3).reshape(B, Q, hg * C)
        out[:, :, g * N:(g + 1) * N] = xg @ w[g].T
    return out
