"""Pins of the V4.1-Flash-form reference (oracle/v4_ref.py): the sink column
against the main oracle's attention over an extra zero-value token (a
different code path), invariance of x and lse when every position shifts by
the same amount (which fails if keys, queries and the inverse rotation do not
use matching positions), the untouched head of the latent, and the empty-row
convention."""
import math

import numpy as np
import pytest

import workloads as W
from oracle import mla_ref as R
from oracle import rope_ref as RR
from oracle import v4_ref as V

C, RDIM = 32, 8  # small latent with an 8-wide rotated tail


def _case(seed, B=2, H=3, Q=2, lens=(9, 5)):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, Q, C))
    lat = [rng.standard_normal((n, C)) for n in lens]
    return q, lat, list(lens)


@pytest.mark.parametrize("style", [RR.INTERLEAVED, RR.HALVES])
def test_sink_is_an_extra_zero_value_token(style):
    q, lat, lens = _case(1)
    table = W.rope_table(64, RDIM).double().numpy()
    scale = 1 / math.sqrt(C)
    sinks = np.array([0.5, -2.0, 3.0])
    got = V.decode_v4(q, lat, lens, table, style, scale, sinks, r=RDIM)
    B, H, Q, _ = q.shape
    for b in range(B):
        n = lens[b]
        keys = np.stack([V.rotate_tail(lat[b][t], table[t], style, RDIM) for t in range(n)])
        for j in range(Q):
            pos = n - Q + j
            for h in range(H):
                qh = V.rotate_tail(q[b, h, j], table[pos], style, RDIM)
                # Tokens 0..pos, then a row with value 0 whose score is the sink,
                # planted through a one-wide position stream.
                c = np.vstack([keys[: pos + 1], np.zeros(C)])
                kpe = np.zeros((pos + 2, 1))
                kpe[-1, 0] = sinks[h] / scale
                x, lse = R.attend_subset(qh, np.ones(1), c, kpe, scale, range(pos + 2))
                x = V.rotate_tail(x, table[pos], style, RDIM, inverse=True)
                np.testing.assert_allclose(got["x"][b, h, j], x, rtol=1e-12, atol=1e-12)
                assert abs(got["lse"][b, h, j] - lse) <= 1e-12 * (1 + abs(lse))


def test_head_of_the_latent_is_not_rotated():
    q, lat, lens = _case(2)
    table = W.rope_table(64, RDIM).double().numpy()
    x = V.rotate_tail(lat[0][3], table[17], RR.INTERLEAVED, RDIM)
    np.testing.assert_array_equal(x[:-RDIM], lat[0][3][:-RDIM])
    assert np.max(np.abs(x[-RDIM:] - lat[0][3][-RDIM:])) > 1e-3


@pytest.mark.parametrize("style", [RR.INTERLEAVED, RR.HALVES])
def test_shifting_every_position_changes_nothing(style):
    q, lat, lens = _case(3)
    table = W.rope_table(4096, RDIM).double().numpy()
    scale = 1 / math.sqrt(C)
    sinks = np.array([0.1, 1.0, -1.0])
    a = V.decode_v4(q, lat, lens, table, style, scale, sinks, r=RDIM)
    b = V.decode_v4(q, lat, lens, table[1000:], style, scale, sinks, r=RDIM)
    np.testing.assert_allclose(b["x"], a["x"], rtol=0, atol=1e-5)  # the table is fp32
    np.testing.assert_allclose(b["lse"], a["lse"], rtol=0, atol=1e-5)
    # Without the inverse rotation (output tail left turned) the shift shows.
    def raw_tail(tab):
        out = []
        for bb in range(len(lens)):
            n = lens[bb]
            keys = np.stack([V.rotate_tail(lat[bb][t], tab[t], style, RDIM) for t in range(n)])
            out.append(keys[-1, -RDIM:])
        return np.stack(out)
    assert np.max(np.abs(raw_tail(table) - raw_tail(table[1000:]))) > 1e-2


def test_query_without_visible_token():
    q, lat, _ = _case(4, B=2, Q=2, lens=(1, 0))
    table = W.rope_table(8, RDIM).double().numpy()
    sinks = np.array([0.7, -0.3, 2.0])
    out = V.decode_v4(q, lat, [1, 0], table, RR.INTERLEAVED, 0.2, sinks, r=RDIM)
    # Sequence 0 (len 1, Q 2): query 0 sees nothing; sequence 1 sees nothing at all.
    assert np.all(out["x"][0, :, 0] == 0) and np.all(out["x"][1] == 0)
    np.testing.assert_array_equal(out["lse"][0, :, 0], sinks)
    np.testing.assert_array_equal(out["lse"][1, :, 1], sinks)
    none = V.decode_v4(q, lat, [1, 0], table, RR.INTERLEAVED, 0.2, None, r=RDIM)
    assert np.all(np.isneginf(none["lse"][1]))


def test_grouped_out_proj_bruteforce_and_structure():
    rng = np.random.default_rng(6)
    B, H, Q, Cc, G, N = 2, 6, 2, 4, 3, 5
    x = rng.standard_normal((B, H, Q, Cc))
    w = rng.standard_normal((G, N, (H // G) * Cc))
    out = V.grouped_out_proj(x, w)
    # Scalar loops straight from the reading.
    ref = np.zeros((B, Q, G * N))
    for b in range(B):
        for q in range(Q):
            for g in range(G):
                for n in range(N):
                    acc = 0.0
                    for j in range(H // G):
                        for c in range(Cc):
                            acc += w[g, n, j * Cc + c] * x[b, g * (H // G) + j, q, c]
                    ref[b, q, g * N + n] = acc
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-13)
    # A change to one group's heads moves only that group's columns.
    x2 = x.copy()
    x2[:, 2:4] += 1.0  # heads of group 1
    d = V.grouped_out_proj(x2, w) - out
    assert np.all(d[:, :, :N] == 0) and np.all(d[:, :, 2 * N:] == 0) and np.any(d[:, :, N:2 * N] != 0)
    # A selector matrix returns the group's second head.
    sel = np.zeros((G, Cc, (H // G) * Cc))
    sel[:, :, Cc:2 * Cc] = np.eye(Cc)
    s = V.grouped_out_proj(x, sel)
    for g in range(G):
        np.testing.assert_array_equal(s[:, :, g * Cc:(g + 1) * Cc], x[:, g * (H // G) + 1].transpose(0, 1, 2))
