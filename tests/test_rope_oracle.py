"""Pins of the RoPE reference (oracle/rope_ref.py) against facts that do not
come from it: hand-computed rotations (golden fixture), the identity at angle
zero, the inverse rotation, norm preservation, the shift invariance of scores
under the usual schedule, the pairing of each style and the positions of the
new tokens."""
import json
import math
import os

import numpy as np
import pytest

import workloads as W
from oracle import rope_ref as RR

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _row(angles):
    a = np.asarray(angles, dtype=np.float64)
    return np.concatenate([np.cos(a), np.sin(a)])


@pytest.mark.parametrize("style,key", [(RR.INTERLEAVED, "interleaved"), (RR.HALVES, "halves")])
def test_hand_computed_rotation(style, key):
    g = json.load(open(os.path.join(GOLDEN, "rope_hand.json")))
    got = RR.rotate(g["x"], _row(g["angles"]), style)
    np.testing.assert_allclose(got, g[key]["expected"], rtol=0, atol=1e-15)
    i0, i1 = RR.pair_index(4, style)
    assert [[int(a), int(b)] for a, b in zip(i0, i1)] == g[key]["pairs"]


@pytest.mark.parametrize("style", [RR.INTERLEAVED, RR.HALVES])
def test_pairing_moves_sine_to_the_partner(style):
    # A unit vector on element 0 turned by a: cos a stays on element 0, sin a
    # lands on its partner (1 for interleaved pairs, d/2 for halves); every
    # other element stays 0.
    d, a = 64, 0.3
    x = np.zeros(d)
    x[0] = 1.0
    angles = np.zeros(d // 2)
    angles[0] = a
    y = RR.rotate(x, _row(angles), style)
    partner = 1 if style == RR.INTERLEAVED else d // 2
    assert y[0] == math.cos(a) and y[partner] == math.sin(a)
    assert np.count_nonzero(y) == 2


@pytest.mark.parametrize("style", [RR.INTERLEAVED, RR.HALVES])
def test_identity_inverse_and_norm(style):
    rng = np.random.default_rng(3)
    d = 64
    x = rng.standard_normal((5, d))
    np.testing.assert_array_equal(RR.rotate(x, _row(np.zeros(d // 2)), style), x)
    ang = rng.uniform(-10, 10, d // 2)
    y = RR.rotate(x, _row(ang), style)
    back = RR.rotate(y, _row(-ang), style)
    np.testing.assert_allclose(back, x, rtol=0, atol=1e-13)
    i0, i1 = RR.pair_index(d, style)
    np.testing.assert_allclose(y[:, i0] ** 2 + y[:, i1] ** 2, x[:, i0] ** 2 + x[:, i1] ** 2, rtol=1e-13)
    # Composition: turning by a then by b is turning by a + b.
    b = rng.uniform(-10, 10, d // 2)
    np.testing.assert_allclose(RR.rotate(y, _row(b), style), RR.rotate(x, _row(ang + b), style), atol=1e-12)


@pytest.mark.parametrize("style", [RR.INTERLEAVED, RR.HALVES])
def test_scores_depend_on_relative_position(style):
    # With the usual schedule, q.k after turning q to position m and k to
    # position n depends on m - n only.
    rng = np.random.default_rng(4)
    d = 64
    table = W.rope_table(4096, d).double().numpy()
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    for m, n, s in ((10, 3, 1000), (500, 499, 2000), (7, 7, 3000)):
        a = RR.rotate(q, table[m], style) @ RR.rotate(k, table[n], style)
        b = RR.rotate(q, table[m + s], style) @ RR.rotate(k, table[n + s], style)
        assert abs(a - b) <= 1e-5 * (1 + abs(a))  # the table is fp32


def test_positions_of_new_tokens_and_out_of_table():
    rng = np.random.default_rng(5)
    B, H, Q, d = 3, 2, 2, 8
    k = rng.standard_normal((B, Q, d))
    q = rng.standard_normal((B, H, Q, d))
    table = W.rope_table(16, d).double().numpy()
    lens = [5, 1, 17]  # positions [3, 4], [-1, 0], [15, 16]
    ko, qo = RR.rope_step(k, q, table, lens, RR.INTERLEAVED)
    np.testing.assert_array_equal(RR.positions(lens, Q), [[3, 4], [-1, 0], [15, 16]])
    np.testing.assert_allclose(ko[0, 1], RR.rotate(k[0, 1], table[4], RR.INTERLEAVED))
    np.testing.assert_allclose(qo[2, 1, 0], RR.rotate(q[2, 1, 0], table[15], RR.INTERLEAVED))
    assert np.isnan(ko[1, 0]).all() and np.isnan(qo[1, :, 0]).all()  # position -1
    assert np.isnan(ko[2, 1]).all() and np.isnan(qo[2, :, 1]).all()  # position 16 = n_pos
    assert np.isfinite(ko[1, 1]).all()
