"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test names what it pins: a printed fact of the pages (golden fixtures), an
algebraic identity, a closed form, a library routine the path reduces to, or a
brute-force evaluation.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import mla_ref as R

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_case(seed, B=3, H=4, Q=2, Dn=8, Dr=4, Vd=6, Ckv=16, lens=(7, 1, 5), wstd=None):
    rng = np.random.default_rng(seed)
    L = max(lens)
    q_nope = rng.standard_normal((B, H, Q, Dn))
    q_pe = rng.standard_normal((B, H, Q, Dr))
    kv = [rng.standard_normal((L, Ckv)) for _ in range(B)]
    pe = [rng.standard_normal((L, Dr)) for _ in range(B)]
    wstd = (1.0 / math.sqrt(Ckv)) if wstd is None else wstd
    wkv_b = rng.standard_normal((H, Dn + Vd, Ckv)) * wstd
    scale = 1.0 / math.sqrt(Dn + Dr)
    return q_nope, q_pe, kv, pe, wkv_b, list(lens), scale


def _relmax(a, b):
    a = np.asarray(a)
    b = np.asarray(b)
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


# P1 -- printed output shape of the exercise page's demo.
def test_demo_output_shape():
    g = json.load(open(os.path.join(GOLDEN, "decode_step_demo_shape.json")))
    B, H, Dn, Dr, Vd, Lk, Ckv = (g[k] for k in ("B", "H", "Dn", "Dr", "Vd", "Lk", "Ckv"))
    rng = np.random.default_rng(0)
    q_nope = rng.standard_normal((B, H, 1, Dn))
    q_pe = rng.standard_normal((B, H, 1, Dr))
    kv = rng.standard_normal((B, Lk, Ckv))
    pe = rng.standard_normal((B, Lk, Dr))
    wkv_b = rng.standard_normal((H, Dn + Vd, Ckv))
    res = R.decode_nonabsorbed(q_nope, q_pe, kv, pe, wkv_b, [Lk] * B, 1.0 / math.sqrt(Dn + Dr))
    assert list(res["out"].shape) == g["out_shape"]
    assert res["x"].shape == (B, H, 1, Ckv)
    assert np.isfinite(res["out"]).all()


# P2 -- absorption is associativity: absorbed and restore-first forms agree.
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_absorbed_equals_nonabsorbed(seed):
    q_nope, q_pe, kv, pe, w, lens, scale = _rand_case(seed)
    a = R.decode_nonabsorbed(q_nope, q_pe, kv, pe, w, lens, scale, token_block=3)
    b = R.decode_absorbed(q_nope, q_pe, kv, pe, w, lens, scale)
    for k in ("out", "x"):
        assert _relmax(a[k], b[k]) < 1e-10, k
    fin = np.isfinite(b["lse"])
    assert (np.isfinite(a["lse"]) == fin).all()
    assert np.max(np.abs(a["lse"][fin] - b["lse"][fin])) < 1e-10


# P3 -- scalar brute force over every index.
def test_bruteforce_matches():
    q_nope, q_pe, kv, pe, w, lens, scale = _rand_case(7, B=2, H=2, Q=2, Dn=3, Dr=2, Vd=3, Ckv=5,
                                                       lens=(4, 2))
    a = R.decode_nonabsorbed(q_nope, q_pe, kv, pe, w, lens, scale)
    c = R.decode_bruteforce(q_nope, q_pe, kv, pe, w, lens, scale)
    for k in ("out", "x"):
        assert _relmax(a[k], c[k]) < 1e-12, k
    assert np.max(np.abs(a["lse"] - c["lse"])) < 1e-12


# P4 -- probabilities are a distribution, lse is consistent with them.
def test_softmax_rows_sum_to_one():
    q_nope, q_pe, kv, pe, w, lens, scale = _rand_case(3, lens=(9, 3, 6))
    res = R.decode_nonabsorbed(q_nope, q_pe, kv, pe, w, lens, scale, return_probs=True)
    for b, L in enumerate(lens):
        for h in range(q_nope.shape[1]):
            for q in range(q_nope.shape[2]):
                p = res["p"][b][h][q]
                assert len(p) == R.visible_count(L, q_nope.shape[2], q)
                assert abs(p.sum() - 1.0) < 1e-12
                assert (p >= 0).all()
                # x is the p-weighted average of the visible latent rows.
                assert np.allclose(res["x"][b, h, q], p @ kv[b][:len(p)], rtol=0, atol=1e-12)


# P5 -- hidden rows cannot influence any output, bit for bit.
@pytest.mark.parametrize("poison", [np.nan, 1e30, -1e30])
def test_hidden_rows_have_no_influence(poison):
    q_nope, q_pe, kv, pe, w, lens, scale = _rand_case(4, lens=(7, 2, 4))
    base = R.decode_nonabsorbed(q_nope, q_pe, kv, pe, w, lens, scale)
    kv2 = [k.copy() for k in kv]
    pe2 = [p.copy() for p in pe]
    for b, L in enumerate(lens):
        kv2[b][L:] = poison
        pe2[b][L:] = poison
    res = R.decode_nonabsorbed(q_nope, q_pe, kv2, pe2, w, lens, scale)
    for k in ("out", "x", "lse"):
        assert np.array_equal(base[k], res[k]), k


def test_causality_inside_new_tokens():
    # Query 0 of Q=2 must not see the last row; changing it leaves query 0 bitwise unchanged.
    q_nope, q_pe, kv, pe, w, lens, scale = _rand_case(5, lens=(6, 3, 2))
    base = R.decode_nonabsorbed(q_nope, q_pe, kv, pe, w, lens, scale)
    kv2 = [k.copy() for k in kv]
    for b, L in enumerate(lens):
        kv2[b][L - 1] += 100.0
    res = R.decode_nonabsorbed(q_nope, q_pe, kv2, pe, w, lens, scale)
    assert np.array_equal(base["out"][:, :, 0], res["out"][:, :, 0])
    assert not np.allclose(base["out"][:, :, 1], res["out"][:, :, 1])


def test_no_visible_position_convention():
    q_nope, q_pe, kv, pe, w, lens, scale = _rand_case(6, lens=(0, 1, 3))
    res = R.decode_nonabsorbed(q_nope, q_pe, kv, pe, w, lens, scale)
    # Sequence 0 has no rows; sequence 1 has one row, so query 0 of Q=2 sees nothing.
    assert np.all(res["out"][0] == 0) and np.all(res["x"][0] == 0)
    assert np.all(np.isneginf(res["lse"][0]))
    assert np.all(res["x"][1, :, 0] == 0) and np.all(np.isneginf(res["lse"][1, :, 0]))
    assert np.isfinite(res["lse"][1, :, 1]).all()


# P6 -- closed forms.
def test_single_visible_token_closed_form():
    q_nope, q_pe, kv, pe, w, lens, scale = _rand_case(8, Q=1, lens=(1, 1, 1))
    res = R.decode_nonabsorbed(q_nope, q_pe, kv, pe, w, lens, scale)
    Dn = q_nope.shape[-1]
    for b in range(3):
        for h in range(q_nope.shape[1]):
            assert np.allclose(res["x"][b, h, 0], kv[b][0], rtol=0, atol=1e-14)
            assert np.allclose(res["out"][b, h, 0], w[h, Dn:] @ kv[b][0], rtol=0, atol=1e-12)


def test_zero_query_gives_uniform_average():
    q_nope, q_pe, kv, pe, w, lens, scale = _rand_case(9, Q=1, lens=(5, 8, 3))
    q_nope[:] = 0
    q_pe[:] = 0
    res = R.decode_nonabsorbed(q_nope, q_pe, kv, pe, w, lens, scale)
    Dn = q_nope.shape[-1]
    for b, L in enumerate(lens):
        mean = kv[b][:L].mean(0)
        for h in range(q_nope.shape[1]):
            assert np.allclose(res["x"][b, h, 0], mean, rtol=0, atol=1e-13)
            assert np.allclose(res["out"][b, h, 0], w[h, Dn:] @ mean, rtol=0, atol=1e-12)
            assert abs(res["lse"][b, h, 0] - math.log(L)) < 1e-12


def test_identical_rows_give_that_row():
    q_nope, q_pe, kv, pe, w, lens, scale = _rand_case(10, Q=2, lens=(6, 4, 9))
    for b in range(3):
        kv[b][:] = kv[b][0]
    res = R.decode_nonabsorbed(q_nope, q_pe, kv, pe, w, lens, scale)
    for b in range(3):
        assert np.allclose(res["x"][b], np.broadcast_to(kv[b][0], res["x"][b].shape), rtol=0, atol=1e-13)


# P7 -- the absorbed core is MQA with one shared key/value head: a library routine.
def test_core_is_single_kv_head_sdpa():
    q_nope, q_pe, kv, pe, w, lens, scale = _rand_case(11, B=2, H=5, Q=1, lens=(13, 13))
    res = R.decode_nonabsorbed(q_nope, q_pe, kv, pe, w, lens, scale)
    q_lat = np.einsum("bhqd,hdc->bhqc", q_nope, w[:, :q_nope.shape[-1]])
    for b in range(2):
        q = torch.tensor(np.concatenate([q_lat[b], q_pe[b]], -1))  # [H, 1, Ckv+Dr]
        k = torch.tensor(np.concatenate([kv[b], pe[b]], -1))[None]  # [1, L, Ckv+Dr]
        v = torch.tensor(kv[b])[None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            q, k.expand(q.shape[0], -1, -1), v.expand(q.shape[0], -1, -1), scale=scale)
        assert _relmax(res["x"][b], ref.numpy()) < 1e-12


def test_identity_weights_reduce_to_mqa():
    # W_UK = W_UV = I (Dn = Vd = Ckv): MLA is plain MQA on K = [c | k_pe], V = c.
    C = 6
    rng = np.random.default_rng(12)
    B, H, Q, Dr, L = 2, 3, 2, 4, 9
    q_nope = rng.standard_normal((B, H, Q, C))
    q_pe = rng.standard_normal((B, H, Q, Dr))
    kv = rng.standard_normal((B, L, C))
    pe = rng.standard_normal((B, L, Dr))
    w = np.stack([np.concatenate([np.eye(C), np.eye(C)], 0)] * H)
    scale = 0.37
    res = R.decode_nonabsorbed(q_nope, q_pe, kv, pe, w, [L, L], scale)
    for b in range(B):
        q = torch.tensor(np.concatenate([q_nope[b], q_pe[b]], -1))  # [H, Q, C+Dr]
        k = torch.tensor(np.concatenate([kv[b], pe[b]], -1))[None].expand(H, -1, -1)
        v = torch.tensor(kv[b])[None].expand(H, -1, -1)
        mask = torch.tensor([[t <= L - Q + qq for t in range(L)] for qq in range(Q)])
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale)
        assert _relmax(res["out"][b], ref.numpy()) < 1e-12


# P8 -- split-KV merge rule: any partition (with empty parts) reproduces the whole.
@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_lse_merge_of_partition(seed):
    rng = np.random.default_rng(100 + seed)
    L, C, Dr = 37, 12, 4
    c = rng.standard_normal((L, C)) * (1 + 3 * (seed == 3))
    kpe = rng.standard_normal((L, Dr))
    ql = rng.standard_normal(C)
    qp = rng.standard_normal(Dr)
    x_all, lse_all = R.attend_subset(ql, qp, c, kpe, 0.4, range(L))
    labels = rng.integers(0, 5, L)  # five parts, some possibly empty
    parts = [np.nonzero(labels == k)[0] for k in range(5)] + [np.array([], dtype=int)]
    xs, ls = zip(*[R.attend_subset(ql, qp, c, kpe, 0.4, p) for p in parts])
    x, lse = R.lse_combine(np.stack(xs), np.array(ls))
    assert np.max(np.abs(x - x_all)) < 1e-12 * max(1, np.abs(x_all).max())
    assert abs(lse - lse_all) < 1e-12 * max(1, abs(lse_all))
    # Cross-check the subset routine with the full oracle on a one-head case.
    xe, le = R.lse_combine(np.zeros((2, C)), np.array([-np.inf, -np.inf]))
    assert np.all(xe == 0) and np.isneginf(le)


def test_attend_subset_matches_oracle():
    q_nope, q_pe, kv, pe, w, lens, scale = _rand_case(13, B=1, H=1, Q=1, lens=(11,))
    res = R.decode_nonabsorbed(q_nope, q_pe, kv, pe, w, lens, scale)
    ql = R.absorb_q(q_nope, w)[0, 0, 0]
    x, lse = R.attend_subset(ql, q_pe[0, 0, 0], kv[0], pe[0], scale, range(11))
    assert _relmax(res["x"][0, 0, 0], x) < 1e-12
    assert abs(res["lse"][0, 0, 0] - lse) < 1e-12


# P9 (oracle side) -- with every row visible the order of tokens does not matter.
def test_token_permutation_invariance():
    q_nope, q_pe, kv, pe, w, lens, scale = _rand_case(14, Q=1, lens=(10, 10, 10))
    res = R.decode_nonabsorbed(q_nope, q_pe, kv, pe, w, lens, scale)
    perm = np.random.default_rng(1).permutation(10)
    res2 = R.decode_nonabsorbed(q_nope, q_pe, [k[perm] for k in kv], [p[perm] for p in pe], w, lens,
                                scale)
    for k in ("out", "x", "lse"):
        assert _relmax(res[k], res2[k]) < 1e-12


# Absorption and up-projection helpers against explicit matrix products.
def test_absorb_and_up_proj_helpers():
    q_nope, q_pe, kv, pe, w, lens, scale = _rand_case(15)
    Dn = q_nope.shape[-1]
    ql = R.absorb_q(q_nope, w)
    for b in range(q_nope.shape[0]):
        for h in range(q_nope.shape[1]):
            for q in range(q_nope.shape[2]):
                assert np.allclose(ql[b, h, q], w[h, :Dn].T @ q_nope[b, h, q], rtol=0, atol=1e-13)
    x = np.random.default_rng(2).standard_normal(ql.shape)
    o = R.up_proj_v(x, w, Dn)
    assert np.allclose(o[1, 2, 1], w[2, Dn:] @ x[1, 2, 1], rtol=0, atol=1e-13)


# P10 -- cache bytes: one shared row per token whatever the head count; FP4 entry size.
def test_cache_bytes_do_not_depend_on_heads():
    g = json.load(open(os.path.join(GOLDEN, "fp4_entry_bytes.json")))
    from oracle import fp4_ref
    assert fp4_ref.entry_bytes(g["latent_dim"]) == g["entry_bytes"]
    lens = [5, 17, 64]
    row = 512 * 2 + 64 * 2
    assert R.cache_bytes(lens, row) == 86 * 1152
    # The oracle consumes exactly one latent row per token for any number of heads.
    for H in (1, 4, 16):
        q_nope, q_pe, kv, pe, w, _, scale = _rand_case(16, H=H, Q=1, lens=(5, 5, 5))
        res = R.decode_nonabsorbed(q_nope, q_pe, kv, pe, w, [5, 5, 5], scale)
        assert res["x"].shape[1] == H and kv[0].shape == (5, 16)


def test_physical_row_paged_and_contiguous():
    table = [[3, 0], [1, 2]]
    assert R.physical_row(0, 0, 128, 64, table) == 192
    assert R.physical_row(0, 65, 128, 64, table) == 1
    assert R.physical_row(1, 63, 128, 64, table) == 127
    assert R.physical_row(1, 70, 0, 0) == 70
    assert R.physical_row(2, 5, 100, 0) == 205
