"""Seeded synthetic workload generators: determinism and structure."""
import numpy as np
import torch

import workloads as W


def _small(name, **kw):
    w = W.WORKLOADS[name]
    if w.lk_range is None and w.lens is None:
        return w.with_(B=2, lk=300, **kw)
    return W.reduced(w, 3, [700, 65, 130])


def test_generation_is_deterministic():
    for name in W.WORKLOAD_ORDER:
        w = _small(name)
        a = W.generate(w).sha256()
        b = W.generate(w).sha256()
        assert a == b, name


def test_shapes_and_dtypes():
    for name in W.WORKLOAD_ORDER:
        w = _small(name)
        inp = W.generate(w)
        T = int(inp.seq_lens.sum())
        assert inp.q_nope.shape == (w.B, w.H, w.Q, w.Dn)
        assert inp.q_pe.shape == (w.B, w.H, w.Q, w.Dr)
        assert inp.latent.shape == (T, w.Ckv) and inp.rope.shape == (T, w.Dr)
        assert inp.wkv_b.shape == (w.H, w.Dn + w.Vd, w.Ckv)
        if w.dtype == "fp4":
            assert inp.latent.dtype == torch.float32 and inp.rope.dtype == torch.bfloat16
        else:
            assert inp.latent.dtype == W.storage_dtype(w)


def test_ragged_lengths_in_range_and_pages_permuted():
    w = W.WORKLOADS["ragged_paged_bf16"]
    g = torch.Generator().manual_seed(w.seed)
    lens = W._lengths(w, g)
    assert lens.numel() == 64 and int(lens.min()) >= 512 and int(lens.max()) <= 32768
    small = W.reduced(w, 4, [100, 64, 1, 129])
    inp = W.generate(small)
    pl = W.place(inp)
    npages = sum((l + 63) // 64 for l in [100, 64, 1, 129])
    assert sorted(inp.page_perm.tolist()) == list(range(npages))
    assert len(set(pl.rows.tolist())) == pl.rows.numel() == 294
    assert int(pl.rows.max()) < pl.n_rows
    # Every logical row of a sequence sits in one of that sequence's own pages.
    off = 0
    for b, L in enumerate([100, 64, 1, 129]):
        pages = set(pl.page_table[b, :(L + 63) // 64].tolist())
        assert {int(r) // 64 for r in pl.rows[off:off + L]} <= pages
        off += L


def test_spikes():
    w = W.WORKLOADS["long_splitkv_bf16"].with_(lk=1000, B=2)
    inp = W.generate(w)
    assert inp.spike_rows.numel() == 2 * 10
    base = W.generate(w.with_(spike_frac=0.0))
    # Spiked rows are exactly x8 of the unspiked draw; all other rows are identical.
    r = inp.spike_rows
    assert torch.equal(inp.latent[r].float(), base.latent[r].float() * 8)
    mask = torch.ones(inp.latent.shape[0], dtype=torch.bool)
    mask[r] = False
    assert torch.equal(inp.latent[mask], base.latent[mask])


def test_weight_std():
    inp = W.generate(W.WORKLOADS["tiny_f32"])
    std = float(inp.wkv_b.float().std())
    assert abs(std - 1 / np.sqrt(512)) < 0.002
    assert float(inp.q_nope.std()) > 0.9


def test_contiguous_placement_and_scatter():
    w = W.WORKLOADS["dsv3_bf16"].with_(B=2, lk=5)
    inp = W.generate(w)
    pl = W.place(inp, capacity=8)
    assert pl.rows.tolist() == [0, 1, 2, 3, 4, 8, 9, 10, 11, 12]
    phys = W.combined_rows(inp.latent, inp.rope, pl)
    assert phys.shape == (16, 576)
    assert torch.equal(phys[9, :512], inp.latent[6]) and torch.isnan(phys[5].float()).all()
