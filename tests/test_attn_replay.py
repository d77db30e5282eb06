"""CPU replay of the matrix-core attention kernel's address arithmetic.

The bf16 / FP4 attention kernel and its merge compute every global address
from host-visible values (lengths, page tables, strides, the split count).
This test restates that arithmetic in plain Python -- block to (run, row
group) mapping, the run plan, the tile cursor, each tile copy's buffer
descriptor and per-lane offsets, the query staging, the partial slots, the x
rows and the merge's reads -- and checks that every access the hardware would
make lies inside its allocation, for the lengths of the case that once
faulted the GPU ([64, 128, 4096], under an earlier form of the tile copies)
and for the shapes the GPU parity tests run. It runs no kernel.

A buffer load with an LDS destination reads only lanes whose offset is below
the descriptor's byte count (the rest read as zero without touching memory);
an access that does happen reads 16 bytes at descriptor base + offset.
"""
import math

import numpy as np
import pytest

import workloads as W

TILE = 32
ROWS = 64
PAGE = 64
CUS = 256


def swz(t):
    return (-(t & 1) & 5) ^ (-((t >> 1) & 1) & 12) ^ (-((t >> 2) & 1) & 3) ^ (-((t >> 3) & 1) & 2)


class Alloc:
    """A named byte interval [lo, hi); every access is checked against it."""

    def __init__(self, name, lo, nbytes):
        self.name, self.lo, self.hi = name, lo, lo + nbytes
        self.touched = 0

    def check(self, addr, n, what):
        """Accesses [addr, addr + n) for every addr in `addr` (an int or an array)."""
        a = np.asarray(addr, dtype=np.int64)
        if a.size == 0:
            return
        lo, hi = int(a.min()), int(a.max()) + n
        assert self.lo <= lo and hi <= self.hi, \
            f"{what}: [{lo}, {hi}) outside {self.name} [{self.lo}, {self.hi})"
        self.touched += int(a.size)


def default_workgroups(B, HQ, max_len):
    groups = -(-HQ // ROWS)
    max_tiles = B * -(-max(max_len, 0) // TILE)
    w = max(1, CUS // groups)
    return min(w, max(1, max_tiles // 4))


LANES = np.arange(64)


def buffer_reads(alloc, base, num_records, offsets, width, what):
    off = np.asarray(offsets, dtype=np.int64)
    alloc.check(base + off[off < num_records], width, what)


def latent_off(ls):
    """Per-lane offsets of the 8 latent-row pieces of the 4 copying waves (tokens 0..31)."""
    t = np.arange(TILE)[:, None]
    return (t * ls + ((LANES ^ np.vectorize(swz)(t)) << 4)).ravel()


def rope_off(rs):
    d = np.arange(4)[:, None]
    return ((8 * d + (LANES & 7)) * rs + ((LANES >> 3) << 4)).ravel()


def fp4_codes_off(cs):
    dh = np.arange(8)[:, None]  # 4 waves x 2 halves: tokens 4*dh + lane/16
    return ((4 * dh + (LANES >> 4)) * cs + ((LANES & 15) << 4)).ravel()


def fp4_rope_off(rs):
    d = np.arange(4)[:, None]
    return ((8 * d + (LANES >> 3)) * rs + ((LANES & 7) << 4)).ravel()


def fp4_scale_off(ss):
    d = np.arange(4)[:, None]
    ln = np.arange(16)
    return ((8 * d + (ln >> 1)) * ss + ((ln & 1) << 4)).ravel()


def replay(B, H, Q, lens, fp4=False, paged=False, page_table=None, num_rows=None, capacity=None,
           workgroups=0, lo=True):
    HQ = H * Q
    G = -(-HQ // ROWS)
    max_len = max(lens) if lens else 0
    W_ = workgroups or default_workgroups(B, HQ, max_len)
    cap = capacity if capacity is not None else max(max_len, 1)
    if num_rows is None:
        num_rows = B * cap
    base = 1 << 40  # fake addresses, far apart
    if fp4:
        row_b = 416
        cache = Alloc("fp4 cache", base, num_rows * row_b)
        lat, scl, rope = base, base + 256, base + 288
        ls = ss = rs = row_b
    else:
        row_b = 1152
        cache = Alloc("cache", base, num_rows * row_b)
        lat, rope = base, base + 1024
        ls = rs = row_b
    qlat = Alloc("q_lat", 2 << 40, B * HQ * 1024)
    qlo = Alloc("q_lat_lo", 3 << 40, B * HQ * 1024)
    qpe = Alloc("q_pe", 4 << 40, B * HQ * 128)
    xo = Alloc("x", 5 << 40, B * HQ * 1024)
    lse = Alloc("lse", 6 << 40, B * HQ * 4)
    part_rows = G * 2 * W_ * ROWS
    part_x = Alloc("partial x", 7 << 40, part_rows * 512 * 2)
    part_scale = Alloc("partial scales", part_x.hi, part_rows * 16)
    part_lse = Alloc("partial lse", part_scale.hi, part_rows * 4)
    plan = Alloc("run plan", part_lse.hi, (B + 1) * 4)
    if paged:
        assert num_rows % PAGE == 0

    L = [min(max(v, 0), cap) for v in lens]
    ntiles = [-(-v // TILE) for v in L]
    total = sum(ntiles)
    per = -(-total // W_)
    cum = [0]
    for n in ntiles:
        cum.append(cum[-1] + n)

    def tile_row0(b, tile):
        t0 = tile * TILE
        if not paged:
            return b * cap + t0, False
        page = int(page_table[b][t0 // PAGE])
        p0 = page * PAGE
        if page < 0 or p0 + PAGE > num_rows:
            return 0, True
        return p0 + t0 % PAGE, False

    def walk(b, tile, count):
        """The tile cursor: (b, tile) of `count` consecutive run tiles."""
        out = []
        for _ in range(count):
            out.append((b, tile))
            tile += 1
            if tile >= ntiles[b]:
                tile = 0
                b += 1
                while b < B and ntiles[b] == 0:
                    b += 1
        return out

    blocks = -(-W_ // 8) * 8 * G
    for bid in range(blocks):
        xcd, q8 = bid & 7, bid >> 3
        g = q8 % G
        wg = xcd * (-(-W_ // 8)) + q8 // G
        if wg >= W_:
            continue
        if wg == 0 and g == 0:
            for b in range(B + 1):
                plan.check(plan.lo + 4 * b, 4, "plan write")
        start, end = wg * per, min(total, wg * per + per)
        if start >= end:
            continue
        b0 = next(b for b in range(B) if start < cum[b + 1])
        tiles = walk(b0, start - cum[b0], end - start)
        # score waves: query staging of the run's first sequence, the low part, later sequences
        grow0 = b0 * HQ + g * ROWS
        nrows = min(ROWS, HQ - g * ROWS)
        r = np.arange(ROWS)[:, None]
        buffer_reads(qlat, qlat.lo + grow0 * 1024, nrows * 1024, (r * 1024 + ((LANES ^ (r & 15)) << 4)).ravel(), 16,
                     "query staging")
        c = np.arange(8)[:, None]
        buffer_reads(qpe, qpe.lo + grow0 * 128, nrows * 128, (LANES * 128 + c * 16).ravel(), 16, "q_pe staging")
        seqs = []
        for (b, tile) in tiles:
            if not seqs or seqs[-1] != b:
                seqs.append(b)
        rl = np.arange(ROWS)
        row_c = np.where(g * ROWS + rl < HQ, g * ROWS + rl, 0)[:, None]
        g4 = np.arange(4)[None, :, None]
        ks16 = np.arange(16)[None, None, :]
        ks2 = np.arange(2)[None, None, :]
        for k, b in enumerate(seqs):
            grow = (b * HQ + row_c)[:, :, None]
            if lo:
                qlo.check(qlo.lo + grow * 1024 + 2 * (8 * g4 + 32 * ks16), 16, "q_lat_lo load")
            if k > 0:
                qlat.check(qlat.lo + grow * 1024 + 2 * (8 * g4 + 32 * ks16), 16, "q_lat load")
                qpe.check(qpe.lo + grow * 128 + 2 * (8 * g4 + 32 * ks2), 16, "q_pe load")
        # P.V waves: tile copies
        for (b, tile) in tiles:
            row0, bad = tile_row0(b, tile)
            valid = 1 if bad else min(TILE, L[b] - tile * TILE)
            assert 1 <= valid <= TILE
            if fp4:
                buffer_reads(cache, lat + row0 * ls, valid * ls, fp4_codes_off(ls), 16, "fp4 codes")
                buffer_reads(cache, rope + row0 * rs, valid * rs, fp4_rope_off(rs), 16, "fp4 rope")
                buffer_reads(cache, scl + row0 * ss, valid * ss, fp4_scale_off(ss), 16, "fp4 scales")
            else:
                buffer_reads(cache, lat + row0 * ls, valid * ls, latent_off(ls), 16, "latent rows")
                buffer_reads(cache, rope + row0 * rs, valid * rs, rope_off(rs), 16, "rope group")
        # P.V waves: segment ends
        first = True
        seg_lo = tiles[0][1]
        for i, (b, tile) in enumerate(tiles):
            last_of_run = i == len(tiles) - 1
            if tile == ntiles[b] - 1 or last_of_run:
                whole = seg_lo == 0 and tile == ntiles[b] - 1
                slot = 2 * wg + (0 if first else 1)
                prow0 = (g * 2 * W_ + slot) * ROWS
                xrow0 = b * HQ + g * ROWS
                r = np.arange(min(ROWS, HQ - g * ROWS))
                if whole:
                    xo.check(xo.lo + (xrow0 + r) * 1024, 1024, "x row")
                    lse.check(lse.lo + (xrow0 + r) * 4, 4, "lse")
                else:
                    part_x.check(part_x.lo + (prow0 + r) * 1024, 1024, "partial row")
                    part_scale.check(part_scale.lo + (prow0 + r) * 16, 16, "partial scales")
                    part_lse.check(part_lse.lo + (prow0 + r) * 4, 4, "partial lse")
                first = False
                seg_lo = 0
    # merge: every sequence's run-plan entries (read with its length, empty
    # sequences included), then each split sequence's partial rows
    for b in range(B):
        plan.check(plan.lo + 4 * b, 4, "merge plan read")
        plan.check(plan.lo + 4 * B, 4, "merge plan end read")
        nb = ntiles[b]
        if nb == 0:
            continue
        i_first, i_last = cum[b] // per, (cum[b] + nb - 1) // per
        if i_first == i_last:
            continue
        row = np.arange(HQ)
        g, rl = row // ROWS, row % ROWS
        for i in range(i_first, i_last + 1):
            slot = 2 * i + (1 if (i == i_first and cum[b] != i_first * per) else 0)
            prow = (g * 2 * W_ + slot) * ROWS + rl
            part_x.check(part_x.lo + prow * 1024, 1024, "merge partial read")
            part_scale.check(part_scale.lo + prow * 16, 16, "merge scale read")
            part_lse.check(part_lse.lo + prow * 4, 4, "merge lse read")
    assert cache.touched > 0
    return cache.touched


def _paged_setup(name, lens, seed=0):
    w = W.reduced(W.WORKLOADS[name], len(lens), lens, seed=seed).with_(paged=True)
    inp = W.generate(w)
    pl = W.place(inp)
    return pl.page_table.tolist(), pl.n_rows, pl.capacity


FAULTED = [64, 128, 4096]


@pytest.mark.parametrize("workgroups", [0, 1, 2, 3, 5, 7, 16, 31, 40, 64, 128, 200])
@pytest.mark.parametrize("lo", [True, False])
def test_faulted_lengths_every_access_in_bounds(workgroups, lo):
    # The case as the parity test builds it: contiguous cache, capacity = the longest sequence.
    assert replay(3, 128, 1, FAULTED, workgroups=workgroups, lo=lo) > 0


@pytest.mark.parametrize("lens,H,Q,fp4,paged", [
    ([1000, 777, 337], 128, 1, False, False),
    ([100, 64, 1, 129, 700], 128, 1, False, True),
    ([3000, 2500], 128, 1, False, False),
    ([0, 1, 2, 190], 128, 2, False, False),
    ([333, 64], 48, 2, False, False),
    ([300, 2, 1, 130], 128, 2, True, False),
    ([700, 33, 1, 260], 128, 2, True, False),
    ([200, 65, 64], 128, 2, True, True),
    ([300, 129, 0, 4096], 40, 1, False, False),
    ([70, 129], 128, 1, False, False),
    ([64, 64, 64, 64], 16, 1, False, True),
    ([4096] * 32, 128, 1, False, False),
])
@pytest.mark.parametrize("workgroups", [0, 1, 3, 40, 200])
def test_parity_shapes_every_access_in_bounds(lens, H, Q, fp4, paged, workgroups):
    if paged:
        table, n_rows, cap = _paged_setup("dsv3_bf16", lens)
        replay(len(lens), H, Q, lens, fp4=fp4, paged=True, page_table=table, num_rows=n_rows, capacity=cap,
               workgroups=workgroups)
    else:
        replay(len(lens), H, Q, lens, fp4=fp4, workgroups=workgroups)


def test_bad_page_index_reads_one_row_of_the_pool():
    # A page index past the pool: the copy's descriptor covers row 0 only (valid = 1).
    table = [[0, 99]]
    assert replay(1, 16, 1, [100], paged=True, page_table=table, num_rows=64, capacity=128) > 0


def test_replay_catches_an_overrun():
    # The checker itself: a cache one page short of the lengths must fail.
    with pytest.raises(AssertionError):
        replay(2, 16, 1, [64, 64], num_rows=64, capacity=64)


def test_default_split_matches_the_library_policy():
    # One workgroup per compute unit over the row groups, at least 4 tiles each.
    assert default_workgroups(32, 128, 4096) == 128
    assert default_workgroups(3, 128, 4096) == 96
    assert default_workgroups(128, 256, 8192) == 64
    assert math.isclose(default_workgroups(1, 16, 256), 2)
