"""GPU parity of the DeepSeek-V4.1-Flash form of latent attention against the
fp64 reference oracle/v4_ref.py, through the C ABI: mla_rope_append in
latent-tail mode (the cache and the query rows), mla_decode_attn, then
mla_sink_inverse_rope (sink column and inverse rotation of x's tail); on the
form's own rows (one 512-wide latent, no RoPE section: 1024 B bf16, 288 B
FP4) and on DeepSeek-V3 rows with an all-zero RoPE slot and q_pe; and of the
grouped output projection that follows it (mla_grouped_out_proj against
v4_ref.grouped_out_proj)."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import fp4_ref as F
from oracle import rope_ref as RR
from oracle import v4_ref as V
from tests import mla_testlib as T

pytestmark = pytest.mark.gpu

CKV, DR = 512, 64


def _inputs(B, H, Q, lens, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, H, Q, CKV, generator=g).to(dtype)
    lat = [torch.randn(n, CKV, generator=g).to(dtype) for n in lens]
    sinks = (2 * torch.randn(H, generator=g)).float()
    return q, lat, sinks


def _run_v4(o, q, lat, lens, sinks, table, style, dtype, Q, workgroups=0, own_rows=False):
    B, H = q.shape[0], q.shape[1]
    cap = max(64, -(-max(lens) // 64) * 64)
    if own_rows:
        # The form's own rows: the 512-wide latent alone, no RoPE section.
        buf = torch.full((B * cap, CKV), float("nan"), dtype=dtype, device="cuda")
        cache = o.LatentCache.latent_only(buf, CKV, cap)
    else:
        buf = torch.zeros(B * cap, CKV + DR, dtype=dtype, device="cuda")
        cache = o.LatentCache.combined(buf, CKV, cap)
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    n = max(lens)
    hist = torch.zeros(B, n, CKV, dtype=dtype)
    for b, rows in enumerate(lat):
        if len(rows):
            hist[b, n - len(rows):] = rows
    tab = table.cuda()
    # Every token (right-aligned: token j of a length-L sequence lands at L - n + j).
    o.mla_rope_append(hist.cuda(), None, cache, sl, tab, style=style, latent_tail=True)
    # The step: its Q new tokens again (same rows, same values) and the query rows.
    new = torch.stack([hist[b, n - Q:] for b in range(B)]).contiguous()
    qg = q.cuda().contiguous()
    o.mla_rope_append(new.cuda(), None, cache, sl, tab, style=style, q_pe=qg, latent_tail=True)
    x = torch.empty(B, H, Q, CKV, dtype=dtype, device="cuda")
    lse = torch.empty(B, H, Q, dtype=torch.float32, device="cuda")
    zero_pe = None if own_rows else torch.zeros(B, H, Q, DR, dtype=dtype, device="cuda")
    scale = 1.0 / math.sqrt(CKV)
    o.mla_decode_attn(qg, zero_pe, cache, sl, n, scale, x, lse, workgroups=workgroups)
    o.mla_sink_inverse_rope(x, lse, sl, sinks.cuda(), tab, style)
    torch.cuda.synchronize()
    return x, lse, scale, buf


@pytest.mark.parametrize("style", [RR.INTERLEAVED, RR.HALVES])
@pytest.mark.parametrize("dtype,Q,workgroups,own_rows", [(torch.bfloat16, 1, 0, False), (torch.bfloat16, 2, 7, False),
                                                         (torch.float32, 2, 0, False), (torch.bfloat16, 1, 0, True),
                                                         (torch.bfloat16, 2, 5, True)])
def test_v4_form_against_oracle(style, dtype, Q, workgroups, own_rows):
    o = T.ops()
    B, H = 3, 64  # the V4.1-Flash form has 64 query heads over one latent
    lens = [300, 2, 129]
    q, lat, sinks = _inputs(B, H, Q, lens, dtype, seed=31 + Q)
    table = W.rope_table(512, DR)
    T.say(f"[case] v4 form style={style} dtype={dtype} Q={Q} lens={lens} workgroups={workgroups} "
          f"own_rows={own_rows}")
    x, lse, scale, _ = _run_v4(o, q, lat, lens, sinks, table, style, dtype, Q, workgroups, own_rows)
    ref = V.decode_v4(q.double().numpy(), [r.double().numpy() for r in lat], lens, table.double().numpy(), style,
                      scale, sinks.double().numpy(), r=DR)
    tol = T.TOL["f32" if dtype == torch.float32 else "bf16"]
    T.assert_close(T.to64(x), ref["x"], tol, "x")
    T.assert_lse_close(T.to64(lse), ref["lse"], tol)


def test_v4_fp4_tail_quantises_the_rotated_latent():
    # The FP4 cache in latent-tail mode holds exactly the codes and scales that
    # quantising the fp32 latent-tail rows would give (same rotation, then the
    # FP4 codec), and a zero RoPE slot.
    o = T.ops()
    B, n, cap = 2, 70, 128
    lens = [70, 33]
    g = torch.Generator().manual_seed(9)
    hist = torch.randn(B, n, CKV, generator=g)
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    table = W.rope_table(256, DR).cuda()
    for style in (RR.INTERLEAVED, RR.HALVES):
        f32 = torch.zeros(B * cap, CKV + DR, dtype=torch.float32, device="cuda")
        o.mla_rope_append(hist.cuda(), None, o.LatentCache.combined(f32, CKV, cap), sl, table, style=style,
                          latent_tail=True)
        row_bytes = o.LatentCache.fp4_row_bytes(CKV, DR)
        a = torch.zeros(B * cap, row_bytes, dtype=torch.uint8, device="cuda")
        o.mla_rope_append(hist.cuda(), None, o.LatentCache.fp4(a, CKV, cap), sl, table, style=style,
                          latent_tail=True)
        # The rotated rows, read back, appended as they are into a second FP4 cache.
        rot = torch.zeros(B, n, CKV, dtype=torch.float32, device="cuda")
        for b in range(B):
            rot[b, n - lens[b]:] = f32[b * cap: b * cap + lens[b], :CKV]
        bref = torch.zeros_like(a)
        o.mla_cache_append(rot, torch.zeros(B, n, DR, dtype=torch.bfloat16, device="cuda"),
                           o.LatentCache.fp4(bref, CKV, cap), sl)
        torch.cuda.synchronize()
        assert torch.equal(a.cpu(), bref.cpu()), f"style {style}"
        assert torch.all(f32[:, CKV:] == 0)


@pytest.mark.parametrize("Q,paged,workgroups", [(1, False, 0), (2, True, 0), (2, False, 9)])
def test_fp4_288_byte_rows_against_oracle(Q, paged, workgroups):
    # Attention over the form's FP4 entry (codes | scales, 288 B, no RoPE
    # section): the rows go in through mla_cache_append (the codec pinned bit
    # for bit elsewhere); the oracle quantises the same fp32 rows with its own
    # codec, and with an identity rotation table decode_v4 is plain latent
    # attention over the dequantised rows.
    o = T.ops()
    B, H = 3, 64
    lens = [300, 33, 129]
    g = torch.Generator().manual_seed(40 + Q)
    q = torch.randn(B, H, Q, CKV, generator=g).to(torch.bfloat16)
    lat = [torch.randn(n, CKV, generator=g) for n in lens]
    n = max(lens)
    cap = -(-n // 64) * 64
    row = o.LatentCache.fp4_row_bytes(CKV, 0)
    assert row == 288
    pt = None
    if paged:
        pages = cap // 64
        perm = torch.randperm(B * pages, generator=g).to(torch.int32)
        pt = perm.reshape(B, pages).cuda()
    buf = torch.full((B * cap, row), 0xFF, dtype=torch.uint8, device="cuda")
    cache = o.LatentCache.fp4(buf, CKV, cap, page_table=pt, rope=False)
    hist = torch.zeros(B, n, CKV)
    for b, rows in enumerate(lat):
        hist[b, n - len(rows):] = rows
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    o.mla_cache_append(hist.cuda(), None, cache, sl)
    x = torch.empty(B, H, Q, CKV, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B, H, Q, dtype=torch.float32, device="cuda")
    scale = 1.0 / math.sqrt(CKV)
    T.say(f"[case] v4 fp4 288-byte rows Q={Q} paged={paged} workgroups={workgroups}")
    o.mla_decode_attn(q.cuda(), None, cache, sl, n, scale, x, lse, workgroups=workgroups)
    torch.cuda.synchronize()
    keys = []
    for rows in lat:
        codes, scs = F.quantize_rows_fast(rows.numpy())
        keys.append(F.dequantize_rows(codes, scs))
    ident = np.concatenate([np.ones((n, DR // 2)), np.zeros((n, DR // 2))], axis=1)
    ref = V.decode_v4(q.double().numpy(), keys, lens, ident, RR.HALVES, scale, None, r=DR)
    T.assert_close(T.to64(x), ref["x"], T.TOL["bf16"], "x")
    T.assert_lse_close(T.to64(lse), ref["lse"], T.TOL["bf16"])


def _v4_samples(B, H, n, seed):
    rng = np.random.default_rng(seed)
    pairs = [(0, 0), (B - 1, H - 1)]
    while len(pairs) < n:
        p = (int(rng.integers(0, B)), int(rng.integers(0, H)))
        if p not in pairs:
            pairs.append(p)
    return pairs


@pytest.mark.parametrize("fp4", [False, True])
def test_v4_full_size_sampled(fp4):
    # The size and launch the benchmark times for the form (B=32, 64 heads,
    # 4096 tokens each, Q=1, the form's own rows, default split): bf16 rows
    # through the whole chain (latent-tail RoPE append, attention, sink and
    # inverse rotation); 288-byte FP4 rows through the plain append and the
    # attention, against decode_v4 over the oracle codec's rows with an
    # identity rotation. Eight (sequence, head) pairs against the fp64 oracle.
    o = T.ops()
    B, H, Q, L = 32, 64, 1, 4096
    lens = [L] * B
    q, lat, sinks = _inputs(B, H, Q, lens, torch.float32 if fp4 else torch.bfloat16, seed=77)
    q = q.to(torch.bfloat16)
    scale = 1.0 / math.sqrt(CKV)
    T.say(f"[case] v4 full size fp4={fp4}")
    if not fp4:
        table = W.rope_table(L, DR)
        x, lse, scale, _ = _run_v4(o, q, lat, lens, sinks, table, RR.INTERLEAVED, torch.bfloat16, Q, 0, True)
    else:
        row = o.LatentCache.fp4_row_bytes(CKV, 0)
        buf = torch.full((B * L, row), 0xFF, dtype=torch.uint8, device="cuda")
        cache = o.LatentCache.fp4(buf, CKV, L, rope=False)
        sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
        o.mla_cache_append(torch.stack(lat).cuda(), None, cache, sl)
        x = torch.empty(B, H, Q, CKV, dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(B, H, Q, dtype=torch.float32, device="cuda")
        o.mla_decode_attn(q.cuda(), None, cache, sl, L, scale, x, lse)
        torch.cuda.synchronize()
    assert torch.isfinite(x.float()).all()
    xs, ls = T.to64(x), T.to64(lse)
    for b, h in _v4_samples(B, H, 8, seed=123 + int(fp4)):
        T.say(f"  sample b={b} h={h}")
        qs = q[b:b + 1, h:h + 1].double().numpy()
        if not fp4:
            ref = V.decode_v4(qs, [lat[b].double().numpy()], [L], W.rope_table(L, DR).double().numpy(),
                              RR.INTERLEAVED, scale, sinks[h:h + 1].double().numpy(), r=DR)
        else:
            codes, scs = F.quantize_rows_fast(lat[b].numpy())
            ident = np.concatenate([np.ones((L, DR // 2)), np.zeros((L, DR // 2))], axis=1)
            ref = V.decode_v4(qs, [F.dequantize_rows(codes, scs)], [L], ident, RR.HALVES, scale, None, r=DR)
        T.assert_close(xs[b:b + 1, h:h + 1], ref["x"], T.TOL["bf16"], f"x b={b} h={h}")
        T.assert_lse_close(ls[b:b + 1, h:h + 1], ref["lse"], T.TOL["bf16"])


def test_sink_inverse_rope_positions_outside_table_and_no_sink():
    o = T.ops()
    B, H, Q = 2, 4, 2
    g = torch.Generator().manual_seed(13)
    x0 = torch.randn(B, H, Q, CKV, generator=g).to(torch.bfloat16)
    lse0 = torch.randn(B, H, Q, generator=g)
    lens = [10, 40]  # positions [8, 9] and [38, 39]; the table has 39 rows
    table = W.rope_table(39, DR)
    x = x0.cuda()
    lse = lse0.cuda()
    o.mla_sink_inverse_rope(x, lse, torch.tensor(lens, dtype=torch.int32, device="cuda"), None, table.cuda(),
                            RR.HALVES)
    torch.cuda.synchronize()
    xr = x.cpu().double().numpy()
    assert torch.equal(lse.cpu(), lse0), "lse changes only with sinks"
    assert np.isnan(xr[1, :, 1, -DR:]).all() and np.isfinite(xr[1, :, 1, :-DR]).all()
    assert np.array_equal(xr[..., :-DR], x0.double().numpy()[..., :-DR]), "the head of x is untouched"
    ref = V.rotate_tail(x0[0, :, 1].double().numpy(), table[9].double().numpy(), RR.HALVES, DR, inverse=True)
    T.assert_close(xr[0, :, 1], ref, 1e-2, "tail turned back")


@pytest.mark.parametrize("B,H,Q,G,N", [(3, 64, 2, 8, 1024), (20, 16, 2, 4, 64), (32, 64, 1, 8, 1024)])
def test_grouped_out_proj_against_oracle(B, H, Q, G, N):
    o = T.ops()
    g = torch.Generator().manual_seed(B * 100 + H)
    x = torch.randn(B, H, Q, CKV, generator=g).to(torch.bfloat16)
    w = (torch.randn(G, N, (H // G) * CKV, generator=g) / math.sqrt((H // G) * CKV)).to(torch.bfloat16)
    T.say(f"[case] grouped W_O B={B} H={H} Q={Q} G={G} N={N}")
    out = torch.full((B, Q, G * N), float("nan"), dtype=torch.bfloat16, device="cuda")
    o.mla_grouped_out_proj(x.cuda(), w.cuda(), out)
    torch.cuda.synchronize()
    ref = V.grouped_out_proj(x.double().numpy(), w.double().numpy())
    T.assert_close(T.to64(out), ref, T.TOL["bf16"], "grouped W_O")


def test_grouped_out_proj_rejects_bad_shapes():
    o = T.ops()
    x = torch.zeros(1, 6, 1, CKV, dtype=torch.bfloat16, device="cuda")
    w = torch.zeros(4, 32, 1024, dtype=torch.bfloat16, device="cuda")  # 4 does not divide 6
    out = torch.zeros(1, 1, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(o.MLAError):
        o.mla_grouped_out_proj(x, w, out)
