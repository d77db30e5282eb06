"""GPU parity of mla_rope_append (RoPE + append + FP4 quantisation in one
pass) against the fp64 RoPE reference, through the C ABI.

The rotated keys (read back from the cache rows) and the rotated queries must
lie within the rounding of the stored dtype of the exact rotation: half an ulp
of the stored value for the final rounding plus the fp32 arithmetic, at most
2^-22 of the pair's length. The latent part of every row must be the bytes
mla_cache_append stores (for FP4: the same codes and scales).
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import rope_ref as RR
from tests import mla_testlib as T

pytestmark = pytest.mark.gpu

CKV, DR = 512, 64


def _ulp(ref: np.ndarray, dtype) -> np.ndarray:
    mant = 7 if dtype == torch.bfloat16 else 23
    a = np.abs(ref)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 2.0 ** (e - mant), 2.0 ** -133)


def _pair_len(x: np.ndarray, style: int) -> np.ndarray:
    """Length of the pair each element belongs to (same shape as x)."""
    i0, i1 = RR.pair_index(x.shape[-1], style)
    n = np.sqrt(x[..., i0] ** 2 + x[..., i1] ** 2)
    out = np.empty_like(x)
    out[..., i0] = n
    out[..., i1] = n
    return out


def _check_rotated(gpu: np.ndarray, exact: np.ndarray, unrotated: np.ndarray, style: int, dtype, name: str):
    fin = np.isfinite(exact)
    assert np.array_equal(np.isnan(gpu), ~fin), f"{name}: NaN pattern differs"
    lim = 0.5 * _ulp(exact, dtype) + 2.0 ** -22 * _pair_len(unrotated, style)
    err = np.abs(gpu - exact)
    T.say(f"  {name}: max err / limit = {float(np.max(np.where(fin, err / lim, 0))):.3f}")
    assert np.all(err[fin] <= lim[fin]), name


def _case(B, Q, H, lens, cap, dtype, n_pos, seed):
    g = torch.Generator().manual_seed(seed)
    c_kv = torch.randn(B, Q, CKV, generator=g).to(dtype)
    k_pe = (3 * torch.randn(B, Q, DR, generator=g)).to(dtype)
    q_pe = torch.randn(B, H, Q, DR, generator=g).to(dtype)
    table = W.rope_table(n_pos, DR)
    return c_kv, k_pe, q_pe, table, torch.tensor(lens, dtype=torch.int32)


@pytest.mark.parametrize("style", [RR.INTERLEAVED, RR.HALVES])
@pytest.mark.parametrize("dtype,Q", [(torch.bfloat16, 1), (torch.bfloat16, 2), (torch.float32, 2)])
def test_rope_append_contiguous(style, dtype, Q):
    o = T.ops()
    B, H, cap = 4, 16, 4096
    lens = [1, 700, 4096, 37][:B]
    c_kv, k_pe, q_pe, table, sl = _case(B, Q, H, lens, cap, dtype, 4096, seed=7 + Q)
    T.say(f"[case] rope_append contiguous style={style} dtype={dtype} Q={Q} lens={lens}")
    bufs = []
    q_gpu = q_pe.cuda()
    for rope in (False, True):
        buf = torch.zeros(B * cap, CKV + DR, dtype=dtype, device="cuda")
        cache = o.LatentCache.combined(buf, CKV, cap)
        if rope:
            o.mla_rope_append(c_kv.cuda(), k_pe.cuda(), cache, sl.cuda(), table.cuda(), style=style, q_pe=q_gpu)
        else:
            o.mla_cache_append(c_kv.cuda(), k_pe.cuda(), cache, sl.cuda())
        torch.cuda.synchronize()
        bufs.append(buf.cpu())
    plain, rot = bufs
    assert torch.equal(plain[:, :CKV].view(torch.int16) if dtype == torch.bfloat16 else plain[:, :CKV].view(torch.int32),
                       rot[:, :CKV].view(torch.int16) if dtype == torch.bfloat16 else rot[:, :CKV].view(torch.int32)), \
        "latent bytes differ from mla_cache_append"
    k_exact, q_exact = RR.rope_step(k_pe.double().numpy(), q_pe.double().numpy(), table.double().numpy(), lens, style)
    pos = RR.positions(lens, Q)
    rows = np.array([[b * cap + pos[b, j] for j in range(Q)] for b in range(B)])
    k_gpu = rot[torch.from_numpy(rows.reshape(-1))][:, CKV:].double().numpy().reshape(B, Q, DR)
    ok = (pos >= 0) & (pos < cap)
    _check_rotated(k_gpu[ok], k_exact[ok], k_pe.double().numpy()[ok], style, dtype, "k_pe in cache")
    _check_rotated(q_gpu.cpu().double().numpy(), q_exact, q_pe.double().numpy(), style, dtype, "q_pe")
    # Rows the step does not write stay as they were (zero).
    written = torch.zeros(B * cap, dtype=torch.bool)
    written[torch.from_numpy(rows[ok])] = True
    assert torch.all(rot[~written] == 0)


def test_rope_append_fp4_paged_and_out_of_table():
    o = T.ops()
    B, Q, H, cap, page = 3, 2, 8, 512, 64
    lens = [130, 2, 512]
    n_pos = 400  # sequence 2's positions 510, 511 lie outside the table
    c_kv, k_pe, q_pe, table, sl = _case(B, Q, H, lens, cap, torch.bfloat16, n_pos, seed=21)
    c_kv = c_kv.float()  # an FP4 cache quantises fp32 or bf16 sources
    T.say(f"[case] rope_append FP4 paged lens={lens} n_pos={n_pos}")
    pages = cap // page
    perm = torch.randperm(B * pages, generator=torch.Generator().manual_seed(3)).to(torch.int32)
    pt = perm.view(B, pages).cuda()
    row_bytes = o.LatentCache.fp4_row_bytes(CKV, DR)
    outs = []
    q_gpu = q_pe.cuda()
    for rope in (False, True):
        buf = torch.zeros(B * cap, row_bytes, dtype=torch.uint8, device="cuda")
        cache = o.LatentCache.fp4(buf, CKV, cap, page_table=pt)
        if rope:
            o.mla_rope_append(c_kv.cuda(), k_pe.cuda(), cache, sl.cuda(), table.cuda(),
                              style=RR.HALVES, q_pe=q_gpu)
        else:
            o.mla_cache_append(c_kv.cuda(), k_pe.cuda(), cache, sl.cuda())
        torch.cuda.synchronize()
        outs.append(buf.cpu())
    plain, rot = outs
    lat_bytes = CKV // 2 + CKV // 16
    assert torch.equal(plain[:, :lat_bytes], rot[:, :lat_bytes]), "FP4 codes / scales differ from mla_cache_append"
    k_exact, q_exact = RR.rope_step(k_pe.double().numpy(), q_pe.double().numpy(), table.double().numpy(), lens,
                                    RR.HALVES)
    pos = RR.positions(lens, Q)
    phys = np.array([[int(perm[b * pages + pos[b, j] // page]) * page + pos[b, j] % page for j in range(Q)]
                     for b in range(B)])
    k_gpu = rot[torch.from_numpy(phys.reshape(-1)).long()][:, lat_bytes:].contiguous().view(torch.bfloat16)
    k_gpu = k_gpu.double().numpy().reshape(B, Q, DR)
    _check_rotated(k_gpu, k_exact, k_pe.double().numpy(), RR.HALVES, torch.bfloat16, "k_pe in FP4 cache")
    _check_rotated(q_gpu.cpu().double().numpy(), q_exact, q_pe.double().numpy(), RR.HALVES, torch.bfloat16, "q_pe")
    assert np.isnan(k_gpu[2]).all() and np.isfinite(k_gpu[:2]).all()


def test_rope_append_without_queries_and_rejects_bad_args():
    o = T.ops()
    B, Q, cap = 2, 1, 128
    lens = [5, 128]
    c_kv, k_pe, _, table, sl = _case(B, Q, 1, lens, cap, torch.bfloat16, 256, seed=5)
    buf = torch.zeros(B * cap, CKV + DR, dtype=torch.bfloat16, device="cuda")
    cache = o.LatentCache.combined(buf, CKV, cap)
    o.mla_rope_append(c_kv.cuda(), k_pe.cuda(), cache, sl.cuda(), table.cuda())
    torch.cuda.synchronize()
    k_exact, _ = RR.rope_step(k_pe.double().numpy(), None, table.double().numpy(), lens, RR.INTERLEAVED)
    got = buf.cpu()[[4, cap + 127], CKV:].double().numpy().reshape(B, Q, DR)
    _check_rotated(got, k_exact, k_pe.double().numpy(), RR.INTERLEAVED, torch.bfloat16, "k_pe (no queries)")
    with pytest.raises(o.MLAError):
        o.mla_rope_append(c_kv.cuda(), k_pe.cuda(), cache, sl.cuda(), table.cuda(), style=7)
    with pytest.raises(o.MLAError):
        o.mla_rope_append(c_kv.cuda(), k_pe.cuda(), cache, sl.cuda(), table[:0].cuda())
