"""The C-ABI library loads, exports every symbol its header declares, and rejects
invalid arguments on the host before any HIP call (no GPU needed)."""
import ctypes
import os
import re

import pytest

from mla_latent_kv_08_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_symbols():
    text = open(os.path.join(ROOT, "include", "mla.h")).read()
    return sorted(set(re.findall(r"MLA_API\s+[\w\s\*]+?\b(mla_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from mla_latent_kv_08_amd import build
        build.build()
    return _lib.load()


def test_exports_match_header(lib):
    syms = _header_symbols()
    assert len(syms) >= 7, syms
    assert sorted(_lib.EXPORTS) == syms
    for s in syms:
        assert getattr(lib, s) is not None


def test_only_c_abi_is_exported(lib):
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True)
    names = {line.split()[-1] for line in out.stdout.splitlines() if " T " in line}
    assert set(_header_symbols()) <= names
    assert all(n.startswith("mla_") or n.startswith("_") for n in names), names


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4):
        assert lib.mla_status_string(code)
    assert lib.mla_status_string(-99) == b"unknown status"


def _dims(**kw):
    d = dict(batch=2, heads=128, q_len=1, d_nope=128, d_rope=64, d_v=128, d_latent=512)
    d.update(kw)
    return _lib.MlaDims(**d)


def _cache(**kw):
    c = dict(latent_dtype=_lib.MLA_BF16, rope_dtype=_lib.MLA_BF16, latent=0x10000, latent_scale=None,
             rope=0x10400, latent_stride=1152, scale_stride=0, rope_stride=1152, num_rows=2 * 4096,
             page_size=0, capacity=4096, page_table=None, page_table_stride=0, reserved=0)
    c.update(kw)
    return _lib.MlaKvCache(**c)


P = 0x20000  # a 16-byte aligned fake device address; never dereferenced on these paths


def test_absorb_validation(lib):
    byref = ctypes.byref
    assert lib.mla_absorb_q(None, 1, P, P, P, None, None) == _lib.MLA_ERR_INVALID_ARG
    assert lib.mla_absorb_q(byref(_dims()), 1, None, P, P, None, None) == _lib.MLA_ERR_INVALID_ARG
    assert lib.mla_absorb_q(byref(_dims()), 1, P + 2, P, P, None, None) == _lib.MLA_ERR_INVALID_ARG
    assert lib.mla_absorb_q(byref(_dims()), 1, P, P, P, P + 2, None) == _lib.MLA_ERR_INVALID_ARG
    # fp32 q_lat has no low part.
    assert lib.mla_absorb_q(byref(_dims()), 0, P, P, P, P, None) == _lib.MLA_ERR_UNSUPPORTED
    assert lib.mla_absorb_q(byref(_dims(heads=0)), 1, P, P, P, None, None) == _lib.MLA_ERR_INVALID_ARG
    assert lib.mla_absorb_q(byref(_dims(d_nope=64)), 1, P, P, P, None, None) == _lib.MLA_ERR_UNSUPPORTED
    assert lib.mla_absorb_q(byref(_dims()), 7, P, P, P, None, None) == _lib.MLA_ERR_UNSUPPORTED
    # An empty batch is a valid no-op.
    assert lib.mla_absorb_q(byref(_dims(batch=0)), 1, P, P, P, None, None) == _lib.MLA_OK
    assert lib.mla_absorb_q(byref(_dims(batch=0)), 1, P, P, P, P, None) == _lib.MLA_OK
    assert lib.mla_up_proj_v(byref(_dims(d_v=64)), 1, P, P, P, None) == _lib.MLA_ERR_UNSUPPORTED
    assert lib.mla_up_proj_v(byref(_dims()), 1, P, None, P, None) == _lib.MLA_ERR_INVALID_ARG


def _attn(lib, dims=None, dtype=1, cache=None, seq=P, max_len=4096, ws=P, ws_bytes=1 << 30, opts=None,
          q=P, q_lo=None):
    dims = dims or _dims()
    cache = cache or _cache()
    return lib.mla_decode_attn(ctypes.byref(dims), dtype, q, q_lo, P, ctypes.byref(cache), seq, max_len,
                               0.072, P, P, ws, ws_bytes, ctypes.byref(opts) if opts else None, None)


def test_attn_validation(lib):
    E = _lib
    assert _attn(lib, q=None) == E.MLA_ERR_INVALID_ARG
    assert _attn(lib, q_lo=P + 8) == E.MLA_ERR_INVALID_ARG
    assert _attn(lib, q_lo=P, dtype=E.MLA_F32, cache=_cache(latent_dtype=E.MLA_F32, rope_dtype=E.MLA_F32,
                                                             latent_stride=2304, rope_stride=2304)) \
        == E.MLA_ERR_UNSUPPORTED  # fp32 q_lat has no low part
    assert _attn(lib, q_lo=P, dims=_dims(batch=0)) == E.MLA_OK
    assert _attn(lib, seq=None) == E.MLA_ERR_INVALID_ARG
    assert _attn(lib, max_len=-1) == E.MLA_ERR_INVALID_ARG
    assert _attn(lib, dims=_dims(q_len=17)) == E.MLA_ERR_UNSUPPORTED
    assert _attn(lib, dims=_dims(heads=2048)) == E.MLA_ERR_UNSUPPORTED
    assert _attn(lib, dims=_dims(d_latent=256)) == E.MLA_ERR_UNSUPPORTED
    assert _attn(lib, cache=_cache(latent_stride=1000)) == E.MLA_ERR_INVALID_ARG
    assert _attn(lib, cache=_cache(latent_stride=512)) == E.MLA_ERR_INVALID_ARG  # row too short
    assert _attn(lib, cache=_cache(num_rows=100)) == E.MLA_ERR_INVALID_ARG  # B*capacity rows missing
    assert _attn(lib, cache=_cache(page_size=32)) == E.MLA_ERR_UNSUPPORTED
    assert _attn(lib, cache=_cache(page_size=64)) == E.MLA_ERR_INVALID_ARG  # no page table
    # A paged pool holds whole 64-row pages.
    assert _attn(lib, cache=_cache(page_size=64, page_table=P, page_table_stride=64, num_rows=4096 + 32)) \
        == E.MLA_ERR_INVALID_ARG
    assert _attn(lib, cache=_cache(latent_dtype=E.MLA_F32)) == E.MLA_ERR_UNSUPPORTED  # bf16 q, f32 cache
    assert _attn(lib, cache=_cache(latent_dtype=E.MLA_FP4_E2M1_E4M3X16)) == E.MLA_ERR_INVALID_ARG
    assert _attn(lib, dtype=E.MLA_F32) == E.MLA_ERR_UNSUPPORTED  # fp32 q, bf16 cache
    assert _attn(lib, opts=_lib.MlaDecodeOpts(-1)) == E.MLA_ERR_INVALID_ARG
    assert _attn(lib, dims=_dims(batch=0)) == E.MLA_OK


def test_append_validation(lib):
    E = _lib
    byref = ctypes.byref
    c = _cache()
    assert lib.mla_cache_append(byref(_dims()), E.MLA_F32, P, P, byref(c), P, None) == E.MLA_ERR_UNSUPPORTED
    assert lib.mla_cache_append(byref(_dims()), E.MLA_BF16, None, P, byref(c), P, None) == E.MLA_ERR_INVALID_ARG
    fp4 = _cache(latent_dtype=E.MLA_FP4_E2M1_E4M3X16, latent_scale=0x10100, scale_stride=416,
                 latent_stride=416, rope_stride=416)
    assert lib.mla_cache_append(byref(_dims(d_latent=256)), E.MLA_F32, P, P, byref(fp4), P,
                                None) == E.MLA_ERR_UNSUPPORTED
    assert lib.mla_cache_append(byref(_dims(batch=0)), E.MLA_F32, P, P, byref(fp4), P, None) == E.MLA_OK
    assert lib.mla_dequant_rows(byref(c), 512, None, 4, P, None) == E.MLA_ERR_INVALID_ARG


def test_rope_append_validation(lib):
    E = _lib
    byref = ctypes.byref
    c = _cache()

    def call(dims=None, k_pe=P, q=None, cs=P, n_pos=4096, style=0):
        return lib.mla_rope_append(byref(dims or _dims()), E.MLA_BF16, P, k_pe, q, cs, n_pos, style, byref(c), P,
                                   None)
    assert call(style=7) == E.MLA_ERR_UNSUPPORTED
    assert call(style=4) == E.MLA_ERR_UNSUPPORTED
    assert call(cs=None) == E.MLA_ERR_INVALID_ARG
    assert call(n_pos=0) == E.MLA_ERR_INVALID_ARG
    assert call(q=P + 4) == E.MLA_ERR_INVALID_ARG
    assert call(k_pe=None) == E.MLA_ERR_INVALID_ARG  # a separate key is needed unless latent-tail
    assert call(dims=_dims(batch=0), k_pe=None, style=E.MLA_ROPE_LATENT_TAIL) == E.MLA_OK
    assert call(dims=_dims(batch=0), style=E.MLA_ROPE_HALVES) == E.MLA_OK


def test_sink_inverse_rope_validation(lib):
    E = _lib
    byref = ctypes.byref

    def call(dims=None, dtype=E.MLA_BF16, x=P, lse=P, sinks=P, cs=P, n_pos=64, style=0, seq=P):
        return lib.mla_sink_inverse_rope(byref(dims or _dims()), dtype, x, lse, sinks, cs, n_pos, style, seq, None)
    assert call(dtype=E.MLA_FP4_E2M1_E4M3X16) == E.MLA_ERR_UNSUPPORTED
    assert call(x=None) == E.MLA_ERR_INVALID_ARG
    assert call(lse=None) == E.MLA_ERR_INVALID_ARG  # sinks need lse
    assert call(seq=None) == E.MLA_ERR_INVALID_ARG  # the rotation needs positions
    assert call(n_pos=0) == E.MLA_ERR_INVALID_ARG
    assert call(style=2) == E.MLA_ERR_UNSUPPORTED
    assert call(dims=_dims(d_rope=63)) == E.MLA_ERR_UNSUPPORTED
    assert call(dims=_dims(d_latent=16384)) == E.MLA_ERR_UNSUPPORTED
    assert call(dims=_dims(batch=0)) == E.MLA_OK
    assert call(sinks=None, cs=None, lse=None, seq=None) == E.MLA_OK  # nothing to do


def test_grouped_out_proj_validation(lib):
    E = _lib
    byref = ctypes.byref

    def call(dims=None, dtype=E.MLA_BF16, g=8, n=1024, x=P, w=P, out=P):
        return lib.mla_grouped_out_proj(byref(dims or _dims(heads=64)), dtype, g, n, x, w, out, None)
    assert call(dtype=E.MLA_F32) == E.MLA_ERR_UNSUPPORTED
    assert call(g=6) == E.MLA_ERR_UNSUPPORTED   # does not divide 64 heads
    assert call(n=48) == E.MLA_ERR_UNSUPPORTED  # not a multiple of 32
    assert call(g=64) == E.MLA_ERR_UNSUPPORTED  # (H/G)*C = 512, not a multiple of 1024
    assert call(g=0) == E.MLA_ERR_INVALID_ARG
    assert call(w=None) == E.MLA_ERR_INVALID_ARG
    assert call(out=P + 8) == E.MLA_ERR_INVALID_ARG
    assert call(dims=_dims(heads=64, batch=0)) == E.MLA_OK


def test_attn_up_and_append_absorb_validation(lib):
    E = _lib
    byref = ctypes.byref
    c = _cache()
    d = _dims()

    def up(wkv=P, out=P, dims=None):
        return lib.mla_decode_attn_up(byref(dims or d), E.MLA_BF16, P, None, P, byref(c), P, 4096, 0.072, P, P,
                                      wkv, out, P, 1 << 30, None, None)
    assert up(wkv=None) == E.MLA_ERR_INVALID_ARG
    assert up(out=None) == E.MLA_ERR_INVALID_ARG
    assert up(dims=_dims(d_v=64)) == E.MLA_ERR_UNSUPPORTED
    assert up(dims=_dims(batch=0)) == E.MLA_OK
    assert lib.mla_append_absorb(byref(d), E.MLA_BF16, P, P, byref(c), P, E.MLA_BF16, None, P, P, None,
                                 None) == E.MLA_ERR_INVALID_ARG
    assert lib.mla_append_absorb(byref(d), E.MLA_BF16, P, P, byref(c), P, E.MLA_BF16, P, P, P, P + 4,
                                 None) == E.MLA_ERR_INVALID_ARG
    assert lib.mla_append_absorb(byref(_dims(batch=0)), E.MLA_BF16, P, P, byref(c), P, E.MLA_BF16, P, P, P, P,
                                 None) == E.MLA_OK


def test_prefill_attn_validation(lib):
    E = _lib
    byref = ctypes.byref

    def call(dims=None, dtype=E.MLA_BF16, cache=None, qn=P, qp=P, sl=P, wkv=P, out=P, ws=None, ws_bytes=0):
        c = cache or _cache()
        return lib.mla_prefill_attn(byref(dims or _dims(q_len=256)), dtype, qn, qp, byref(c), sl, wkv, 0.1, out,
                                    None, ws, ws_bytes, None)
    assert call(dtype=E.MLA_F32) == E.MLA_ERR_UNSUPPORTED
    assert call(dims=_dims(q_len=256, d_v=64)) == E.MLA_ERR_UNSUPPORTED
    assert call(cache=_cache(latent_dtype=E.MLA_F32, latent_stride=2048)) == E.MLA_ERR_UNSUPPORTED
    assert call(dims=_dims(q_len=0)) == E.MLA_ERR_INVALID_ARG
    assert call(wkv=None) == E.MLA_ERR_INVALID_ARG
    assert call(out=P + 8) == E.MLA_ERR_INVALID_ARG
    assert call(sl=None) == E.MLA_ERR_INVALID_ARG
    assert call(cache=_cache(num_rows=100)) == E.MLA_ERR_INVALID_ARG  # 2 x 4096 rows do not fit
    assert call(dims=_dims(q_len=256, batch=0)) == E.MLA_OK
    # Two-kernel path (Q >= 256 with a workspace): too small or misaligned.
    assert call(ws=P, ws_bytes=1 << 20) == E.MLA_ERR_WORKSPACE
    assert call(ws=P + 8, ws_bytes=1 << 40) == E.MLA_ERR_WORKSPACE


def test_rope_less_cache_validation(lib):
    """A cache without a RoPE section (rope NULL, rope_stride 0) is taken by the bf16 / FP4 decode (with q_pe
    NULL), by the append without k_pe and by the latent-tail RoPE append; everything else rejects it."""
    E = _lib
    byref = ctypes.byref
    c = _cache(rope=None, rope_stride=0, latent_stride=1024)
    d = _dims()
    # decode: q_pe must be NULL exactly when the cache has no RoPE keys (checked before any device query)
    assert lib.mla_decode_attn(byref(d), E.MLA_BF16, P, None, P, byref(c), P, 4096, 0.07, P, P, P, 1 << 30, None,
                               None) == E.MLA_ERR_INVALID_ARG
    assert lib.mla_decode_attn(byref(d), E.MLA_BF16, P, None, None, byref(_cache()), P, 4096, 0.07, P, P, P,
                               1 << 30, None, None) == E.MLA_ERR_INVALID_ARG
    cf = _cache(rope=None, rope_stride=0, latent_stride=2048, latent_dtype=E.MLA_F32, rope_dtype=E.MLA_F32)
    assert lib.mla_decode_attn(byref(d), E.MLA_F32, P, None, None, byref(cf), P, 4096, 0.07, P, P, P, 1 << 30,
                               None, None) == E.MLA_ERR_UNSUPPORTED
    # a NULL rope with a nonzero stride is malformed
    bad = _cache(rope=None, rope_stride=128, latent_stride=1024)
    assert lib.mla_decode_attn(byref(d), E.MLA_BF16, P, None, None, byref(bad), P, 4096, 0.07, P, P, P, 1 << 30,
                               None, None) == E.MLA_ERR_INVALID_ARG
    # appends: no k_pe to store; the rotated-key append needs a RoPE section
    assert lib.mla_cache_append(byref(d), E.MLA_BF16, P, P, byref(c), P, None) == E.MLA_ERR_INVALID_ARG
    assert lib.mla_cache_append(byref(_dims(batch=0)), E.MLA_BF16, P, None, byref(c), P, None) == E.MLA_OK
    assert lib.mla_rope_append(byref(d), E.MLA_BF16, P, None, None, P, 64, E.MLA_ROPE_HALVES, byref(c), P,
                               None) == E.MLA_ERR_INVALID_ARG
    assert lib.mla_rope_append(byref(_dims(batch=0)), E.MLA_BF16, P, None, None, P, 64,
                               E.MLA_ROPE_HALVES | E.MLA_ROPE_LATENT_TAIL, byref(c), P, None) == E.MLA_OK
    # prefill needs the RoPE keys
    assert lib.mla_prefill_attn(byref(_dims(q_len=4)), E.MLA_BF16, P, P, byref(c), P, P, 0.1, P, None, None, 0,
                                None) == E.MLA_ERR_INVALID_ARG


def test_prefill_workspace_size(lib):
    """B * H * ceil(capacity / 32) tiles of 16 KiB (K [32][128] and V^T [128][32], bf16) from Q = 256 on;
    0 below (the fused path needs none)."""
    byref = ctypes.byref
    n = ctypes.c_size_t(7)
    for B, H, Q, cap in ((2, 128, 256, 4096), (1, 128, 4096, 4096), (3, 5, 300, 1000), (2, 128, 255, 4096),
                         (8, 128, 64, 4096), (1, 1, 256, 0)):
        assert lib.mla_prefill_workspace_size(byref(_dims(batch=B, heads=H, q_len=Q)), cap, byref(n)) == 0
        want = 0 if Q < 256 else B * H * ((cap + 31) // 32) * 16384
        assert n.value == want, (B, H, Q, cap, n.value)
    assert lib.mla_prefill_workspace_size(byref(_dims()), -1, byref(n)) == _lib.MLA_ERR_INVALID_ARG
    assert lib.mla_prefill_workspace_size(byref(_dims()), 64, None) == _lib.MLA_ERR_INVALID_ARG


def test_attn_noalloc_validation(lib):
    """Host-side rejections of mla_decode_attn_noalloc (before any device query)."""
    E = _lib
    byref = ctypes.byref
    c = _cache()

    def call(dims=None, dtype=E.MLA_BF16, opts=None):
        return lib.mla_decode_attn_noalloc(byref(dims or _dims()), dtype, P, None, P, byref(c), P, 4096, 0.072, P,
                                           P, byref(opts) if opts else None, None)
    assert lib.mla_decode_attn_noalloc(None, E.MLA_BF16, P, None, P, byref(c), P, 4096, 0.072, P, P, None,
                                       None) == E.MLA_ERR_INVALID_ARG
    assert call(dims=_dims(q_len=17)) == E.MLA_ERR_UNSUPPORTED
    assert call(dtype=7) == E.MLA_ERR_UNSUPPORTED
    assert call(opts=_lib.MlaDecodeOpts(-1)) == E.MLA_ERR_INVALID_ARG
    text = open(os.path.join(ROOT, "include", "mla.h")).read()
    m = re.search(r"#define MLA_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == _lib.MLA_NOALLOC_SCRATCH_BYTES
