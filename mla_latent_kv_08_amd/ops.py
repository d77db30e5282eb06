"""Python binding of libmla.so: the C ABI's calls, taking torch tensors.

Argument marshalling only -- every step runs in the library's HIP kernels.
Tensors must be contiguous and on the current HIP device; torch provides
device memory and the stream (torch's current stream unless one is given).
"""
from __future__ import annotations

import ctypes
import dataclasses
from typing import Optional

import torch

from . import _lib
from ._lib import (MLA_BF16, MLA_F32, MLA_FP4_E2M1_E4M3X16, MLA_ROPE_HALVES, MLA_ROPE_INTERLEAVED,
                   MLA_ROPE_LATENT_TAIL, MLAError, MlaDecodeOpts, MlaDims, MlaKvCache)

__all__ = [
    "MLA_F32", "MLA_BF16", "MLA_FP4_E2M1_E4M3X16", "MLA_ROPE_INTERLEAVED", "MLA_ROPE_HALVES",
    "MLA_ROPE_LATENT_TAIL", "MLAError", "LatentCache", "mla_rope_append", "mla_sink_inverse_rope",
    "mla_grouped_out_proj", "mla_prefill_attn",
    "mla_absorb_q", "mla_decode_workspace_size", "mla_decode_attn", "mla_decode_attn_up", "mla_up_proj_v",
    "mla_decode_attn_noalloc",
    "mla_cache_append", "mla_append_absorb", "mla_dequant_rows",
]


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MLA_F32
    if t.dtype == torch.bfloat16:
        return MLA_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _ptr(t: Optional[torch.Tensor]) -> ctypes.c_void_p:
    if t is None:
        return ctypes.c_void_p(0)
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _dims(B, H, Q, Dn, Dr, Vd, Ckv) -> MlaDims:
    return MlaDims(int(B), int(H), int(Q), int(Dn), int(Dr), int(Vd), int(Ckv))


@dataclasses.dataclass
class LatentCache:
    """Device tensors plus the descriptor fields of an mla_kv_cache.

    Rows are physical cache rows; strides are in bytes. Build one with
    `combined` ([latent | rope] rows, the CacheCompressed layout), `fp4`
    ([codes | scales | rope] rows, or [codes | scales] without RoPE keys) or
    `latent_only` (bf16 latent rows whose tail carries the rotation: no RoPE
    section, rope None).
    """
    latent: torch.Tensor
    rope: Optional[torch.Tensor]
    latent_dtype: int
    rope_dtype: int
    latent_stride: int
    rope_stride: int
    num_rows: int
    capacity: int
    latent_offset: int = 0
    rope_offset: int = 0
    latent_scale: Optional[torch.Tensor] = None
    scale_offset: int = 0
    scale_stride: int = 0
    page_table: Optional[torch.Tensor] = None  # int32 [B, max_pages]

    @property
    def page_size(self) -> int:
        return 0 if self.page_table is None else 64

    def desc(self) -> MlaKvCache:
        pt = self.page_table
        if pt is not None:
            if pt.dtype != torch.int32 or pt.dim() != 2:
                raise ValueError("page_table must be int32 [B, max_pages]")
        return MlaKvCache(
            latent_dtype=self.latent_dtype,
            rope_dtype=self.rope_dtype,
            latent=_ptr(self.latent).value + self.latent_offset,
            latent_scale=(_ptr(self.latent_scale).value + self.scale_offset
                          if self.latent_scale is not None else None),
            rope=_ptr(self.rope).value + self.rope_offset if self.rope is not None else None,
            latent_stride=self.latent_stride,
            scale_stride=self.scale_stride,
            rope_stride=self.rope_stride,
            num_rows=self.num_rows,
            page_size=self.page_size,
            capacity=self.capacity,
            page_table=_ptr(pt).value if pt is not None else None,
            page_table_stride=int(pt.shape[1]) if pt is not None else 0,
            reserved=0,
        )

    @staticmethod
    def combined(buf: torch.Tensor, d_latent: int, capacity: int,
                 page_table: Optional[torch.Tensor] = None) -> "LatentCache":
        """buf: [n_rows, d_latent + d_rope] bf16 or fp32, each row [latent | rope]."""
        code = _code(buf)
        es = buf.element_size()
        row = buf.shape[1] * es
        return LatentCache(buf, buf, code, code, row, row, buf.shape[0], capacity,
                           rope_offset=d_latent * es, page_table=page_table)

    @staticmethod
    def latent_only(buf: torch.Tensor, d_latent: int, capacity: int,
                    page_table: Optional[torch.Tensor] = None) -> "LatentCache":
        """buf: [n_rows, d_latent] bf16 latent rows, no RoPE section (the DeepSeek-V4.1-Flash layout: the
        rotation is applied to the latent's last d_rope dims)."""
        code = _code(buf)
        row = buf.shape[1] * buf.element_size()
        return LatentCache(buf, None, code, code, row, 0, buf.shape[0], capacity, page_table=page_table)

    @staticmethod
    def fp4(buf: torch.Tensor, d_latent: int, capacity: int,
            page_table: Optional[torch.Tensor] = None, rope: bool = True) -> "LatentCache":
        """buf: uint8 [n_rows, d_latent/2 + d_latent/16 + 2*d_rope]: codes | E4M3 scales | bf16 rope; with
        rope=False, [n_rows, d_latent/2 + d_latent/16]: codes | scales (288 B for 512 dims)."""
        if buf.dtype != torch.uint8:
            raise TypeError("FP4 cache buffer must be uint8")
        row = buf.shape[1]
        if not rope:
            return LatentCache(buf, None, MLA_FP4_E2M1_E4M3X16, MLA_BF16, row, 0, buf.shape[0], capacity,
                               latent_scale=buf, scale_offset=d_latent // 2, scale_stride=row,
                               page_table=page_table)
        return LatentCache(buf, buf, MLA_FP4_E2M1_E4M3X16, MLA_BF16, row, row, buf.shape[0], capacity,
                           rope_offset=d_latent // 2 + d_latent // 16, latent_scale=buf,
                           scale_offset=d_latent // 2, scale_stride=row, page_table=page_table)

    @staticmethod
    def fp4_row_bytes(d_latent: int, d_rope: int) -> int:
        return d_latent // 2 + d_latent // 16 + 2 * d_rope


def mla_absorb_q(q_nope: torch.Tensor, wkv_b: torch.Tensor, q_lat: torch.Tensor,
                 q_lat_lo: Optional[torch.Tensor] = None, stream=None) -> None:
    """q_lat[b,h,q,:] = W_UK[h]^T q_nope[b,h,q,:]; q_nope [B,H,Q,Dn], wkv_b [H,Dn+Vd,Ckv]. With q_lat_lo
    (bf16 only) the residual of q_lat's rounding is written there too."""
    B, H, Q, Dn = q_nope.shape
    Vd = wkv_b.shape[1] - Dn
    Ckv = wkv_b.shape[2]
    d = _dims(B, H, Q, Dn, 64, Vd, Ckv)
    _lib.check(_lib.load().mla_absorb_q(ctypes.byref(d), _code(q_nope), _ptr(q_nope), _ptr(wkv_b),
                                        _ptr(q_lat), _ptr(q_lat_lo), _stream(stream)), "mla_absorb_q")


def mla_decode_workspace_size(batch: int, heads: int, q_len: int, dtype: int, max_seq_len: int,
                              workgroups: int = 0, d_nope: int = 128, d_rope: int = 64,
                              d_v: int = 128, d_latent: int = 512) -> int:
    d = _dims(batch, heads, q_len, d_nope, d_rope, d_v, d_latent)
    opts = MlaDecodeOpts(int(workgroups))
    out = ctypes.c_size_t(0)
    _lib.check(_lib.load().mla_decode_workspace_size(ctypes.byref(d), int(dtype), int(max_seq_len),
                                                     ctypes.byref(opts), ctypes.byref(out)),
               "mla_decode_workspace_size")
    return int(out.value)


def mla_decode_attn(q_lat: torch.Tensor, q_pe: Optional[torch.Tensor], cache: LatentCache,
                    seq_lens: torch.Tensor, max_seq_len: int, softmax_scale: float,
                    x_lat: torch.Tensor, lse: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None, workgroups: int = 0,
                    d_nope: int = 128, d_v: int = 128, q_lat_lo: Optional[torch.Tensor] = None,
                    stream=None, d_rope: int = 64) -> None:
    """Absorbed attention over the latent cache; see mla_decode_attn in include/mla.h. q_pe is None
    exactly when the cache has no RoPE section (then d_rope only fills the dims)."""
    B, H, Q, Ckv = q_lat.shape
    Dr = q_pe.shape[-1] if q_pe is not None else d_rope
    if seq_lens.dtype != torch.int32:
        raise TypeError("seq_lens must be int32")
    if lse is not None and lse.dtype != torch.float32:
        raise TypeError("lse must be float32")
    code = _code(q_lat)
    d = _dims(B, H, Q, d_nope, Dr, d_v, Ckv)
    opts = MlaDecodeOpts(int(workgroups))
    if workspace is None:
        nbytes = mla_decode_workspace_size(B, H, Q, code, max_seq_len, workgroups, d_nope, Dr, d_v, Ckv)
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q_lat.device)
    desc = cache.desc()
    _lib.check(_lib.load().mla_decode_attn(
        ctypes.byref(d), code, _ptr(q_lat), _ptr(q_lat_lo), _ptr(q_pe), ctypes.byref(desc), _ptr(seq_lens),
        int(max_seq_len), float(softmax_scale), _ptr(x_lat), _ptr(lse), _ptr(workspace),
        workspace.numel() * workspace.element_size(), ctypes.byref(opts), _stream(stream)),
        "mla_decode_attn")


def mla_decode_attn_noalloc(q_lat: torch.Tensor, q_pe: Optional[torch.Tensor], cache: LatentCache,
                            seq_lens: torch.Tensor, max_seq_len: int, softmax_scale: float,
                            x_lat: torch.Tensor, lse: Optional[torch.Tensor] = None, workgroups: int = 0,
                            d_nope: int = 128, d_v: int = 128, q_lat_lo: Optional[torch.Tensor] = None,
                            stream=None, d_rope: int = 64) -> None:
    """mla_decode_attn with the library's own scratch instead of a workspace; see
    mla_decode_attn_noalloc in include/mla.h."""
    B, H, Q, Ckv = q_lat.shape
    Dr = q_pe.shape[-1] if q_pe is not None else d_rope
    if seq_lens.dtype != torch.int32:
        raise TypeError("seq_lens must be int32")
    if lse is not None and lse.dtype != torch.float32:
        raise TypeError("lse must be float32")
    d = _dims(B, H, Q, d_nope, Dr, d_v, Ckv)
    opts = MlaDecodeOpts(int(workgroups))
    desc = cache.desc()
    _lib.check(_lib.load().mla_decode_attn_noalloc(
        ctypes.byref(d), _code(q_lat), _ptr(q_lat), _ptr(q_lat_lo), _ptr(q_pe), ctypes.byref(desc),
        _ptr(seq_lens), int(max_seq_len), float(softmax_scale), _ptr(x_lat), _ptr(lse), ctypes.byref(opts),
        _stream(stream)), "mla_decode_attn_noalloc")


def mla_prefill_workspace_size(B: int, H: int, Q: int, capacity: int, Dn: int = 128, Dr: int = 64, Vd: int = 128,
                               Ckv: int = 512) -> int:
    """Bytes of the two-kernel prefill's workspace (0 when Q < 256); see include/mla.h."""
    d = _dims(B, H, Q, Dn, Dr, Vd, Ckv)
    n = ctypes.c_size_t(0)
    _lib.check(_lib.load().mla_prefill_workspace_size(ctypes.byref(d), int(capacity), ctypes.byref(n)),
               "mla_prefill_workspace_size")
    return int(n.value)


def mla_prefill_attn(q_nope: torch.Tensor, q_pe: torch.Tensor, cache: LatentCache, seq_lens: torch.Tensor,
                     wkv_b: torch.Tensor, softmax_scale: float, out: torch.Tensor,
                     lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                     stream=None) -> None:
    """Non-absorbed attention with K and V formed from the latent: fused on chip without a workspace, in two
    kernels (K and V formed once, then flash attention) with one; see mla_prefill_attn in include/mla.h."""
    B, H, Q, Dn = q_nope.shape
    Dr = q_pe.shape[-1]
    Vd = out.shape[-1]
    Ckv = wkv_b.shape[-1]
    if seq_lens.dtype != torch.int32:
        raise TypeError("seq_lens must be int32")
    if lse is not None and lse.dtype != torch.float32:
        raise TypeError("lse must be float32")
    d = _dims(B, H, Q, Dn, Dr, Vd, Ckv)
    desc = cache.desc()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _lib.check(_lib.load().mla_prefill_attn(
        ctypes.byref(d), _code(q_nope), _ptr(q_nope), _ptr(q_pe), ctypes.byref(desc), _ptr(seq_lens),
        _ptr(wkv_b), float(softmax_scale), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream)),
        "mla_prefill_attn")


def mla_decode_attn_up(q_lat: torch.Tensor, q_pe: Optional[torch.Tensor], cache: LatentCache,
                       seq_lens: torch.Tensor, max_seq_len: int, softmax_scale: float,
                       x_lat: torch.Tensor, lse: Optional[torch.Tensor], wkv_b: torch.Tensor, out: torch.Tensor,
                       workspace: Optional[torch.Tensor] = None, workgroups: int = 0,
                       q_lat_lo: Optional[torch.Tensor] = None, stream=None, d_rope: int = 64) -> None:
    """mla_decode_attn then mla_up_proj_v on its x; see mla_decode_attn_up in include/mla.h."""
    B, H, Q, Ckv = q_lat.shape
    Dr = q_pe.shape[-1] if q_pe is not None else d_rope
    Vd = out.shape[-1]
    d_nope = wkv_b.shape[1] - Vd
    if seq_lens.dtype != torch.int32:
        raise TypeError("seq_lens must be int32")
    if lse is not None and lse.dtype != torch.float32:
        raise TypeError("lse must be float32")
    code = _code(q_lat)
    d = _dims(B, H, Q, d_nope, Dr, Vd, Ckv)
    opts = MlaDecodeOpts(int(workgroups))
    if workspace is None:
        nbytes = mla_decode_workspace_size(B, H, Q, code, max_seq_len, workgroups, d_nope, Dr, Vd, Ckv)
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q_lat.device)
    desc = cache.desc()
    _lib.check(_lib.load().mla_decode_attn_up(
        ctypes.byref(d), code, _ptr(q_lat), _ptr(q_lat_lo), _ptr(q_pe), ctypes.byref(desc), _ptr(seq_lens),
        int(max_seq_len), float(softmax_scale), _ptr(x_lat), _ptr(lse), _ptr(wkv_b), _ptr(out),
        _ptr(workspace), workspace.numel() * workspace.element_size(), ctypes.byref(opts), _stream(stream)),
        "mla_decode_attn_up")


def mla_up_proj_v(x_lat: torch.Tensor, wkv_b: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    """out[b,h,q,:] = W_UV[h] x_lat[b,h,q,:]; x_lat [B,H,Q,Ckv], out [B,H,Q,Vd] (Dn = rows - Vd)."""
    B, H, Q, Ckv = x_lat.shape
    Vd = out.shape[-1]
    d_nope = wkv_b.shape[1] - Vd
    d = _dims(B, H, Q, d_nope, 64, Vd, Ckv)
    _lib.check(_lib.load().mla_up_proj_v(ctypes.byref(d), _code(x_lat), _ptr(x_lat), _ptr(wkv_b),
                                         _ptr(out), _stream(stream)), "mla_up_proj_v")


def mla_cache_append(c_kv_new: torch.Tensor, k_pe_new: Optional[torch.Tensor], cache: LatentCache,
                     seq_lens: torch.Tensor, stream=None, d_rope: int = 64) -> None:
    """Store the new tokens [B, Qn, Ckv] / [B, Qn, Dr] at positions len-Qn .. len-1 (k_pe_new None for a
    cache without a RoPE section; d_rope then only fills the dims)."""
    B, Qn, Ckv = c_kv_new.shape
    Dr = k_pe_new.shape[-1] if k_pe_new is not None else d_rope
    if seq_lens.dtype != torch.int32:
        raise TypeError("seq_lens must be int32")
    d = _dims(B, 1, Qn, 128, Dr, 128, Ckv)
    desc = cache.desc()
    _lib.check(_lib.load().mla_cache_append(ctypes.byref(d), _code(c_kv_new), _ptr(c_kv_new),
                                            _ptr(k_pe_new), ctypes.byref(desc), _ptr(seq_lens),
                                            _stream(stream)), "mla_cache_append")


def mla_rope_append(c_kv_new: torch.Tensor, k_pe_new: Optional[torch.Tensor], cache: LatentCache,
                    seq_lens: torch.Tensor, cos_sin: torch.Tensor, style: int = MLA_ROPE_INTERLEAVED,
                    q_pe: Optional[torch.Tensor] = None, latent_tail: bool = False, d_rope: int = 64,
                    stream=None) -> None:
    """mla_cache_append with k_pe_new (unrotated) turned to each token's position on the way in, and
    q_pe [B, H, Qn, Dr] (optional) turned in place; cos_sin: fp32 [n_pos, Dr]. With latent_tail (the
    V4.1-Flash form) the last d_rope dims of the latent are turned instead, k_pe_new may be None and q_pe
    is the query rows [B, H, Qn, Ckv]. See mla_rope_append in include/mla.h."""
    B, Qn, Ckv = c_kv_new.shape
    Dr = d_rope if latent_tail else k_pe_new.shape[-1]
    if seq_lens.dtype != torch.int32:
        raise TypeError("seq_lens must be int32")
    if cos_sin.dtype != torch.float32 or cos_sin.dim() != 2 or cos_sin.shape[1] != Dr:
        raise TypeError("cos_sin must be float32 [n_pos, Dr]")
    H = 1
    if q_pe is not None:
        width = Ckv if latent_tail else Dr
        if q_pe.dim() != 4 or q_pe.shape[0] != B or q_pe.shape[2] != Qn or q_pe.shape[3] != width:
            raise TypeError(f"q_pe must be [B, H, Qn, {width}]")
        if not q_pe.is_contiguous():
            raise TypeError("q_pe must be contiguous")
        H = q_pe.shape[1]
    d = _dims(B, H, Qn, 128, Dr, 128, Ckv)
    desc = cache.desc()
    st = int(style) | (MLA_ROPE_LATENT_TAIL if latent_tail else 0)
    _lib.check(_lib.load().mla_rope_append(ctypes.byref(d), _code(c_kv_new), _ptr(c_kv_new), _ptr(k_pe_new),
                                           _ptr(q_pe), _ptr(cos_sin), int(cos_sin.shape[0]), st,
                                           ctypes.byref(desc), _ptr(seq_lens), _stream(stream)), "mla_rope_append")


def mla_sink_inverse_rope(x_lat: torch.Tensor, lse: Optional[torch.Tensor], seq_lens: Optional[torch.Tensor] = None,
                          sinks: Optional[torch.Tensor] = None, cos_sin: Optional[torch.Tensor] = None,
                          style: int = MLA_ROPE_INTERLEAVED, stream=None) -> None:
    """In place on x_lat [B, H, Q, Ckv] / lse [B, H, Q]: fold per-head sink logits (fp32 [H]) into them,
    then turn x's last cos_sin.shape[1] dims back by each query's position. See mla_sink_inverse_rope in
    include/mla.h."""
    B, H, Q, Ckv = x_lat.shape
    Dr = cos_sin.shape[1] if cos_sin is not None else 0
    if sinks is not None and (sinks.dtype != torch.float32 or sinks.numel() != H):
        raise TypeError("sinks must be float32 [H]")
    if lse is not None and lse.dtype != torch.float32:
        raise TypeError("lse must be float32")
    if seq_lens is not None and seq_lens.dtype != torch.int32:
        raise TypeError("seq_lens must be int32")
    d = _dims(B, H, Q, 128, Dr, 128, Ckv)
    n_pos = int(cos_sin.shape[0]) if cos_sin is not None else 0
    _lib.check(_lib.load().mla_sink_inverse_rope(ctypes.byref(d), _code(x_lat), _ptr(x_lat), _ptr(lse), _ptr(sinks),
                                                 _ptr(cos_sin), n_pos, int(style), _ptr(seq_lens), _stream(stream)),
               "mla_sink_inverse_rope")


def mla_append_absorb(c_kv_new: torch.Tensor, k_pe_new: torch.Tensor, cache: LatentCache,
                      seq_lens: torch.Tensor, q_nope: torch.Tensor, wkv_b: torch.Tensor, q_lat: torch.Tensor,
                      q_lat_lo: Optional[torch.Tensor] = None, stream=None) -> None:
    """mla_cache_append(c_kv_new, k_pe_new, cache, seq_lens) then mla_absorb_q(q_nope, wkv_b, q_lat),
    in one launch for bf16. The new tokens are the queries: [B, Q, ...] and [B, H, Q, ...]."""
    B, Qn, Ckv = c_kv_new.shape
    Dr = k_pe_new.shape[-1]
    _, H, Q, Dn = q_nope.shape
    if Q != Qn:
        raise ValueError("mla_append_absorb: the new tokens must be the queries (same Q)")
    if seq_lens.dtype != torch.int32:
        raise TypeError("seq_lens must be int32")
    Vd = wkv_b.shape[1] - Dn
    d = _dims(B, H, Q, Dn, Dr, Vd, Ckv)
    desc = cache.desc()
    _lib.check(_lib.load().mla_append_absorb(ctypes.byref(d), _code(c_kv_new), _ptr(c_kv_new), _ptr(k_pe_new),
                                             ctypes.byref(desc), _ptr(seq_lens), _code(q_nope), _ptr(q_nope),
                                             _ptr(wkv_b), _ptr(q_lat), _ptr(q_lat_lo), _stream(stream)),
               "mla_append_absorb")


def mla_dequant_rows(cache: LatentCache, rows: torch.Tensor, out: torch.Tensor, d_latent: int = 512,
                     stream=None) -> None:
    """out [n, d_latent] fp32 = decoded latent of physical rows `rows` (int32 [n])."""
    if rows.dtype != torch.int32 or out.dtype != torch.float32:
        raise TypeError("rows must be int32 and out float32")
    desc = cache.desc()
    _lib.check(_lib.load().mla_dequant_rows(ctypes.byref(desc), int(d_latent), _ptr(rows),
                                            int(rows.numel()), _ptr(out), _stream(stream)),
               "mla_dequant_rows")


def mla_grouped_out_proj(x: torch.Tensor, w_o: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    """out [B, Q, G*N] = grouped W_O of x [B, H, Q, C] with w_o [G, N, (H/G)*C]; see mla_grouped_out_proj in
    include/mla.h."""
    B, H, Q, C = x.shape
    G, N, _ = w_o.shape
    if out.shape != (B, Q, G * N):
        raise TypeError("out must be [B, Q, G*N]")
    d = _dims(B, H, Q, 128, 64, 128, C)
    _lib.check(_lib.load().mla_grouped_out_proj(ctypes.byref(d), _code(x), G, N, _ptr(x), _ptr(w_o), _ptr(out),
                                                _stream(stream)), "mla_grouped_out_proj")
