"""mla_decode_attn_noalloc (scratch inside the library, no workspace, no
allocation) against mla_decode_attn with a caller workspace, through the C
ABI: two calls in a row, the second on a smaller input, each bit for bit equal
to the workspace call and within the bf16 bar of the fp64 oracle; a call whose
workspace would exceed the library's scratch is rejected."""
import pytest
import torch

import workloads as W
from mla_latent_kv_08_amd import _lib
from tests import mla_testlib as T

pytestmark = pytest.mark.gpu


def _both(lens, workgroups):
    o = T.ops()
    w = W.reduced(W.WORKLOADS["dsv3_bf16"], len(lens), lens)
    T.say(f"[case] noalloc {w.name} lens={lens} workgroups={workgroups}")
    inp = W.generate(w)
    g = T.GpuCase(inp)
    B, H, Q = w.B, w.H, w.Q
    q_lat = torch.empty(B, H, Q, w.Ckv, dtype=torch.bfloat16, device="cuda")
    q_lo = torch.empty_like(q_lat)
    o.mla_absorb_q(g.q_nope, g.wkv_b, q_lat, q_lat_lo=q_lo)
    res = []
    for noalloc in (False, True):
        x = torch.full((B, H, Q, w.Ckv), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((B, H, Q), float("nan"), dtype=torch.float32, device="cuda")
        if noalloc:
            o.mla_decode_attn_noalloc(q_lat, g.q_pe, g.cache, g.seq_lens, g.max_len, w.softmax_scale, x, lse,
                                      workgroups=workgroups, q_lat_lo=q_lo)
        else:
            o.mla_decode_attn(q_lat, g.q_pe, g.cache, g.seq_lens, g.max_len, w.softmax_scale, x, lse,
                              workgroups=workgroups, q_lat_lo=q_lo)
        torch.cuda.synchronize()
        res.append((x, lse))
    (x0, l0), (x1, l1) = res
    assert torch.equal(x0.view(torch.int16), x1.view(torch.int16)), "x differs from the workspace call"
    assert torch.equal(l0.view(torch.int32), l1.view(torch.int32)), "lse differs from the workspace call"
    ref = T.oracle(inp)
    T.assert_close(T.to64(x1), ref["x"], T.TOL["bf16"], "x (noalloc)")
    T.assert_lse_close(T.to64(l1), ref["lse"], T.TOL["bf16"])


def test_noalloc_two_calls_second_smaller():
    # The first call leaves its partials in the scratch; the second, smaller
    # one (fewer sequences, other lengths, other split) must not see them.
    _both([1000, 777, 337], 0)
    _both([300, 65], 5)


def test_noalloc_rejects_oversized_workspace():
    o = T.ops()
    w = W.reduced(W.WORKLOADS["dsv3_bf16"], 2, [300, 65])
    inp = W.generate(w)
    g = T.GpuCase(inp)
    q_lat = torch.zeros(w.B, w.H, w.Q, w.Ckv, dtype=torch.bfloat16, device="cuda")
    x = torch.zeros_like(q_lat)
    huge = 1 << 20  # workgroups per row block: far past the scratch
    need = o.mla_decode_workspace_size(w.B, w.H, w.Q, o.MLA_BF16, g.max_len, huge)
    assert need > _lib.MLA_NOALLOC_SCRATCH_BYTES
    with pytest.raises(_lib.MLAError) as e:
        o.mla_decode_attn_noalloc(q_lat, g.q_pe, g.cache, g.seq_lens, g.max_len, w.softmax_scale, x,
                                  workgroups=huge)
    assert e.value.status == _lib.MLA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.count_nonzero(x.float()) == 0  # nothing was enqueued


def test_noalloc_full_headline_equals_workspace():
    # The launch bench.py times (B=32, H=128, 4096 tokens each, default split):
    # its workspace fits the library's scratch, and the scratch call gives the
    # workspace call's bits; then a smaller reduced call on the same scratch.
    o = T.ops()
    w = W.WORKLOADS["dsv3_bf16"]
    T.say(f"[case] noalloc full {w.name}")
    inp = W.generate(w)
    g = T.GpuCase(inp)
    need = o.mla_decode_workspace_size(w.B, w.H, w.Q, o.MLA_BF16, g.max_len)
    assert need <= _lib.MLA_NOALLOC_SCRATCH_BYTES
    q_lat = torch.empty(w.B, w.H, w.Q, w.Ckv, dtype=torch.bfloat16, device="cuda")
    o.mla_absorb_q(g.q_nope, g.wkv_b, q_lat)
    res = []
    for noalloc in (False, True):
        x = torch.full((w.B, w.H, w.Q, w.Ckv), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((w.B, w.H, w.Q), float("nan"), dtype=torch.float32, device="cuda")
        call = o.mla_decode_attn_noalloc if noalloc else o.mla_decode_attn
        call(q_lat, g.q_pe, g.cache, g.seq_lens, g.max_len, w.softmax_scale, x, lse)
        torch.cuda.synchronize()
        res.append((x, lse))
    (x0, l0), (x1, l1) = res
    assert torch.isfinite(x1.float()).all()
    assert torch.equal(x0.view(torch.int16), x1.view(torch.int16)), "x differs from the workspace call"
    assert torch.equal(l0.view(torch.int32), l1.view(torch.int32)), "lse differs from the workspace call"
    del g, q_lat, res, x0, x1
    torch.cuda.empty_cache()
    _both([300, 65], 0)
