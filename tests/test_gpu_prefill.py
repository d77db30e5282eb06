"""GPU parity of mla_prefill_attn (non-absorbed attention for many new tokens,
K and V formed from the latent) against the fp64 oracle
mla_ref.decode_nonabsorbed, through the C ABI, on both of its paths: fused
(K and V formed chunk by chunk on chip, no workspace) and two kernels (K and
V formed once into a workspace, then flash attention; Q >= 256).

Cases span several query tiles with a ragged last one, several 32-token
chunks with a ragged tail, sequences shorter than Q (leading queries that see
nothing: out 0, lse -inf), Q = 1, the paged layout and the contiguous one; planted logit jumps that
move the running maximum mid-sequence, on both paths; and, at the two sizes bench.py times, in the launch
configuration it times, sampled (sequence, head) pairs."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from tests import mla_testlib as T

pytestmark = pytest.mark.gpu

CASES = [
    # B, H, Q, lens, paged
    (2, 4, 100, (300, 100), False),
    (3, 2, 64, (97, 17, 200), True),
    (1, 3, 1, (77,), False),
    (1, 2, 130, (500,), True),
    (2, 2, 40, (40, 1), False),
]


def _workspace(case):
    """The two-kernel path's workspace, filled with NaN bytes (every tile read is written first)."""
    o = T.ops()
    w = case.w
    n = o.mla_prefill_workspace_size(w.B, w.H, w.Q, case.pl.capacity)
    assert n > 0
    return torch.full((n,), 0xFF, dtype=torch.uint8, device="cuda")


def _run(inp, out_dtype=torch.bfloat16, two_kernel=False, case=None):
    o = T.ops()
    w = inp.w
    case = case or T.GpuCase(inp, poison=True)
    out = torch.full((w.B, w.H, w.Q, w.Vd), float("nan"), dtype=out_dtype, device="cuda")
    lse = torch.full((w.B, w.H, w.Q), float("nan"), dtype=torch.float32, device="cuda")
    ws = _workspace(case) if two_kernel else None
    o.mla_prefill_attn(case.q_nope, case.q_pe, case.cache, case.seq_lens, case.wkv_b, w.softmax_scale, out, lse,
                       workspace=ws)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("B,H,Q,lens,paged", CASES)
def test_prefill_against_oracle(B, H, Q, lens, paged):
    w = W.reduced(W.WORKLOADS["dsv3_bf16"], B, list(lens), seed=500 + Q).with_(H=H, Q=Q, paged=paged)
    inp = W.generate(w)
    T.say(f"[case] prefill B={B} H={H} Q={Q} lens={lens} paged={paged}")
    out, lse = _run(inp)
    ref = T.oracle(inp)
    T.assert_close(T.to64(out), ref["out"], T.TOL["bf16"], "out")
    T.assert_lse_close(T.to64(lse), ref["lse"], T.TOL["bf16"])
    # Rows that see no position: exactly zero output.
    dead = np.isneginf(ref["lse"])
    assert np.all(T.to64(out)[dead] == 0.0)


# Two-kernel path (Q >= 256): several 128-query tiles with a ragged last one,
# sequences shorter than Q, paged and contiguous, a capacity that is not a
# multiple of the 256-token decompression chunk.
CASES_TWO = [
    # B, H, Q, lens, paged
    (1, 3, 300, (330,), False),
    (2, 2, 257, (600, 257), True),
    (2, 2, 400, (100, 450), False),
    (1, 1, 256, (256,), True),
    (1, 2, 300, (2000,), True),  # a long history before the new tokens
]


@pytest.mark.parametrize("B,H,Q,lens,paged", CASES_TWO)
def test_prefill_two_kernel_against_oracle(B, H, Q, lens, paged):
    w = W.reduced(W.WORKLOADS["dsv3_bf16"], B, list(lens), seed=600 + Q).with_(H=H, Q=Q, paged=paged)
    inp = W.generate(w)
    T.say(f"[case] prefill two-kernel B={B} H={H} Q={Q} lens={lens} paged={paged}")
    case = T.GpuCase(inp, poison=True)
    out, lse = _run(inp, two_kernel=True, case=case)
    ref = T.oracle(inp)
    T.assert_close(T.to64(out), ref["out"], T.TOL["bf16"], "out")
    T.assert_lse_close(T.to64(lse), ref["lse"], T.TOL["bf16"])
    dead = np.isneginf(ref["lse"])
    assert np.all(T.to64(out)[dead] == 0.0)
    # The fused path on the same inputs: the same roundings of K, V and P.
    out_f, lse_f = _run(inp, case=case)
    T.assert_close(T.to64(out), T.to64(out_f), T.TOL["bf16"], "two-kernel vs fused")
    T.assert_lse_close(T.to64(lse), T.to64(lse_f), T.TOL["bf16"])


# Planted logit jumps (log2 domain) through the RoPE stream: every query's
# q_pe carries a * u (u a unit vector) and the RoPE keys of chosen tokens carry
# lam * u on top of their noise, so those tokens' logits sit about
# scale * log2(e) * a * lam above the rest. Jumps of more than 2^8 at a token
# a query reaches mid-sequence make the flash-attention kernel move its
# reference maximum and rescale O (and the fused kernel its running max);
# levels up to 2^120 leave the earlier weights to underflow. Inputs are
# bf16-exact, so the fp64 oracle sees exactly the values the kernels read.
JUMPS = [(100, 600, 12.0), (250, 600, 40.0), (301, 302, 60.0), (330, 331, 9.0), (420, 600, 120.0)]


@pytest.mark.parametrize("two", [True, False])
def test_prefill_planted_score_jumps(two):
    w = W.reduced(W.WORKLOADS["dsv3_bf16"], 1, [600], seed=31).with_(H=3, Q=300)
    inp = W.generate(w)
    rng = np.random.default_rng(5)
    u = rng.standard_normal(w.Dr)
    u /= np.linalg.norm(u)
    a = 4.0
    per_unit = w.softmax_scale * math.log2(math.e) * a
    q_pe = a * u + 0.05 * rng.standard_normal((w.B, w.H, w.Q, w.Dr))
    lam = np.zeros(600)
    for t0, t1, level in JUMPS:
        lam[t0:t1] = level / per_unit
    rope = inp.rope.float().numpy() * 0.3 + lam[:, None] * u[None, :]
    inp.q_pe = torch.from_numpy(q_pe.astype(np.float32)).to(inp.q_pe.dtype)
    inp.rope = torch.from_numpy(rope.astype(np.float32)).to(inp.rope.dtype)
    T.say(f"[case] prefill planted jumps B=1 H=3 Q=300 len=600 two_kernel={two}")
    case = T.GpuCase(inp, poison=True)
    out, lse = _run(inp, two_kernel=two, case=case)
    ref = T.oracle(inp)
    T.assert_close(T.to64(out), ref["out"], T.TOL["bf16"], "out")
    T.assert_lse_close(T.to64(lse), ref["lse"], T.TOL["bf16"])


def test_prefill_two_kernel_bad_page_gives_nan():
    o = T.ops()
    w = W.reduced(W.WORKLOADS["dsv3_bf16"], 2, [300, 300], seed=6).with_(H=2, Q=260, paged=True)
    inp = W.generate(w)
    case = T.GpuCase(inp, poison=False)
    pt = case.cache.page_table.clone()
    pt[1, 2] = 1 << 20  # sequence 1, third page: outside the pool
    case.cache = o.LatentCache.combined(case.buf, w.Ckv, case.pl.capacity, page_table=pt)
    T.say("[case] prefill two-kernel bad page index")
    out, _ = _run(inp, two_kernel=True, case=case)
    r = T.to64(out)
    # Sequence 1 (query q sees positions 0 .. 40 + q): each of its three
    # query tiles reads positions up to 167 or more, so all of them read the
    # bad page (128..191), and a block that reads it writes NaN throughout,
    # as on the fused path.
    assert np.isnan(r[1]).all() and np.isfinite(r[0]).all()


def test_prefill_matches_absorbed_path_for_small_q():
    # The two forms compute the same attention: for Q within the decode
    # kernel's range they agree to the bf16 bar (both against the fp64 oracle,
    # and with each other).
    w = W.reduced(W.WORKLOADS["dsv3_bf16"], 2, [150, 33], seed=77).with_(H=16, Q=4)
    inp = W.generate(w)
    T.say("[case] prefill vs absorbed B=2 H=16 Q=4 lens=(150, 33)")
    out, lse = _run(inp)
    ab = T.GpuCase(inp, poison=True).run()
    T.assert_close(T.to64(out), T.to64(ab["out"]), 2 * T.TOL["bf16"], "out vs absorbed")
    T.assert_lse_close(T.to64(lse), T.to64(ab["lse"]), 2 * T.TOL["bf16"])


def test_prefill_bad_page_gives_nan_and_rejects_fp32():
    o = T.ops()
    w = W.reduced(W.WORKLOADS["dsv3_bf16"], 2, [70, 70], seed=5).with_(H=2, Q=8, paged=True)
    inp = W.generate(w)
    case = T.GpuCase(inp, poison=False)
    pt = case.cache.page_table.clone()
    pt[1, 1] = 1 << 20  # sequence 1, second page: outside the pool
    cache = o.LatentCache.combined(case.buf, w.Ckv, case.pl.capacity, page_table=pt)
    T.say("[case] prefill bad page index")
    out = torch.zeros(w.B, w.H, w.Q, w.Vd, dtype=torch.bfloat16, device="cuda")
    o.mla_prefill_attn(case.q_nope, case.q_pe, cache, case.seq_lens, case.wkv_b, w.softmax_scale, out)
    torch.cuda.synchronize()
    r = T.to64(out)
    assert np.isnan(r[1]).all() and np.isfinite(r[0]).all()
    with pytest.raises(o.MLAError):
        o.mla_prefill_attn(case.q_nope.float(), case.q_pe.float(), cache, case.seq_lens, case.wkv_b.float(),
                           w.softmax_scale, out.float())


@pytest.mark.parametrize("B,Q,L,heads,batch,two", [(8, 64, 4096, [0, 31, 77, 127], [0, 3, 5, 7], False),
                                                   (1, 4096, 4096, [0, 3, 17, 41, 64, 88, 100, 127], [0], True)])
def test_prefill_full_size_sampled(B, Q, L, heads, batch, two):
    # The two prefill shapes bench.py times (H = 128), in the same launch
    # configuration (chunked: fused; full: two kernels); the oracle evaluates
    # the sampled (sequence, head) pairs.
    w = W.reduced(W.WORKLOADS["dsv3_bf16"], B, [L] * B, seed=900 + Q).with_(Q=Q)
    inp = W.generate(w)
    T.say(f"[case] prefill full size B={B} H={w.H} Q={Q} L={L} heads={heads} batch={batch} two_kernel={two}")
    out, lse = _run(inp, two_kernel=two)
    ref = T.oracle(inp, heads=heads, batch=batch)
    got = T.to64(out[batch][:, heads])
    T.assert_close(got, ref["out"], T.TOL["bf16"], "out")
    T.assert_lse_close(T.to64(lse[batch][:, heads]), ref["lse"], T.TOL["bf16"])
