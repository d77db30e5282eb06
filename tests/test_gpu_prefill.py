"""GPU parity of mla_prefill_attn (non-absorbed attention for many new tokens,
K and V formed from the latent chunk by chunk on chip) against the fp64
oracle mla_ref.decode_nonabsorbed, through the C ABI.

Cases span several 64-query tiles with a ragged last one, several 32-token
chunks with a ragged tail, sequences shorter than Q (leading queries that see
nothing: out 0, lse -inf), Q = 1, the paged layout and the contiguous one; and, at the two sizes bench.py
times, sampled (sequence, head) pairs."""
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


def _run(inp, out_dtype=torch.bfloat16):
    o = T.ops()
    w = inp.w
    case = T.GpuCase(inp, poison=True)
    out = torch.full((w.B, w.H, w.Q, w.Vd), float("nan"), dtype=out_dtype, device="cuda")
    lse = torch.full((w.B, w.H, w.Q), float("nan"), dtype=torch.float32, device="cuda")
    o.mla_prefill_attn(case.q_nope, case.q_pe, case.cache, case.seq_lens, case.wkv_b, w.softmax_scale, out, lse)
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


@pytest.mark.parametrize("B,Q,L,heads,batch", [(8, 64, 4096, [0, 77], [0, 5]), (1, 4096, 4096, [3, 100], [0])])
def test_prefill_full_size_sampled(B, Q, L, heads, batch):
    # The two prefill shapes bench.py times (H = 128), in the same launch
    # configuration; the oracle evaluates the sampled (sequence, head) pairs.
    w = W.reduced(W.WORKLOADS["dsv3_bf16"], B, [L] * B, seed=900 + Q).with_(Q=Q)
    inp = W.generate(w)
    T.say(f"[case] prefill full size B={B} H={w.H} Q={Q} L={L} heads={heads} batch={batch}")
    out, lse = _run(inp)
    ref = T.oracle(inp, heads=heads, batch=batch)
    got = T.to64(out[batch][:, heads])
    T.assert_close(got, ref["out"], T.TOL["bf16"], "out")
    T.assert_lse_close(T.to64(lse[batch][:, heads]), ref["lse"], T.TOL["bf16"])
