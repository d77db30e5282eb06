"""One decode step captured in a HIP graph through the C ABI (append, absorb,
attention, up-projection): every replay reproduces the eager step bit for
bit, with eager work and synchronisation between the replays."""
import pytest
import torch

import workloads as W
from tests import mla_testlib as T

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    w = W.reduced(W.WORKLOADS["dsv3_bf16"], 3, [1000, 777, 337])
    T.say(f"[case] graph capture of one step, {w.name} lens={w.lens}")
    inp = W.generate(w)
    g = T.GpuCase(inp)
    o = T.ops()
    B, H, Q = w.B, w.H, w.Q
    bf16 = torch.bfloat16
    last = inp.seq_offsets[1:] - 1
    c_new = inp.latent[last].reshape(B, 1, w.Ckv).contiguous().cuda()
    r_new = inp.rope[last].reshape(B, 1, w.Dr).contiguous().cuda()
    q_lat = torch.empty(B, H, Q, w.Ckv, dtype=bf16, device="cuda")
    q_lo = torch.empty_like(q_lat)
    x = torch.empty_like(q_lat)
    lse = torch.empty(B, H, Q, dtype=torch.float32, device="cuda")
    out = torch.empty(B, H, Q, w.Vd, dtype=bf16, device="cuda")
    ws = torch.empty(max(o.mla_decode_workspace_size(B, H, Q, o.MLA_BF16, g.max_len), 16),
                     dtype=torch.uint8, device="cuda")

    def step(stream):
        o.mla_cache_append(c_new, r_new, g.cache, g.seq_lens, stream=stream)
        o.mla_absorb_q(g.q_nope, g.wkv_b, q_lat, q_lat_lo=q_lo, stream=stream)
        o.mla_decode_attn(q_lat, g.q_pe, g.cache, g.seq_lens, g.max_len, w.softmax_scale, x, lse,
                          workspace=ws, q_lat_lo=q_lo, stream=stream)
        o.mla_up_proj_v(x, g.wkv_b, out, stream=stream)

    def snapshot():
        return {"q_lat": q_lat.view(torch.int16).clone(), "q_lat_lo": q_lo.view(torch.int16).clone(),
                "x": x.view(torch.int16).clone(),
                "lse": lse.clone(), "out": out.view(torch.int16).clone()}

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = snapshot()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(torch.cuda.current_stream())
    torch.cuda.synchronize()

    for rep in range(4):
        # Eager work between replays: overwrite every output, and run an eager step.
        x.fill_(float("nan"))
        out.zero_()
        lse.fill_(1.0)
        q_lat.zero_()
        q_lo.zero_()
        if rep == 2:
            step(torch.cuda.current_stream())
            torch.cuda.synchronize()
            x.zero_()
        graph.replay()
        torch.cuda.synchronize()
        now = snapshot()
        for k, v in eager.items():
            assert torch.equal(now[k], v), f"replay {rep}: {k} differs from the eager step"
        T.say(f"  replay {rep}: identical to the eager step")
