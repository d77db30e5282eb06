"""Seeded sweep of the decode path against the fp64 oracle, through the C ABI:
each case draws its batch, head count (not always a multiple of the 64-row
block), Q, per-sequence lengths (page and tile boundaries, empty and one-token
sequences among them), cache dtype, paging and split count from its own seed,
at sizes the oracle evaluates in a second or two."""
import numpy as np
import pytest

import workloads as W
from tests import mla_testlib as T

pytestmark = pytest.mark.gpu

SPECIAL_LENS = (0, 1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 191, 257)


def _case(i):
    rng = np.random.default_rng(1000 + i)
    dtype = ("bf16", "fp4", "f32")[i % 3]
    B = int(rng.integers(1, 5))
    H = int(rng.choice([8, 16, 24, 40, 64]))
    Q = int(rng.integers(1, 3))
    lens = [int(rng.choice(SPECIAL_LENS)) if rng.random() < 0.5 else int(rng.integers(1, 901)) for _ in range(B)]
    lens = [max(v, 0) for v in lens]
    if max(lens) == 0:
        lens[0] = 1
    paged = bool(rng.random() < 0.5)
    workgroups = int(rng.choice([0, 1, 2, 5, 31]))
    base = {"bf16": "dsv3_bf16", "fp4": "mtp_fp4", "f32": "tiny_f32"}[dtype]
    w = W.reduced(W.WORKLOADS[base], B, lens, seed=2000 + i).with_(H=H, Q=Q, paged=paged)
    return w, workgroups


@pytest.mark.parametrize("i", range(15))
def test_sweep(i):
    w, workgroups = _case(i)
    T.say(f"[case] sweep {i}: {w.dtype} B={w.B} H={w.H} Q={w.Q} lens={list(w.lens)} paged={w.paged} "
          f"workgroups={workgroups}")
    inp = W.generate(w)
    g = T.GpuCase(inp)
    T.compare(g.run(workgroups), T.oracle(inp), w)
