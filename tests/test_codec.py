"""Pins of the reference FP4 latent codec (E2M1 codes, E4M3 scale per 16 channels)."""
import json
import os
import struct

import numpy as np
import pytest
import torch

from oracle import fp4_ref as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_e4m3_table_matches_torch_float8_e4m3fn():
    # Library routine: torch's float8_e4m3fn decoding of all 256 bytes.
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan_t = np.isnan(t)
    assert np.array_equal(nan_t, np.isnan(F.E4M3_TABLE))
    assert np.array_equal(t[~nan_t], F.E4M3_TABLE[~nan_t])
    assert F.E4M3_TABLE[126] == 448.0 and nan_t.sum() == 2


def test_e2m1_table_from_float_bit_patterns():
    # Independent route: an E2M1 normal code (e, m) is the fp32 with biased exponent
    # e - 1 + 127 and top mantissa bit m; the subnormal code 1 is 2^-1.
    def via_bits(code):
        e, m = (code >> 1) & 3, code & 1
        if e == 0:
            v = 0.0 if m == 0 else struct.unpack("<f", struct.pack("<I", 126 << 23))[0]
        else:
            v = struct.unpack("<f", struct.pack("<I", ((e - 1 + 127) << 23) | (m << 22)))[0]
        return -v if code & 8 else v
    for code in range(16):
        assert F.E2M1_TABLE[code] == via_bits(code), code
    assert list(F.E2M1_TABLE[:8]) == sorted(F.E2M1_TABLE[:8])


def test_e4m3_rne_matches_torch_in_range():
    rng = np.random.default_rng(0)
    vals = np.concatenate([
        rng.uniform(0, 448, 20000), np.exp(rng.uniform(np.log(1e-4), np.log(448), 20000)),
        # every midpoint between consecutive finite values: ties go to the even code
        0.5 * (F.E4M3_TABLE[:126] + F.E4M3_TABLE[1:127]),
        F.E4M3_TABLE[:127], [0.0, 448.0, 2.0 ** -10, 3 * 2.0 ** -11]])
    vals = vals.astype(np.float32).astype(np.float64)
    ref = torch.tensor(vals, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = np.array([F.e4m3_encode_rne(v) for v in vals])
    assert np.array_equal(ours, ref)


def test_e4m3_saturates_above_max():
    for v in (448.0, 449.0, 464.0, 470.0, 1e6):
        assert F.e4m3_encode_rne(v) == 126


def test_all_products_exact_in_bf16_and_fp32():
    fin = [c for c in range(256) if np.isfinite(F.E4M3_TABLE[c])]
    prods = np.array([F.E2M1_TABLE[a] * F.E4M3_TABLE[s] for a in range(16) for s in fin])
    assert np.array_equal(prods, prods.astype(np.float32).astype(np.float64))
    bf = torch.tensor(prods, dtype=torch.float64).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(prods, bf)


def _group_with(s_code, mags, signs=None):
    s = F.E4M3_TABLE[s_code]
    v = np.array(mags, dtype=np.float64) * s
    if signs is not None:
        v = v * np.array(signs)
    return v.astype(np.float32)


def test_representable_groups_round_trip():
    # A group whose amax is 6*s with s an E4M3 value reproduces itself exactly.
    rng = np.random.default_rng(1)
    for s_code in (8, 40, 56, 57, 70, 100, 119):
        mags = rng.choice(F.E2M1_TABLE[:8], size=16)
        mags[3] = 6.0
        signs = rng.choice([-1.0, 1.0], size=16)
        g = _group_with(s_code, mags, signs)
        if float(np.float32(np.float32(np.abs(g).max()) / np.float32(6))) != F.E4M3_TABLE[s_code]:
            continue
        row = np.tile(g, 32)[None, :]
        codes, scales = F.quantize_rows(row)
        assert np.all(scales == s_code)
        deq = F.dequantize_rows(codes, scales)
        assert np.array_equal(deq[0], row[0].astype(np.float64))


def test_nibble_order_and_sign():
    row = np.zeros((1, 512), dtype=np.float32)
    row[0, 0] = 6.0   # s = 1 -> code 7 in the low nibble of byte 0
    row[0, 1] = -1.0  # code 0b1010 in the high nibble of byte 0
    row[0, 2] = -0.1  # rounds to zero magnitude -> code 0
    codes, scales = F.quantize_rows(row)
    assert scales[0, 0] == 0x38  # 1.0 in E4M3
    assert codes[0, 0] == 0x07 | (0xA << 4)
    assert codes[0, 1] == 0x00
    assert np.all(scales[0, 1:] == 0) and np.all(codes[0, 8:] == 0)


def test_ties_go_to_even_code():
    # s = 1: midpoints 0.25 (codes 0/1 -> 0), 0.75 (1/2 -> 2), 1.25 (2/3 -> 2),
    # 1.75 (3/4 -> 4), 2.5 (4/5 -> 4), 3.5 (5/6 -> 6), 5 (6/7 -> 6).
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    expect = [0, 2, 2, 4, 4, 6, 6]
    for m, e in zip(mids, expect):
        assert F.e2m1_encode(m, 1.0) == e
        assert F.e2m1_encode(-m, 1.0) == (e | 8 if e else 0)
    assert F.e2m1_encode(7.9, 1.0) == 7  # saturation


def test_error_bound_random_rows():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((256, 512)).astype(np.float32)
    x[::7] *= 1e-3
    codes, scales = F.quantize_rows_fast(x)
    deq = F.dequantize_rows(codes, scales)
    s = np.repeat(F.E4M3_TABLE[scales], 16, axis=1)
    err = np.abs(deq - x)
    # Non-saturated: within half of the widest E2M1 gap (1.0) times s, and within
    # half the local gap; saturated values are +-6s.
    sat = np.abs(x) > 6 * s
    assert np.all(err[~sat] <= 1.0 * s[~sat] + 1e-30)
    assert np.all(np.abs(deq[sat]) == 6 * s[sat])
    mags = np.abs(deq[~sat]) / s[~sat]
    assert np.all(np.isin(mags, F.E2M1_TABLE[:8]))


def test_zero_group_and_tiny_group():
    row = np.zeros((1, 512), dtype=np.float32)
    row[0, 16:32] = 1e-12  # amax/6 below half the smallest E4M3 subnormal -> s = 0
    codes, scales = F.quantize_rows(row)
    assert np.all(codes == 0) and np.all(scales == 0)


def test_fast_matches_elementwise():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((48, 512)).astype(np.float32)
    x[5, :16] = np.float32(0.75)  # tie cases at s = 0.125
    x[5, 0] = np.float32(6 * 0.125)
    x[9, 32:48] = 0.0
    x[11] *= 1000
    a = F.quantize_rows(x)
    b = F.quantize_rows_fast(x, chunk=16)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_entry_is_288_bytes():
    g = json.load(open(os.path.join(GOLDEN, "fp4_entry_bytes.json")))
    codes, scales = F.quantize_rows(np.ones((1, g["latent_dim"]), dtype=np.float32))
    assert codes.nbytes + scales.nbytes == g["entry_bytes"]
    assert scales.shape[1] * g["scale_group_channels"] == g["latent_dim"]
