"""Reference FP4 latent codec: E2M1 elements with one E4M3 scale per 16 channels.

TEST INFRASTRUCTURE. Only tests/, the smoke check and bench.py's CPU-baseline
leg may import this module; the product path never does.

The DeepSeek-V4.1-Flash MLA course page ("4A", profiling section) describes a
512-dim latent stored as FP4 with an E4M3 scale per 16 channels, whose
compressed K/V entry is 288 B (256 B of 4-bit codes + 32 one-byte scales).
The page fixes neither the rounding rules nor the bit order, so this codec
takes the plainest reading, stated here and in the design notes:

  * E2M1 code (4 bits): bit 3 sign, bits 2..1 exponent (bias 1), bit 0
    mantissa; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 for codes 0..7.
  * E4M3 scale byte ("FN" variant: no infinities, 448 max, S.1111.111 = NaN):
    bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa.
  * channel 2i sits in the low nibble of byte i, channel 2i+1 in the high one;
    the 32 scales are stored in channel-group order.
  * scale of a 16-channel group: s = E4M3 round-to-nearest-even of
    fp32(amax / 6), where amax is the group's largest |x| and the division is
    a correctly rounded fp32 division; values above 448 saturate to 448.
  * element code: the E2M1 magnitude nearest to |x|/s (exact real quotient),
    ties to the even code, saturating at 6; sign bit = sign of x; a value whose
    magnitude rounds to 0 gets code 0 (positive zero). If s = 0 every code is 0.
  * dequantised value = E2M1(code) * E4M3(scale), which is exact in fp32 and
    in bf16 (at most 6 significant bits, exponent within range).
"""
from __future__ import annotations

import numpy as np

GROUP = 16


def e2m1_value(code: int) -> float:
    """Value of a 4-bit E2M1 code from its bit fields."""
    code = int(code) & 0xF
    sign = -1.0 if code & 0x8 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    mag = 0.5 * m if e == 0 else (2.0 ** (e - 1)) * (1.0 + 0.5 * m)
    return sign * mag


def e4m3_value(byte: int) -> float:
    """Value of an OCP E4M3 ("FN") byte from its bit fields."""
    byte = int(byte) & 0xFF
    sign = -1.0 if byte & 0x80 else 1.0
    e = (byte >> 3) & 0xF
    m = byte & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
# Non-negative finite E4M3 values are codes 0..126, in increasing order.
_E4M3_POS = E4M3_TABLE[:127]
# Midpoints between consecutive E2M1 magnitudes (codes k and k+1).
_E2M1_MAG = E2M1_TABLE[:8]
_E2M1_MID = 0.5 * (_E2M1_MAG[:-1] + _E2M1_MAG[1:])


def e4m3_encode_rne(v: float) -> int:
    """Nearest non-negative finite E4M3 code to v >= 0, ties to the even code.

    Values beyond 448 saturate to code 126 (448).
    """
    v = float(v)
    assert v >= 0.0 and not np.isnan(v)
    if v >= _E4M3_POS[-1]:
        return 126
    k = int(np.searchsorted(_E4M3_POS, v, side="left"))  # first value >= v
    if _E4M3_POS[k] == v:
        return k
    lo, hi = k - 1, k
    dlo = v - _E4M3_POS[lo]
    dhi = _E4M3_POS[hi] - v
    if dlo < dhi:
        return lo
    if dhi < dlo:
        return hi
    return lo if lo % 2 == 0 else hi


def group_scale_code(group: np.ndarray) -> int:
    """E4M3 scale byte of one 16-channel group (fp32 values)."""
    amax = np.float32(np.max(np.abs(group.astype(np.float32))))
    ratio = np.float32(amax) / np.float32(6.0)  # IEEE fp32 division, correctly rounded
    return e4m3_encode_rne(float(ratio))


def e2m1_encode(x: float, s: float) -> int:
    """E2M1 code of x under scale s > 0: nearest magnitude to |x|/s, ties to even."""
    ax = abs(float(x))
    # Exact decision: compare |x| with s * midpoint (both exact in fp64).
    k = 0
    for j, mid in enumerate(_E2M1_MID):
        t = s * mid
        if ax > t:
            k = j + 1
        elif ax == t:
            k = j if j % 2 == 0 else j + 1  # tie between codes j and j+1
            break
        else:
            break
    if k == 0:
        return 0
    return k | (0x8 if x < 0 else 0)


def quantize_rows(x) -> tuple:
    """fp32 latent rows [N, C] (C multiple of 32) -> (codes uint8 [N, C/2], scales uint8 [N, C/16])."""
    x = np.asarray(x, dtype=np.float32)
    N, C = x.shape
    assert C % (2 * GROUP) == 0
    codes = np.zeros((N, C // 2), dtype=np.uint8)
    scales = np.zeros((N, C // GROUP), dtype=np.uint8)
    for n in range(N):
        row = x[n]
        nib = np.zeros(C, dtype=np.uint8)
        for g in range(C // GROUP):
            grp = row[g * GROUP:(g + 1) * GROUP]
            sc = group_scale_code(grp)
            scales[n, g] = sc
            s = E4M3_TABLE[sc]
            if s == 0.0:
                continue
            for i in range(GROUP):
                nib[g * GROUP + i] = e2m1_encode(grp[i], s)
        codes[n] = nib[0::2] | (nib[1::2] << 4)
    return codes, scales


def quantize_rows_fast(x, chunk: int = 8192) -> tuple:
    """Vectorised form of quantize_rows with the same rules (large inputs).

    It is checked against the element-by-element form in the tests.
    """
    x = np.asarray(x, dtype=np.float32)
    if x.shape[0] > chunk:
        parts = [_quantize_block(x[i:i + chunk]) for i in range(0, x.shape[0], chunk)]
        return (np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts]))
    return _quantize_block(x)


def _quantize_block(x) -> tuple:
    N, C = x.shape
    G = C // GROUP
    grp = x.reshape(N, G, GROUP)
    amax = np.max(np.abs(grp), axis=2).astype(np.float32)
    ratio = (amax / np.float32(6.0)).astype(np.float32).astype(np.float64)
    # E4M3 RNE over the ordered value list.
    pos = _E4M3_POS
    k = np.searchsorted(pos, ratio, side="left")
    k = np.minimum(k, 126)
    lo = np.maximum(k - 1, 0)
    vk = pos[k]
    vlo = pos[lo]
    exact = vk == ratio
    dlo = ratio - vlo
    dhi = vk - ratio
    pick_lo = (dlo < dhi) | ((dlo == dhi) & (lo % 2 == 0))
    sc = np.where(exact, k, np.where(pick_lo, lo, k))
    sc = np.where(ratio >= pos[-1], 126, sc)
    sc = np.where(ratio == 0.0, 0, sc).astype(np.uint8)
    s = E4M3_TABLE[sc][:, :, None]  # [N, G, 1]
    ax = np.abs(grp).astype(np.float64)
    mids = s * _E2M1_MID[None, None, :]  # [N, G, 7] broadcast per element below
    gt = (ax[..., None] > mids[:, :, None, :])  # [N, G, 16, 7]
    eq = (ax[..., None] == mids[:, :, None, :])
    kk = np.sum(gt, axis=-1)  # magnitudes strictly above midpoints
    tie = np.any(eq, axis=-1)
    # On a tie with midpoint j (= kk), choose the even one of j, j+1.
    kk = np.where(tie & (kk % 2 == 1), kk + 1, kk)
    kk = np.where(s == 0.0, 0, kk)
    nib = np.where((kk > 0) & (grp < 0), kk | 0x8, kk).astype(np.uint8).reshape(N, C)
    codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    return codes, sc.reshape(N, G)


def dequantize_rows(codes, scales) -> np.ndarray:
    """(codes [N, C/2], scales [N, C/16]) -> fp64 latent [N, C]."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    N, half = codes.shape
    C = half * 2
    nib = np.empty((N, C), dtype=np.uint8)
    nib[:, 0::2] = codes & 0xF
    nib[:, 1::2] = codes >> 4
    vals = E2M1_TABLE[nib]
    s = np.repeat(E4M3_TABLE[scales], GROUP, axis=1)
    return vals * s


def entry_bytes(latent_dim: int) -> int:
    """Bytes of one quantised latent entry: 4-bit codes plus one scale byte per group."""
    return latent_dim // 2 + latent_dim // GROUP
