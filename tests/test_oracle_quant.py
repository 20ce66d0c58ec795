"""Pins for the oracle's int4 group-64 quantiser and dequantiser.

FlexGen paper notes, section 5: a group of 64 consecutive elements is coded as
round((x - min) / (max - min) * 15) and converted back to FP16 before use.
The pins below come from that definition, not from the oracle's code:
brute-force nearest level, hand-worked groups, degenerate groups and the
error bound of rounding to the nearest of 16 evenly spaced levels.
"""
import os

import numpy as np
import pytest

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def unpack(codes):
    lo = codes & 15
    hi = codes >> 4
    return np.stack([lo, hi], axis=-1).reshape(codes.shape[:-1] + (codes.shape[-1] * 2,))


def _groups(seed, n):
    rng = np.random.default_rng(seed)
    a = (rng.standard_normal((n, 64))).astype(np.float16)
    b = (rng.standard_normal((n, 64)) * 0.02).astype(np.float16)
    c = rng.uniform(-3, 7, (n, 64)).astype(np.float16)
    d = rng.choice(np.array([-1.5, 0.25, 3.0, 3.0078125], np.float16), (n, 64))
    return np.concatenate([a, b, c, d])


def test_golden_group(orc):
    lines = {}
    for ln in open(os.path.join(GOLD, "q4_group_example.txt")):
        if ln.startswith("#") or ":" not in ln:
            continue
        k, v = ln.split(":", 1)
        lines[k.strip()] = v.split()
    x = (-1 + (np.arange(64) % 16) * 0.125).astype(np.float16)[None]
    codes, sm = orc.quantize_g64(x)
    assert unpack(codes)[0].tolist() == [int(v) for v in lines["codes"]]
    assert codes[0].tolist() == [int(v) for v in lines["bytes"]]
    assert sm[0, 0, 0] == int(lines["scale_bits"][0], 16)
    assert sm[0, 0, 1] == int(lines["min_bits"][0], 16)


def test_nearest_level_brute_force(orc):
    """code = the nearest of the 16 levels min + c (max-min)/15, except at near-ties."""
    x = _groups(3, 4000)
    codes, sm = orc.quantize_g64(x)
    c = unpack(codes).astype(np.int64)
    xd = x.astype(np.float64)
    mn = xd.min(1, keepdims=True)
    mx = xd.max(1, keepdims=True)
    levels = mn + np.arange(16)[None, :] * (mx - mn) / 15.0         # [n][16]
    dist = np.abs(xd[:, :, None] - levels[:, None, :])               # [n][64][16]
    best = dist.argmin(-1)
    t = (xd - mn) / (mx - mn) * 15.0
    near_tie = np.abs(t - np.floor(t) - 0.5) < 1e-5
    bad = (best != c) & ~near_tie
    assert not bad.any(), np.argwhere(bad)[:5]
    assert near_tie.mean() < 1e-3


def test_stored_scale_and_min(orc):
    x = _groups(4, 500)
    _, sm = orc.quantize_g64(x)
    xd = x.astype(np.float64)
    mn = x.min(1)
    rng32 = (x.max(1).astype(np.float32) - mn.astype(np.float32))
    assert np.array_equal(sm[:, 0, 1], mn.view(np.uint16))
    assert np.array_equal(sm[:, 0, 0], (rng32 / np.float32(15)).astype(np.float16).view(np.uint16))
    assert np.all(xd.max(1) > xd.min(1))


def test_degenerate_groups(orc):
    g = np.zeros((6, 64), np.float16)
    g[0] = 2.5                                   # constant
    g[1] = np.where(np.arange(64) % 2, -0.0, 0.0)  # signed zeros only
    g[2] = np.where(np.arange(64) % 3, 1.0, -2.0)  # two values
    g[3] = np.linspace(-1, 1, 64)
    g[3, 5] = np.nan                               # NaN skipped by min/max
    g[4] = np.nan                                  # nothing finite
    g[5] = -0.0
    codes, sm = orc.quantize_g64(g)
    c = unpack(codes)
    assert (c[0] == 0).all() and sm[0, 0, 0] == 0 and sm[0, 0, 1] == np.float16(2.5).view(np.uint16)
    assert (c[1] == 0).all() and sm[1, 0].tolist() == [0, 0]
    assert set(c[2][g[2] == 1.0]) == {15} and set(c[2][g[2] == -2.0]) == {0}
    assert sm[2, 0, 0] == np.float16(np.float32(3.0) / np.float32(15)).view(np.uint16)
    assert c[3, 5] == 0 and c[3, 0] == 0 and c[3, 63] == 15
    assert sm[3, 0, 1] == np.float16(-1.0).view(np.uint16)
    assert (c[4] == 0).all() and sm[4, 0].tolist() == [0, 0]
    assert (c[5] == 0).all() and sm[5, 0].tolist() == [0, 0]


def test_dequant_error_bound(orc):
    """|x - y| <= S/2 plus the fp16 rounding of the scale and of y (S = (max-min)/15)."""
    x = _groups(5, 3000)
    codes, sm = orc.quantize_g64(x)
    y = orc.dequantize_g64(codes, sm).astype(np.float64)
    xd = x.astype(np.float64)
    S = (xd.max(1, keepdims=True) - xd.min(1, keepdims=True)) / 15.0
    bound = (0.5 + 2.0 ** -17 + 15 * 2.0 ** -11) * S + 2.0 ** -11 * np.abs(y) + 2.0 ** -25
    assert np.all(np.abs(xd - y) <= bound)
    # and the exact-level reconstruction error is at most half a step
    c = unpack(codes).astype(np.float64)
    lv = xd.min(1, keepdims=True) + c * S
    assert np.all(np.abs(xd - lv) <= S * (0.5 + 1e-5))


def test_dequant_single_rounding(orc):
    """y = fp16(c*scale + min) with one rounding: equals numpy's direct float64->float16."""
    rng = np.random.default_rng(6)
    codes = rng.integers(0, 256, (200, 32), dtype=np.uint8)
    scale = np.abs(rng.standard_normal(200)).astype(np.float16)
    mn = rng.standard_normal(200).astype(np.float16)
    sm = np.stack([scale.view(np.uint16), mn.view(np.uint16)], -1)[:, None, :]
    y = orc.dequantize_g64(codes, sm)
    c = unpack(codes).astype(np.float64)
    ref = (c * scale.astype(np.float64)[:, None] + mn.astype(np.float64)[:, None]).astype(np.float16)
    assert np.array_equal(y.view(np.uint16), ref.view(np.uint16))


def test_groups_follow_rows(orc):
    """Groups are 64 consecutive elements of the last dimension; rows are independent."""
    x = _groups(7, 10).reshape(20, 128)
    codes, sm = orc.quantize_g64(x)
    c1, s1 = orc.quantize_g64(x.reshape(40, 64))
    assert np.array_equal(codes.reshape(40, 32), c1)
    assert np.array_equal(sm.reshape(40, 1, 2), s1)
