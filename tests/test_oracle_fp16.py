"""Pins for the oracle's binary16 conversions.

numpy's float16 casts are an independent implementation of IEEE 754
binary16 (round to nearest, ties to even, with subnormals); the oracle's own
conversions must agree with them bit for bit.
"""
import numpy as np


def test_h2f_exhaustive(orc):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = orc.h2f(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def _boundary_floats():
    v = [0.0, -0.0, 65504.0, 65519.996, 65520.0, 65536.0, 1e9, -65520.0, np.inf, -np.inf,
         2.0 ** -24, 2.0 ** -25, 2.0 ** -25 * 1.0000001, 3 * 2.0 ** -26, 2.0 ** -14,
         2.0 ** -14 - 2.0 ** -25, 2.0 ** -14 - 2.0 ** -26, 1.0 + 2.0 ** -11,
         1.0 + 3 * 2.0 ** -11, 2049.0, 2051.0, 4097.0, 1e-8, 6e-8]
    # every binary16 tie point between consecutive positive finite values
    h = np.arange(0, 0x7bff, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = (h[:-1] + h[1:]) / 2.0
    return np.concatenate([np.array(v), mids, -mids]).astype(np.float32)


def test_f2h_matches_numpy(orc):
    rng = np.random.default_rng(1)
    parts = [
        _boundary_floats(),
        (rng.standard_normal(1 << 20) * 10.0 ** rng.integers(-9, 6, 1 << 20)).astype(np.float32),
        rng.integers(0, 2 ** 32, 1 << 20, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ]
    f = np.concatenate(parts)
    got = orc.f2h(f)
    ref = f.astype(np.float16).view(np.uint16)
    nan = np.isnan(f)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all((got[nan] & 0x7c00) == 0x7c00) and np.all((got[nan] & 0x3ff) != 0)


def test_d2h_single_rounding(orc):
    # just above a binary16 tie: a double-to-float-to-half route would round
    # to the tie and then to even; the direct rounding goes up.
    d = np.array([1.0 + 2.0 ** -11 + 2.0 ** -40, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11 - 2.0 ** -45])
    assert orc.d2h(d).tolist() == d.astype(np.float16).view(np.uint16).tolist()
    assert orc.d2h(d)[0] == np.float16(1.0 + 2.0 ** -10).view(np.uint16)
    rng = np.random.default_rng(2)
    x = rng.standard_normal(1 << 20) * 10.0 ** rng.integers(-9, 6, 1 << 20)
    assert np.array_equal(orc.d2h(x), x.astype(np.float16).view(np.uint16))
