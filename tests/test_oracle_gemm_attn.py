"""Pins for the oracle's matrix product and attention.

Matrix product (FlexGen paper notes, background section: every projection is
x·w): pinned to exact rational arithmetic on tiny shapes and to numpy's
float64 matmul followed by numpy's binary16 rounding.
Attention (same section: softmax(q k^T / sqrt(.)) v): pinned to closed forms
(one key returns its value; equal values return that value), to PyTorch's
scaled_dot_product_attention in float64 with explicit masks, and to key
permutation invariance.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch


def f16(rng, shape, s=1.0):
    return (rng.standard_normal(shape) * s).astype(np.float16)


def ulps(a, b):
    ai = a.view(np.uint16).astype(np.int32)
    bi = b.view(np.uint16).astype(np.int32)
    ai = np.where(ai & 0x8000, 0x8000 - ai, ai)
    bi = np.where(bi & 0x8000, 0x8000 - bi, bi)
    return np.abs(ai - bi)


@pytest.mark.parametrize("relu,res", [(False, False), (True, False), (False, True)])
def test_gemm_vs_numpy(orc, relu, res):
    rng = np.random.default_rng(10)
    x = f16(rng, (37, 192))
    w = f16(rng, (192, 130), 0.1)
    r = f16(rng, (37, 130)) if res else None
    y = orc.gemm(x, w, r, relu)
    acc = x.astype(np.float64) @ w.astype(np.float64)
    if relu:
        acc = np.maximum(acc, 0)
    if res:
        acc = acc + r.astype(np.float64)
    ref = acc.astype(np.float16)
    u = ulps(y, ref)
    assert u.max() <= 1 and (u > 0).mean() < 1e-3


def test_gemm_exact_rational(orc):
    rng = np.random.default_rng(11)
    x = f16(rng, (3, 9))
    w = f16(rng, (9, 4))
    r = f16(rng, (3, 4))
    y = orc.gemm(x, w, r)
    for m in range(3):
        for n in range(4):
            ex = sum(Fraction(float(x[m, k])) * Fraction(float(w[k, n])) for k in range(9))
            ex += Fraction(float(r[m, n]))
            ref = np.float64(ex).astype(np.float16)   # binary64 then binary16: ties impossible here
            assert ulps(y[m:m + 1, n], np.array([ref])).max() <= 1


def test_gemm_rows_independent(orc):
    rng = np.random.default_rng(12)
    x = f16(rng, (16, 64))
    w = f16(rng, (64, 64))
    y = orc.gemm(x, w)
    assert np.array_equal(orc.gemm(x[5:9], w).view(np.uint16), y[5:9].view(np.uint16))


def test_single_key_returns_value(orc):
    rng = np.random.default_rng(13)
    q, k, v = f16(rng, (1, 128)), f16(rng, (1, 128)), f16(rng, (1, 128))
    out = orc.attention(q, k, v, [1])
    assert np.array_equal(out.view(np.uint16), v.view(np.uint16))


def test_uniform_values(orc):
    rng = np.random.default_rng(14)
    q, k = f16(rng, (8, 64)), f16(rng, (50, 64))
    v = np.repeat(f16(rng, (1, 64)), 50, 0)
    out = orc.attention(q, k, v, [50] * 8)
    assert np.array_equal(out.view(np.uint16), np.repeat(v[:1], 8, 0).view(np.uint16))


def _sdpa(q, k, v, allowed):
    qt = torch.from_numpy(q.astype(np.float64))[None, None]
    kt = torch.from_numpy(k.astype(np.float64))[None, None]
    vt = torch.from_numpy(v.astype(np.float64))[None, None]
    m = torch.from_numpy(allowed)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m)
    return o[0, 0].numpy().astype(np.float16)


@pytest.mark.parametrize("d", [64, 128])
def test_causal_vs_torch_sdpa(orc, d):
    rng = np.random.default_rng(15 + d)
    T = 70
    q, k, v = f16(rng, (T, d), 2.0), f16(rng, (T, d), 2.0), f16(rng, (T, d))
    out = orc.attention(q, k, v, np.arange(1, T + 1))
    ref = _sdpa(q, k, v, np.tril(np.ones((T, T), bool)))
    assert ulps(out, ref).max() <= 1


def test_prefix_plus_mask_vs_torch_sdpa(orc):
    rng = np.random.default_rng(16)
    P, nq, d = 40, 7, 64
    q, k, v = f16(rng, (nq, d)), f16(rng, (P + nq, d)), f16(rng, (P + nq, d))
    mask = rng.integers(0, 2 ** nq, nq).astype(np.uint64)
    allowed = np.zeros((nq, P + nq), bool)
    allowed[:, :P] = True
    for i in range(nq):
        for u in range(nq):
            allowed[i, P + u] = bool((int(mask[i]) >> u) & 1)
    out = orc.attention(q, k, v, [P] * nq, mask, P)
    assert ulps(out, _sdpa(q, k, v, allowed)).max() <= 1


def test_key_permutation_invariance(orc):
    rng = np.random.default_rng(17)
    q, k, v = f16(rng, (4, 64)), f16(rng, (33, 64)), f16(rng, (33, 64))
    p = rng.permutation(33)
    a = orc.attention(q, k, v, [33] * 4)
    b = orc.attention(q, k[p], v[p], [33] * 4)
    assert ulps(a, b).max() <= 1
