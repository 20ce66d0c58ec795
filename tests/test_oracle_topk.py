"""Pins for the oracle's Top-K sparse attention ([FlexGen] section 5, sparse
attention: per query the indices of its Top-K tokens in the K cache, the
other tokens dropped, only those V rows read).

Pins: Top-K over every token is dense attention (bitwise); Top-1 returns the
best key's value exactly; on small integer data (exact scores, many ties) the
kept set is the one a brute force over all subsets picks (largest score sum,
then the lowest indices); a zero query keeps the first tokens; changing a
dropped token leaves the output unchanged; the 10% count.
"""
import itertools

import numpy as np
import pytest

import synth

SEED = synth.seed_for(80)


def _qkv(T, d, stream):
    q = synth.normal_f16(SEED, stream, (d,))
    k = synth.normal_f16(SEED, stream + 1, (T, d))
    v = synth.normal_f16(SEED, stream + 2, (T, d))
    return q, k, v


def _exact_scores(q, k):
    """Integer-valued q, k: exact scores with Python integers."""
    qi = [int(x) for x in q]
    return [sum(a * int(b) for a, b in zip(qi, row)) for row in k]


@pytest.mark.parametrize("T", [1, 7, 64, 129])
def test_topk_all_is_dense(orc, T):
    q, k, v = _qkv(T, 64, 10 + T)
    out, kept = orc.topk_attention(q, k, v, T)
    dense = orc.attention(q[None], k, v, [T])[0]
    assert list(kept) == list(range(T))
    assert np.array_equal(out.view(np.uint16), dense.view(np.uint16))


def test_top1_is_best_value(orc):
    q, k, v = _qkv(200, 128, 30)
    out, kept = orc.topk_attention(q, k, v, 1)
    best = int(np.argmax(k.astype(np.float64) @ q.astype(np.float64)))
    assert list(kept) == [best]
    assert np.array_equal(out.view(np.uint16), v[best].view(np.uint16))


@pytest.mark.parametrize("trial", range(12))
def test_topk_brute_force_small_integer(orc, trial):
    rng = np.random.default_rng(100 + trial)
    T, d = int(rng.integers(2, 10)), 8
    q = rng.integers(-2, 3, d).astype(np.float16)
    k = rng.integers(-2, 3, (T, d)).astype(np.float16)  # scores collide often
    v = rng.standard_normal((T, d)).astype(np.float16)
    z = _exact_scores(q, k)
    for K in range(1, T + 1):
        best = None
        for comb in itertools.combinations(range(T), K):  # lexicographic order
            tot = sum(z[j] for j in comb)
            if best is None or tot > best[0]:
                best = (tot, comb)
        out, kept = orc.topk_attention(q, k, v, K)
        assert tuple(int(j) for j in kept) == best[1], (T, K, z)


def test_zero_query_keeps_first(orc):
    T, d, K = 90, 64, 9
    _, k, v = _qkv(T, d, 40)
    q = np.zeros(d, np.float16)
    out, kept = orc.topk_attention(q, k, v, K)
    assert list(kept) == list(range(K))
    mean = v[:K].astype(np.float64).mean(axis=0)  # equal weights
    assert np.all(np.abs(out.astype(np.float64) - mean) <= 2 ** -10 * np.maximum(1, np.abs(mean)))


def test_dropped_tokens_do_not_matter(orc):
    T, d = 300, 128
    q, k, v = _qkv(T, d, 50)
    K = orc.topk_count(T)
    out, kept = orc.topk_attention(q, k, v, K)
    dropped = np.setdiff1d(np.arange(T), kept)
    k2, v2 = k.copy(), v.copy()
    v2[dropped] = np.float16(1000.0)          # any values
    k2[dropped] = (k2[dropped].astype(np.float32) * 0.25).astype(np.float16)  # lower |scores|
    z = k.astype(np.float64) @ q.astype(np.float64)
    z2 = k2.astype(np.float64) @ q.astype(np.float64)
    assert z2[dropped].max() < z[kept].min()  # still below every kept score
    out2, kept2 = orc.topk_attention(q, k2, v2, K)
    assert list(kept2) == list(kept)
    assert np.array_equal(out.view(np.uint16), out2.view(np.uint16))


def test_topk_count(orc):
    assert [orc.topk_count(T) for T in (1, 9, 10, 11, 528, 2112)] == [1, 1, 1, 2, 53, 212]
