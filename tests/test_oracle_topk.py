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


def _tiny_layer(cid, h1, h2):
    sh = {"wq": (h1, h1), "wk": (h1, h1), "wv": (h1, h1), "wo": (h1, h1), "w1": (h1, h2),
          "w2": (h2, h1)}
    return {k: synth.normal_f16(SEED, 900 + 10 * cid + i, v, 0.05) for i, (k, v) in enumerate(sh.items())}


@pytest.mark.parametrize("fmt", [0, 1])
def test_layer_decode_topk_all_rows_is_layer_decode(orc, fmt):
    """With every row kept, the composed sparse decode step is the oracle's
    dense decode step bit for bit (outputs and the appended cache rows)."""
    b, s, h1, h2, heads = 2, 9, 128, 256, 2
    W = _tiny_layer(0, h1, h2)
    x = synth.normal_f16(SEED, 950, (b, s, h1))
    t = synth.normal_f16(SEED, 951, (b, 1, h1))
    kva, kvb = (orc.KV(fmt, b, heads, s + 1, h1 // heads) for _ in range(2))
    orc.layer_prefill(x, W, kva, heads)
    orc.layer_prefill(x, W, kvb, heads)
    ya = orc.layer_decode_topk(t, W, kva, heads, s, topk=10 ** 6)
    yb = orc.layer_decode(t, W, kvb, heads, s)
    assert np.array_equal(ya.view(np.uint16), yb.view(np.uint16))
    assert np.array_equal(kva.k, kvb.k) and np.array_equal(kva.v, kvb.v)


def test_run_block_topk_all_rows_is_run_block(orc):
    b, s, n, h1, h2, heads, l = 2, 6, 3, 128, 256, 2, 2
    Ws = [_tiny_layer(j, h1, h2) for j in range(l)]
    x = synth.normal_f16(SEED, 960, (b, s, h1))
    t = synth.normal_f16(SEED, 961, (n, b, h1))
    ka = [orc.KV(1, b, heads, s + n, h1 // heads) for _ in range(l)]
    kb = [orc.KV(1, b, heads, s + n, h1 // heads) for _ in range(l)]
    xa, ta = orc.run_block_topk(x, t, Ws, ka, heads, topk=10 ** 6)
    xb, tb = orc.run_block(x, t, Ws, kb, heads, b)
    assert np.array_equal(xa.view(np.uint16), xb.view(np.uint16))
    assert np.array_equal(ta.view(np.uint16), tb.view(np.uint16))


def test_layer_decode_topk_uses_kept_rows_only(orc):
    """With K < T, the step's attention output changes only through the kept
    rows: perturbing a dropped row's V leaves the output bitwise unchanged."""
    b, s, h1, h2, heads = 1, 40, 128, 256, 2
    W = _tiny_layer(1, h1, h2)
    x = synth.normal_f16(SEED, 970, (b, s, h1))
    t = synth.normal_f16(SEED, 971, (b, 1, h1))
    kva, kvb = (orc.KV(0, b, heads, s + 1, h1 // heads) for _ in range(2))
    orc.layer_prefill(x, W, kva, heads)
    orc.layer_prefill(x, W, kvb, heads)
    # the kept rows of head 0 and 1 (same query as the step will form)
    q = orc.gemm(t.reshape(b, h1), W["wq"])
    kn = orc.gemm(t.reshape(b, h1), W["wk"])
    K = orc.topk_count(s + 1)
    d = h1 // heads
    keys = np.concatenate([kva.values("k", s)[0], kn.reshape(1, heads, 1, d).repeat(1, 0)[0]], axis=1)
    kept = set()
    for h in range(heads):
        z = keys[h].astype(np.float64) @ q[0, h * d:(h + 1) * d].astype(np.float64)
        kept |= {int(j) for j in np.argsort(-z, kind="stable")[:K]}
    row = next(j for j in range(s) if j not in kept)
    kvb.v[0, :, row] = np.float16(7.0).view(np.uint16)
    ya = orc.layer_decode_topk(t, W, kva, heads, s)
    yb = orc.layer_decode_topk(t, W, kvb, heads, s)
    assert np.array_equal(ya.view(np.uint16), yb.view(np.uint16))
