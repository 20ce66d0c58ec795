"""Pins for the oracle's layer prefill/decode, tree masks and block schedule.

FlexGen paper notes, background section: prefill and decode equations of one
layer; section 4: Algorithm 1 (block schedule).  SpecPipe article, 2.2.1:
tree tokens see themselves and their ancestors.
Pins: special weights that reduce the layer to closed forms (zero values,
uniform attention = running mean), the page's literal single-head unmasked
formula built from library routines, prefill/decode consistency, the page's
tree example, and schedule invariance.
"""
import os

import numpy as np
import pytest
import scipy.special

import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def f16(rng, shape, s=1.0):
    return (rng.standard_normal(shape) * s).astype(np.float16)


def weights(rng, h1, h2, s=0.05):
    return {"wq": f16(rng, (h1, h1), s), "wk": f16(rng, (h1, h1), s), "wv": f16(rng, (h1, h1), s),
            "wo": f16(rng, (h1, h1), s), "w1": f16(rng, (h1, h2), s), "w2": f16(rng, (h2, h1), s)}


def ulps(a, b):
    ai = a.view(np.uint16).astype(np.int32)
    bi = b.view(np.uint16).astype(np.int32)
    ai = np.where(ai & 0x8000, 0x8000 - ai, ai)
    bi = np.where(bi & 0x8000, 0x8000 - bi, bi)
    return np.abs(ai - bi)


def r16(a):
    return np.asarray(a, np.float64).astype(np.float16)


@pytest.mark.parametrize("fmt", [0, 1])
def test_zero_values_pass_through(orc, fmt):
    """wV = 0 and w2 = 0: attention adds nothing and the MLP adds nothing, so x' = x."""
    rng = np.random.default_rng(20)
    b, s, h1, h2, H = 2, 9, 128, 192, 2
    W = weights(rng, h1, h2)
    W["wv"] = np.zeros_like(W["wv"])
    W["w2"] = np.zeros_like(W["w2"])
    x = f16(rng, (b, s, h1))
    kv = orc.KV(fmt, b, H, s + 1, h1 // H)
    y = orc.layer_prefill(x, W, kv, H)
    assert np.array_equal(y.view(np.uint16), x.view(np.uint16))
    t = f16(rng, (b, 1, h1))
    assert np.array_equal(orc.layer_decode(t, W, kv, H, s).view(np.uint16), t.view(np.uint16))


@pytest.mark.parametrize("heads", [1, 2])
def test_uniform_attention_closed_form(orc, heads):
    """wQ = wK = 0 makes every score 0, so causal attention is the running mean of V.
    With wV = wO = w1 = w2 = I: x_out = mean_{j<=i} x_j + x_i and x' = relu(x_out) + x_out."""
    rng = np.random.default_rng(21)
    b, s, h1 = 2, 12, 128
    eye = np.eye(h1, dtype=np.float16)
    W = {"wq": np.zeros((h1, h1), np.float16), "wk": np.zeros((h1, h1), np.float16),
         "wv": eye, "wo": eye, "w1": eye, "w2": eye}
    x = f16(rng, (b, s, h1))
    kv = orc.KV(0, b, heads, s, h1 // heads)
    y = orc.layer_prefill(x, W, kv, heads)
    xd = x.astype(np.float64)
    mean = np.cumsum(xd, 1) / np.arange(1, s + 1)[None, :, None]
    xo = r16(r16(mean).astype(np.float64) + xd)
    ref = r16(r16(np.maximum(xo.astype(np.float64), 0)).astype(np.float64) + xo.astype(np.float64))
    assert ulps(y, ref).max() <= 1


def test_literal_single_head_unmasked(orc):
    """heads = 1, no mask: the page's formula softmax(xQ xK^T/sqrt(h1)) xV wO + x, then the MLP."""
    rng = np.random.default_rng(22)
    b, s, h1, h2 = 1, 10, 64, 128
    W = weights(rng, h1, h2, 0.2)
    x = f16(rng, (b, s, h1))
    kv = orc.KV(0, b, 1, s, h1)
    y = orc.layer_prefill(x, W, kv, 1, causal=False)
    X = x[0].astype(np.float64)
    w = {k: v.astype(np.float64) for k, v in W.items()}
    Q, K, V = (r16(X @ w["wq"]).astype(np.float64), r16(X @ w["wk"]).astype(np.float64),
               r16(X @ w["wv"]).astype(np.float64))
    A = r16(scipy.special.softmax(Q @ K.T / np.sqrt(h1), axis=-1) @ V).astype(np.float64)
    XO = r16(A @ w["wo"] + X).astype(np.float64)
    HD = r16(np.maximum(XO @ w["w1"], 0)).astype(np.float64)
    ref = r16(HD @ w["w2"] + XO)
    assert ulps(y[0], ref).max() <= 2


def test_prefill_then_decode_equals_longer_prefill(orc):
    """Causal reading: prefill(s) then decode(token s) == row s of prefill(s + 1) (fp16 cache)."""
    rng = np.random.default_rng(23)
    b, s, h1, h2, H = 2, 11, 128, 256, 2
    W = weights(rng, h1, h2)
    x = f16(rng, (b, s + 1, h1))
    kv_a = orc.KV(0, b, H, s + 1, h1 // H)
    ya = orc.layer_prefill(x, W, kv_a, H)
    kv_b = orc.KV(0, b, H, s + 1, h1 // H)
    orc.layer_prefill(x[:, :s], W, kv_b, H)
    yb = orc.layer_decode(x[:, s:], W, kv_b, H, s)
    assert np.array_equal(ya[:, s:].view(np.uint16), yb.view(np.uint16))
    assert np.array_equal(kv_a.k, kv_b.k) and np.array_equal(kv_a.v, kv_b.v)


def test_prefill_one_token_equals_first_decode(orc):
    rng = np.random.default_rng(24)
    b, h1, h2, H = 3, 128, 128, 1
    W = weights(rng, h1, h2)
    x = f16(rng, (b, 1, h1))
    for fmt in (0, 1):
        ka, kb = orc.KV(fmt, b, H, 4, h1), orc.KV(fmt, b, H, 4, h1)
        ya = orc.layer_prefill(x, W, ka, H)
        yb = orc.layer_decode(x, W, kb, H, 0)
        assert np.array_equal(ka.k, kb.k) and np.array_equal(ka.v, kb.v)
        if fmt == 0:   # fresh fp16 K/V and stored fp16 K/V are the same values
            assert np.array_equal(ya.view(np.uint16), yb.view(np.uint16))


def test_int4_cache_close_to_fp16_cache(orc):
    rng = np.random.default_rng(25)
    b, s, h1, h2, H = 2, 16, 128, 128, 2
    W = weights(rng, h1, h2)
    x = f16(rng, (b, s, h1))
    t = f16(rng, (b, 1, h1))
    outs = []
    for fmt in (0, 1):
        kv = orc.KV(fmt, b, H, s + 1, h1 // H)
        orc.layer_prefill(x, W, kv, H)
        outs.append(orc.layer_decode(t, W, kv, H, s).astype(np.float64))
    assert np.abs(outs[0] - outs[1]).max() < 0.05


def test_cache_rows_hold_quantised_kv(orc):
    """Stored rows are the quantised x·wK and x·wV, grouped 64 along the hidden dim, head-major."""
    rng = np.random.default_rng(26)
    b, s, h1, h2, H = 2, 5, 256, 128, 2
    W = weights(rng, h1, h2)
    x = f16(rng, (b, s, h1))
    kv = orc.KV(1, b, H, s + 3, h1 // H)
    orc.layer_prefill(x, W, kv, H)
    Kx = x.reshape(b * s, h1).astype(np.float64) @ W["wk"].astype(np.float64)
    K16 = r16(Kx).reshape(b, s, H, h1 // H).transpose(0, 2, 1, 3)
    y = kv.values("k", s).astype(np.float64)
    S = np.abs(K16.astype(np.float64)).max() * 2 / 15
    assert np.abs(y - K16).max() <= S
    assert (kv.k[:, :, s:] == 0).all()


# ---------------------------------------------------------------- tree masks
def _golden_tree():
    d = {}
    for ln in open(os.path.join(GOLD, "tree_page_example.txt")):
        if ln.startswith("#") or ":" not in ln:
            continue
        k, v = ln.split(":", 1)
        d[k.strip()] = [int(t) for t in v.split()]
    return d


def test_tree_page_example(orc):
    g = _golden_tree()
    m = orc.tree_masks(g["parent"])
    for i in range(5):
        assert [u for u in range(5) if (int(m[i]) >> u) & 1] == g[f"row{i}"]


def test_tree_chain_and_star(orc):
    q = 64
    chain = orc.tree_masks(np.arange(-1, q - 1))
    assert [int(v) for v in chain] == [(1 << (i + 1)) - 1 for i in range(q)]
    star = orc.tree_masks(np.array([-1] + [0] * (q - 1)))
    assert int(star[0]) == 1 and all(int(star[i]) == 1 | (1 << i) for i in range(1, q))
    for bad in ([0, 0], [-1, 1], [-1, -2, 0], [-1, 0, 3]):
        with pytest.raises(ValueError):
            orc.tree_masks(np.array(bad))


@pytest.mark.parametrize("fmt", [0, 1])
def test_chain_tree_equals_sequential_decode(orc, fmt):
    """A chain tree of nq tokens == nq single-token decode steps (same cache rows)."""
    rng = np.random.default_rng(27)
    b, s, h1, h2, H, nq = 2, 6, 128, 128, 2, 5
    W = weights(rng, h1, h2)
    x = f16(rng, (b, s, h1))
    t = f16(rng, (b, nq, h1))
    ka, kb = orc.KV(fmt, b, H, s + nq, h1 // H), orc.KV(fmt, b, H, s + nq, h1 // H)
    orc.layer_prefill(x, W, ka, H)
    orc.layer_prefill(x, W, kb, H)
    masks = np.tile(orc.tree_masks(np.arange(-1, nq - 1)), (b, 1))
    ya = orc.layer_decode(t, W, ka, H, s, masks)
    yb = np.concatenate([orc.layer_decode(t[:, i:i + 1], W, kb, H, s + i) for i in range(nq)], 1)
    assert np.array_equal(ya.view(np.uint16), yb.view(np.uint16))
    assert np.array_equal(ka.k, kb.k) and np.array_equal(ka.v, kb.v)
    yc = orc.layer_decode(t, W, orc.KV(fmt, b, H, s + nq, h1 // H), H, s)  # masks=None is a chain
    assert yc.shape == ya.shape


def test_tree_token_ignores_other_branches(orc):
    """Changing a token outside i's ancestor set leaves token i's output unchanged."""
    rng = np.random.default_rng(28)
    b, s, h1, h2, H = 1, 4, 128, 128, 2
    parent = np.array([-1, 0, 0, 1, 1, 2])
    masks = orc.tree_masks(parent)[None]
    W = weights(rng, h1, h2)
    x = f16(rng, (b, s, h1))
    t = f16(rng, (b, 6, h1))
    t2 = t.copy()
    t2[0, 2] = f16(rng, (h1,))  # tau3: not an ancestor of tokens 1, 3, 4
    outs = []
    for tt in (t, t2):
        kv = orc.KV(1, b, H, s + 6, h1 // H)
        orc.layer_prefill(x, W, kv, H)
        outs.append(orc.layer_decode(tt, W, kv, H, s, masks))
    for i in (0, 1, 3, 4):
        assert np.array_equal(outs[0][0, i].view(np.uint16), outs[1][0, i].view(np.uint16))
    assert not np.array_equal(outs[0][0, 5].view(np.uint16), outs[1][0, 5].view(np.uint16))


# ------------------------------------------------------------- block schedule
@pytest.mark.parametrize("fmt", [0, 1])
def test_schedule_invariance(orc, fmt):
    """Zig-zag (any GPU batch size) and row-by-row orders give bitwise-equal results."""
    rng = np.random.default_rng(29)
    b, s, n, h1, h2, l, H = 4, 6, 3, 128, 128, 2, 2
    layers = [weights(rng, h1, h2) for _ in range(l)]
    x = f16(rng, (b, s, h1))
    t = f16(rng, (n, b, h1))
    ref = None
    for gbs, order in ((4, 0), (2, 0), (1, 0), (2, 1), (1, 1)):
        kvs = [orc.KV(fmt, b, H, s + n, h1 // H) for _ in range(l)]
        xo, to = orc.run_block(x, t, layers, kvs, H, gbs, order)
        got = (xo.view(np.uint16), to.view(np.uint16), [k.k for k in kvs], [k.v for k in kvs])
        if ref is None:
            ref = got
        else:
            assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])
            for a, c in zip(got[2] + got[3], ref[2] + ref[3]):
                assert np.array_equal(a, c)


def _diagonal_cells(nb, n):
    """[FlexGen] appendix A.2, Fig. 5, as read here: the iterations of the diagonal
    block schedule, each a list of (GPU batch, step) cells (step 0 is the prefill)."""
    its = []
    for it in range(nb + n):
        its.append([(k, it - k) for k in range(nb) if 0 <= it - k <= n])
    return its


@pytest.mark.parametrize("nb,n", [(1, 3), (2, 8), (4, 2), (6, 3), (40, 8)])
def test_diagonal_schedule_cells(nb, n):
    """Every (batch, step) cell runs exactly once, a batch's steps run in order in
    consecutive iterations, and in steady state an iteration holds one batch at
    every step 0..n: n decode cells, so gbs * n tokens per weight load, the same
    weight reads per token as a zig-zag block of gbs * n requests (the page's
    statement); at most n + 1 batches are live at once, the cache slots needed."""
    its = _diagonal_cells(nb, n)
    cells = [c for it in its for c in it]
    assert sorted(cells) == [(k, i) for k in range(nb) for i in range(n + 1)]
    for k in range(nb):
        when = [t for t, it in enumerate(its) for (kk, i) in it if kk == k]
        assert when == list(range(k, k + n + 1))
    assert max(len(it) for it in its) == min(nb, n + 1)
    for it in its[n:nb]:  # steady state (exists when nb > n)
        assert sorted(i for _, i in it) == list(range(n + 1))


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("b,gbs,n", [(4, 1, 2), (6, 1, 3), (4, 2, 3), (4, 4, 2)])
def test_diagonal_schedule_equals_zigzag(orc, fmt, b, gbs, n):
    """The diagonal order (cache slots reused: the KV arrays hold only min(b/gbs, n+1)
    GPU batches) gives the zig-zag block's outputs bit for bit: requests never
    interact, so only the order of the cells changes."""
    rng = np.random.default_rng(31 + b + n)
    s, h1, h2, l, H = 5, 128, 128, 2, 2
    layers = [weights(rng, h1, h2) for _ in range(l)]
    x = f16(rng, (b, s, h1))
    t = f16(rng, (n, b, h1))
    kz = [orc.KV(fmt, b, H, s + n, h1 // H) for _ in range(l)]
    xz, tz = orc.run_block(x, t, layers, kz, H, gbs, 0)
    slots = min(b // gbs, n + 1) * gbs
    kd = [orc.KV(fmt, slots, H, s + n, h1 // H) for _ in range(l)]
    xd, td = orc.run_block(x, t, layers, kd, H, gbs, 2)
    assert np.array_equal(xd.view(np.uint16), xz.view(np.uint16))
    assert np.array_equal(td.view(np.uint16), tz.view(np.uint16))
    last = (b // gbs - 1) % (slots // gbs)  # the slot of the last batch holds its cache
    for j in range(l):
        assert np.array_equal(kd[j].k[last * gbs:(last + 1) * gbs], kz[j].k[b - gbs:])


def test_block_equals_layer_composition(orc):
    rng = np.random.default_rng(30)
    b, s, n, h1, h2, l, H = 2, 5, 2, 128, 128, 2, 2
    layers = [weights(rng, h1, h2) for _ in range(l)]
    x = f16(rng, (b, s, h1))
    t = f16(rng, (n, b, h1))
    kvs = [orc.KV(1, b, H, s + n, h1 // H) for _ in range(l)]
    xo, to = orc.run_block(x, t, layers, kvs, H, b, 0)
    kv2 = [orc.KV(1, b, H, s + n, h1 // H) for _ in range(l)]
    cur = x
    for j in range(l):
        cur = orc.layer_prefill(cur, layers[j], kv2[j], H)
    assert np.array_equal(cur.view(np.uint16), xo.view(np.uint16))
    for i in range(n):
        cur = t[i][:, None]
        for j in range(l):
            cur = orc.layer_decode(cur, layers[j], kv2[j], H, s + i)
        assert np.array_equal(cur[:, 0].view(np.uint16), to[i].view(np.uint16))


def test_kv_append_layout(orc):
    """Appended rows land head-major at [pos, pos+nq), coded like the quantiser."""
    b, nq, heads, d, pos = 2, 3, 2, 128, 5
    h1 = heads * d
    k = synth.normal_f16(91, 1, (b, nq, h1))
    v = synth.normal_f16(91, 2, (b, nq, h1))
    for fmt in (orc.F16, orc.Q4):
        kv = orc.KV(fmt, b, heads, pos + nq + 1, d)
        orc.kv_append(kv, k, v, pos)
        for r in range(b):
            for h in range(heads):
                for i in range(nq):
                    for name, src in (("k", k), ("v", v)):
                        row = src[r, i, h * d:(h + 1) * d]
                        if fmt == orc.F16:
                            assert np.array_equal(getattr(kv, name)[r, h, pos + i].view(np.float16), row)
                        else:
                            c, sm = orc.quantize_g64(row[None, :])
                            assert np.array_equal(getattr(kv, name)[r, h, pos + i], c[0])
                            assert np.array_equal(getattr(kv, name + "sm")[r, h, pos + i], sm[0])
        assert not getattr(kv, "k")[:, :, :pos].any() and not getattr(kv, "k")[:, :, pos + nq:].any()
