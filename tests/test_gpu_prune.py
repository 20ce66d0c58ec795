"""GPU token-tree pruning and KV compaction against the oracle (SpecPipe
article, 2.2.1 sub-tree pruning, Fig. 5-b; 2.2.2, Fig. 8).

Plans (new prefix length, kept count, old indices, new parents) and
compacted cache rows must be bit-exact; attention of the kept tokens over
the compacted cache, with the committed path as part of each request's own
prefix, is then checked against the oracle within the parity tolerance.
"""
import numpy as np
import pytest

import synth
from helpers import TOL, assert_close, dev, host

pytestmark = pytest.mark.gpu
SEED = synth.seed_for(70)


@pytest.fixture(scope="module")
def hp():
    import torch
    from decode_step_transformer_amd import hp as _hp
    assert torch.cuda.is_available()
    assert _hp.hp_device_check() == 0, _hp.hp_last_error()
    return _hp


def _trees(b, q, stream0):
    return np.stack([synth.bfs_parents(SEED, stream0 + r, q) for r in range(b)]).astype(np.int32)


@pytest.mark.parametrize("b,q", [(8, 1), (8, 5), (8, 64), (37, 64), (16, 33)])
def test_tree_prune_matches_oracle(hp, orc, b, q):
    parent = _trees(b, q, 100 + q)
    verified = (synth.words(SEED, 200 + q, 0, b) % np.uint64(q)).astype(np.int32)
    pos = 123
    new_parent, src, prefix, kept, err = hp.hp_tree_prune(dev(parent), dev(verified), pos)
    new_parent, src, prefix, kept = host(new_parent), host(src), host(prefix), host(kept)
    assert int(host(err)[0]) == 0
    for r in range(b):
        rp, rs, rk, depth = orc.tree_prune(parent[r], int(verified[r]))
        assert int(kept[r]) == rk and int(prefix[r]) == pos + depth
        assert np.array_equal(new_parent[r], rp) and np.array_equal(src[r], rs)


def test_tree_prune_page_example(hp, orc):
    """The SpecPipe article's Fig. 5-b / Fig. 8 example (tests/golden): tau2 verified
    keeps tau2, tau4, tau5 with tau2 as the new root; tau1 commits to the prefix."""
    import os
    g = {}
    for ln in open(os.path.join(os.path.dirname(__file__), "golden", "tree_prune_example.txt")):
        if ln.startswith("#") or ":" not in ln:
            continue
        k, v = ln.split(":", 1)
        g[k.strip()] = [int(t) for t in v.split()]
    parent = np.array([g["parent"]], np.int32)
    new_parent, src, prefix, kept, err = hp.hp_tree_prune(dev(parent), dev(np.array(g["verified"], np.int32)), 10)
    k, dpt = int(host(kept)[0]), g["depth"][0]
    assert int(host(err)[0]) == 0 and k == len(g["kept"]) and int(host(prefix)[0]) == 10 + dpt
    assert list(host(src)[0][:dpt + k]) == g["rows"]
    assert list(host(new_parent)[0][:k]) == g["new_parent"]


def test_tree_masks_many_requests(hp, orc):
    """More requests than waves in the launch; one request with a broken
    entry: its descendants' sets stop at (and include) that entry, the
    entry itself keeps only its own bit (hp_tree_masks contract)."""
    b, q = 37, 64
    parent = _trees(b, q, 800)
    ref = np.stack([orc.tree_masks(p) for p in parent])
    masks, err = hp.hp_tree_masks(dev(parent))
    assert int(host(err)[0]) == 0
    assert np.array_equal(host(masks).view(np.uint64), ref)
    bad = parent.copy()
    bad[20, 10] = 40
    masks, err = hp.hp_tree_masks(dev(bad))
    assert int(host(err)[0]) == 1
    got = host(masks).view(np.uint64)
    assert np.array_equal(np.delete(got, 20, 0), np.delete(ref, 20, 0))
    for i in range(q):  # walk up from i, stopping after the broken entry
        want, t = 0, i
        while True:
            want |= 1 << t
            if t == 10 or bad[20, t] < 0:
                break
            t = int(bad[20, t])
        assert int(got[20, i]) == want, i


def test_tree_prune_rejects_bad_requests(hp, orc):
    q = 8
    parent = _trees(3, q, 300)
    parent[1, 5] = 6                       # parent after its child
    verified = np.array([2, 3, q], np.int32)  # request 2: index out of range
    new_parent, src, prefix, kept, err = hp.hp_tree_prune(dev(parent), dev(verified), 40)
    kept, new_parent, prefix = host(kept), host(new_parent), host(prefix)
    assert int(host(err)[0]) == 2
    ref = orc.tree_prune(parent[0], 2)
    assert list(kept) == [ref[2], 0, 0] and list(prefix) == [40 + ref[3], 40, 40]
    for r in (1, 2):  # a request that keeps nothing gets a valid star
        orc.tree_masks(new_parent[r])


@pytest.mark.parametrize("fmt,heads,h1", [(1, 2, 256), (1, 4, 256), (0, 2, 256), (0, 2, 128)])
def test_kv_compact_matches_oracle(hp, orc, fmt, heads, h1):
    b, pos, q = 3, 37, 64
    D = h1 // heads
    cap = pos + q + 3
    kv = hp.KVCache(fmt, b, heads, cap, D)
    rk = orc.KV(fmt, b, heads, cap, D)
    qkv = synth.normal_f16(SEED, 400 + fmt, (b, pos + q, 3 * h1))
    hp.hp_kv_append(b, pos + q, h1, heads, dev(qkv), 0, kv)
    for which in ("k", "v"):
        setattr(rk, which, host(getattr(kv, which)).copy())
    if fmt == 1:
        rk.ksm, rk.vsm = host(kv.k_sm).copy(), host(kv.v_sm).copy()
    parent = _trees(b, q, 500)
    verified = np.array([0, 9, 63], np.int32)
    new_parent, src, prefix, kept, err = hp.hp_tree_prune(dev(parent), dev(verified), pos)
    hp.hp_kv_compact(b, q, h1, heads, pos, src, prefix, kept, kv)
    orc.kv_compact(rk, pos, host(src), host(prefix) - pos + host(kept))
    pairs = [("k", "k"), ("v", "v")] + ([("k_sm", "ksm"), ("v_sm", "vsm")] if fmt == 1 else [])
    for name, oname in pairs:  # bit patterns, fp16 rows included
        g, r = host(getattr(kv, name)), getattr(rk, oname)
        assert np.array_equal(g.view(np.uint8), r.view(np.uint8)), name


@pytest.mark.parametrize("fmt", [0, 1])
def test_attention_after_pruning(hp, orc, fmt):
    """Kept tokens attend over the compacted cache with the new masks and each
    request's new prefix length (old prefix + committed path): the result matches
    the oracle, and those tokens' attention before pruning within rounding."""
    b, heads, h1, pos, q = 4, 4, 512, 300, 64
    D = h1 // heads
    cap = pos + 2 * q  # the next tree (q slots) starts after the longer prefix
    kv = hp.KVCache(fmt, b, heads, cap, D)
    pre = synth.normal_f16(SEED, 600 + fmt, (b, pos, 3 * h1))
    qkv = synth.normal_f16(SEED, 610 + fmt, (b, q, 3 * h1))
    hp.hp_kv_append(b, pos, h1, heads, dev(pre), 0, kv)
    hp.hp_kv_append(b, q, h1, heads, dev(qkv), pos, kv)
    parent = _trees(b, q, 700)
    masks, _ = hp.hp_tree_masks(dev(parent))
    before = host(hp.hp_decode_attention(b, q, h1, heads, dev(qkv), pos, kv, masks=masks))
    verified = np.array([0, 3, 20, 63], np.int32)
    new_parent, src, prefix, kept, err = hp.hp_tree_prune(dev(parent), dev(verified), pos)
    hp.hp_kv_compact(b, q, h1, heads, pos, src, prefix, kept, kv)
    new_masks, e2 = hp.hp_tree_masks(new_parent)
    assert int(host(e2)[0]) == 0
    srch, kepth, preh = host(src), host(kept), host(prefix)
    qkv2 = np.zeros_like(qkv)
    kept_old = []
    for r in range(b):  # queries of the kept tokens, in their new slots
        dpt = int(preh[r]) - pos
        kept_old.append(srch[r, dpt:dpt + kepth[r]])
        qkv2[r, :kepth[r]] = qkv[r, kept_old[r]]
    assert int(preh.max()) > pos  # some request committed rows
    after = host(hp.hp_decode_attention_ragged(b, q, h1, heads, dev(qkv2), prefix, pos + q - 1, kv,
                                               masks=new_masks))
    ok = orc.KV(fmt, b, heads, cap, D)
    for name, oname in (("k", "k"), ("v", "v")) + ((("k_sm", "ksm"), ("v_sm", "vsm")) if fmt else ()):
        setattr(ok, oname, host(getattr(kv, name)).copy())
    Kc, Vc = ok.values("k", cap), ok.values("v", cap)
    nm = orc.tree_masks
    for r in range(b):
        k, P2 = int(kepth[r]), int(preh[r])
        m = nm(host(new_parent)[r])[:k]
        for h in range(heads):
            ref = orc.attention(qkv2[r, :k, h * D:(h + 1) * D], Kc[r, h], Vc[r, h],
                                np.full(k, P2, np.int32), m, P2)
            assert_close(after[r, :k, h * D:(h + 1) * D], ref, what=f"r{r} h{h}")
        # the same tokens before pruning, within the tolerance (block boundaries moved)
        assert_close(after[r, :k], before[r, kept_old[r]], tol=TOL, what=f"r{r} before/after")


@pytest.mark.parametrize("fmt,q", [(1, 64), (1, 4), (0, 64), (0, 4)])
def test_ragged_attention_matches_oracle(hp, orc, fmt, q):
    """Per-request prefix lengths (ragged, not multiples of 64, one of them 0): each
    request's queries see its own prefix plus its tree rows, on both the multi-query
    (q >= 16, int4) and the streaming kernels."""
    b, heads, h1, cap = 5, 2, 256, 400
    D = h1 // heads
    plen = np.array([0, 1, 77, 200, cap - q], np.int32)
    kv = hp.KVCache(fmt, b, heads, cap, D)
    rows = synth.normal_f16(SEED, 650 + fmt, (b, cap, 3 * h1))
    hp.hp_kv_append(b, cap, h1, heads, dev(rows), 0, kv)
    qkv = synth.normal_f16(SEED, 660 + fmt, (b, q, 3 * h1))
    parent = _trees(b, q, 900 + q)
    masks, _ = hp.hp_tree_masks(dev(parent))
    out = host(hp.hp_decode_attention_ragged(b, q, h1, heads, dev(qkv), dev(plen), cap - q, kv,
                                             masks=masks))
    ok = orc.KV(fmt, b, heads, cap, D)
    for name, oname in (("k", "k"), ("v", "v")) + ((("k_sm", "ksm"), ("v_sm", "vsm")) if fmt else ()):
        setattr(ok, oname, host(getattr(kv, name)).copy())
    Kc, Vc = ok.values("k", cap), ok.values("v", cap)
    for r in range(b):
        m = orc.tree_masks(parent[r])
        P = int(plen[r])
        for h in range(heads):
            ref = orc.attention(qkv[r, :, h * D:(h + 1) * D], Kc[r, h], Vc[r, h],
                                np.full(q, P, np.int32), m, P)
            assert_close(out[r, :, h * D:(h + 1) * D], ref, what=f"r{r} h{h} P{P}")
