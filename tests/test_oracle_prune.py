"""Pins for the oracle's token-tree pruning and KV compaction.

SpecPipe article, 2.2.1 (sub-tree pruning, Fig. 5-b) and 2.2.2 (Fig. 8):
when token u is verified the tree keeps u's subtree with u as the new root,
and the cache keeps the verified path above u as committed prefix.  Pins:
the article's worked example (tests/golden), closed forms on special trees
(chain, star, root, leaf, one token), the invariant that every kept token
sees exactly the same original tokens as before (committed path plus its new
ancestors), checked against parent walks done here, and the attention of
every kept token being bitwise unchanged by pruning + compaction.
"""
import os

import numpy as np
import pytest

import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    d = {}
    for ln in open(os.path.join(GOLD, "tree_prune_example.txt")):
        if ln.startswith("#") or ":" not in ln:
            continue
        k, v = ln.split(":", 1)
        d[k.strip()] = [int(t) for t in v.split()]
    return d


def _path(parent, i):
    """Tokens from i up to the root (i included), by walking the parent links."""
    out = []
    while i >= 0:
        out.append(int(i))
        i = parent[i]
    return out


def test_prune_page_example(orc):
    g = _golden()
    new_parent, src, kept, depth = orc.tree_prune(g["parent"], g["verified"][0])
    assert depth == g["depth"][0] and kept == len(g["kept"])
    assert list(src[:depth + kept]) == g["rows"]
    assert list(src[depth:depth + kept]) == g["kept"]
    assert all(s == -1 for s in src[depth + kept:])
    assert list(new_parent[:kept]) == g["new_parent"]
    m = orc.tree_masks(new_parent)
    for j in range(kept):
        assert [t for t in range(kept) if (int(m[j]) >> t) & 1] == g[f"row{j}"]


def test_prune_special_trees(orc):
    q = 64
    chain = np.arange(-1, q - 1)
    for u in (0, 17, q - 1):  # a chain: u's ancestors commit, u and below stay as a chain
        new_parent, src, kept, depth = orc.tree_prune(chain, u)
        assert depth == u and kept == q - u and list(src) == list(range(q))
        assert list(new_parent[:kept]) == list(range(-1, kept - 1))
        assert all(p == (0 if kept == 1 else kept - 2) for p in new_parent[kept:])
    star = np.array([-1] + [0] * (q - 1))
    new_parent, src, kept, depth = orc.tree_prune(star, 0)  # root verified: nothing dropped
    assert depth == 0 and kept == q and list(new_parent) == list(star)
    new_parent, src, kept, depth = orc.tree_prune(star, 9)  # a leaf: the root commits
    assert depth == 1 and kept == 1 and list(src[:2]) == [0, 9] and list(new_parent) == [-1] + [0] * (q - 1)
    assert all(s == -1 for s in src[2:])
    new_parent, src, kept, depth = orc.tree_prune(np.array([-1]), 0)
    assert kept == 1 and depth == 0 and list(new_parent) == [-1] and list(src) == [0]
    for bad_parent, u in (([-1, 0, 0], 3), ([-1, 0, 0], -1), ([0, 0], 0), ([-1, 2, 0], 1)):
        with pytest.raises(ValueError):
            orc.tree_prune(np.array(bad_parent), u)


@pytest.mark.parametrize("seed", range(6))
def test_prune_keeps_visible_sets(orc, seed):
    """Every kept token sees the same original tokens after pruning (the committed
    path, now prefix, plus its ancestors in the new tree); the committed rows are u's
    ancestors and the kept tokens are u's subtree, both found by parent walks; the new
    parent array is a valid BFS array (filler leaves included)."""
    q = 64
    parent = synth.bfs_parents(synth.seed_for(40 + seed), 1, q)
    old = orc.tree_masks(parent)
    for u in range(0, q, 7):
        new_parent, src, kept, depth = orc.tree_prune(parent, u)
        above = sorted(set(_path(parent, u)) - {u})
        subtree = sorted(i for i in range(q) if u in _path(parent, i))
        assert [int(s) for s in src[:depth]] == above
        assert [int(s) for s in src[depth:depth + kept]] == subtree and int(src[depth]) == u
        new = orc.tree_masks(new_parent)  # raises if not a valid BFS array
        assert int(new_parent[0]) == -1
        for j in range(kept):
            seen_new = set(above) | {int(src[depth + t]) for t in range(kept)
                                     if (int(new[j]) >> t) & 1}
            seen_old = {i for i in range(q) if (int(old[src[depth + j]]) >> i) & 1}
            assert seen_new == seen_old
        for j in range(kept, q):  # filler slots are leaves: nobody kept sees them
            assert all(not (int(new[t]) >> j) & 1 for t in range(kept))


@pytest.mark.parametrize("fmt", [0, 1])
def test_prune_attention_unchanged(orc, fmt):
    """Attention of each kept token over the compacted cache, with the committed path
    as part of the prefix, equals bit for bit its attention before pruning (the same
    keys, in the same order)."""
    rng = np.random.default_rng(5 + fmt)
    b, H, d, P, q = 2, 2, 64, 70, 24
    kv = orc.KV(fmt, b, H, P + q, d)
    rows = rng.standard_normal((b, H, P + q, d)).astype(np.float16)
    vrows = rng.standard_normal((b, H, P + q, d)).astype(np.float16)
    if fmt == 1:
        kv.k[:], kv.ksm[:] = orc.quantize_g64(rows)
        kv.v[:], kv.vsm[:] = orc.quantize_g64(vrows)
    else:
        kv.k[:] = rows.view(np.uint16)
        kv.v[:] = vrows.view(np.uint16)
    Q = rng.standard_normal((b, H, q, d)).astype(np.float16)
    parents = [synth.bfs_parents(synth.seed_for(60), r, q) for r in range(b)]
    verified = [5, 11]
    before = np.zeros((b, H, q, d), np.float16)
    for r in range(b):
        m = orc.tree_masks(parents[r])
        K, V = kv.values("k", P + q)[r], kv.values("v", P + q)[r]
        for h in range(H):
            before[r, h] = orc.attention(Q[r, h], K[h], V[h], np.full(q, P, np.int32), m, P)
    plans = [orc.tree_prune(parents[r], verified[r]) for r in range(b)]
    src = np.stack([p[1] for p in plans])
    count = np.array([p[2] + p[3] for p in plans])
    orc.kv_compact(kv, P, src, count)
    for r in range(b):
        new_parent, s, k, depth = plans[r]
        assert depth > 0
        m = orc.tree_masks(new_parent)
        K, V = kv.values("k", P + q)[r], kv.values("v", P + q)[r]
        P2 = P + depth
        kept_old = s[depth:depth + k]
        for h in range(H):
            after = orc.attention(Q[r, h, kept_old], K[h], V[h], np.full(k, P2, np.int32), m[:k],
                                  P2)
            assert np.array_equal(after.view(np.uint16), before[r, h, kept_old].view(np.uint16))
