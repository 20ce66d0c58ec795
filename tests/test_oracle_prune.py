"""Pins for the oracle's token-tree pruning and KV compaction.

SpecPipe article, 2.2.1 (sub-tree pruning, Fig. 5-b) and 2.2.2 (Fig. 8):
when token u is verified the tree keeps u's subtree and the cache keeps the
verified path.  Pins: the article's worked example (tests/golden), closed
forms on special trees (root, leaf of a chain, star), the invariant that
every kept token sees exactly the same original tokens as before, checked
against parent walks done here, and the attention of every kept token being
bitwise unchanged by pruning + compaction.
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
    new_parent, src, kept = orc.tree_prune(g["parent"], g["verified"][0])
    assert kept == len(g["kept"])
    assert list(src[:kept]) == g["kept"]
    assert list(new_parent[:kept]) == g["new_parent"]
    m = orc.tree_masks(new_parent)
    for j in range(kept):
        assert [t for t in range(kept) if (int(m[j]) >> t) & 1] == g[f"row{j}"]


def test_prune_special_trees(orc):
    q = 64
    chain = np.arange(-1, q - 1)
    for u in (0, 17, q - 1):  # a chain keeps everything: ancestors + descendants
        new_parent, src, kept = orc.tree_prune(chain, u)
        assert kept == q and list(src) == list(range(q)) and list(new_parent) == list(chain)
    star = np.array([-1] + [0] * (q - 1))
    new_parent, src, kept = orc.tree_prune(star, 0)  # root verified: nothing dropped
    assert kept == q and list(new_parent) == list(star)
    new_parent, src, kept = orc.tree_prune(star, 9)  # a leaf: root and the leaf
    assert kept == 2 and list(src[:2]) == [0, 9] and list(new_parent[:2]) == [-1, 0]
    assert all(p == 0 for p in new_parent[2:])        # filler leaves under the new root
    new_parent, src, kept = orc.tree_prune(np.array([-1]), 0)
    assert kept == 1 and list(new_parent) == [-1]
    for bad_parent, u in (([-1, 0, 0], 3), ([-1, 0, 0], -1), ([0, 0], 0), ([-1, 2, 0], 1)):
        with pytest.raises(ValueError):
            orc.tree_prune(np.array(bad_parent), u)


@pytest.mark.parametrize("seed", range(6))
def test_prune_keeps_visible_sets(orc, seed):
    """Every kept token sees the same original tokens after pruning, the kept
    set is the verified token's path plus its subtree, and the new parent
    array is a valid BFS array (filler leaves included)."""
    q = 64
    parent = synth.bfs_parents(synth.seed_for(40 + seed), 1, q)
    old = orc.tree_masks(parent)
    for u in range(0, q, 7):
        new_parent, src, kept = orc.tree_prune(parent, u)
        path_u = set(_path(parent, u))
        subtree = {i for i in range(q) if u in _path(parent, i)}
        assert [int(s) for s in src[:kept]] == sorted(path_u | subtree)
        new = orc.tree_masks(new_parent)  # raises if not a valid BFS array
        for j in range(kept):
            seen_new = {int(src[t]) for t in range(kept) if (int(new[j]) >> t) & 1}
            seen_old = {i for i in range(q) if (int(old[src[j]]) >> i) & 1}
            assert seen_new == seen_old
        for j in range(kept, q):  # filler slots are leaves: nobody kept sees them
            assert all(not (int(new[t]) >> j) & 1 for t in range(kept))


@pytest.mark.parametrize("fmt", [0, 1])
def test_prune_attention_unchanged(orc, fmt):
    """Attention of each kept token over the compacted cache equals, bit for
    bit, its attention before pruning (the same keys, in the same order)."""
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
    kept = np.array([p[2] for p in plans])
    orc.kv_compact(kv, P, src, kept)
    for r in range(b):
        new_parent, s, k = plans[r]
        m = orc.tree_masks(new_parent)
        K, V = kv.values("k", P + q)[r], kv.values("v", P + q)[r]
        for h in range(H):
            after = orc.attention(Q[r, h, s[:k]], K[h], V[h], np.full(k, P, np.int32), m[:k], P)
            assert np.array_equal(after.view(np.uint16), before[r, h, s[:k]].view(np.uint16))
