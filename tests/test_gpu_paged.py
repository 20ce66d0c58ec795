"""Paged KV caches and the diagonal block schedule that needs them (FlexGen
paper notes, appendix A.2: the diagonal schedule's peak memory counts every
live request's cache at its current length).

A paged cache stores the same rows as a contiguous one, only elsewhere: the
append and the streaming decode attention must give bit-identical rows and
outputs through a page table.  The diagonal schedule with page pools runs the
same products as with contiguous cache slots, so its outputs must be equal
bit for bit, while its pool holds only the pages of the live requests'
current lengths.
"""
import numpy as np
import pytest

import synth
from helpers import dev, host

pytestmark = pytest.mark.gpu
SEED = synth.seed_for(90)


@pytest.fixture(scope="module")
def hp():
    import torch
    from decode_step_transformer_amd import hp as _hp
    assert torch.cuda.is_available()
    assert _hp.hp_device_check() == 0, _hp.hp_last_error()
    return _hp


def _gather(kv, pages, cap):
    """Paged pool -> contiguous [b][heads][cap][...] through the page table (host)."""
    pr = kv.page_rows
    out = []
    for name in ("k", "v", "k_sm", "v_sm"):
        pool = getattr(kv, name)
        if pool is None:
            out.append(None)
            continue
        p = host(pool)
        rows = [np.concatenate([p[pages[r, j]] for j in range(cap // pr)], axis=1)
                for r in range(pages.shape[0])]
        out.append(np.stack(rows))
    return out


@pytest.mark.parametrize("fmt,heads,h1", [(1, 2, 256), (1, 4, 256), (0, 2, 256), (0, 4, 256)])
def test_paged_cache_matches_contiguous(hp, fmt, heads, h1):
    """Append (prefill rows, then ragged per-request rows) and decode attention (one
    query, and a chain of 4) through a shuffled page table against the contiguous
    cache: identical rows and identical outputs."""
    b, cap, pr = 3, 256, 64
    D = h1 // heads
    ppr = cap // pr
    pool = b * ppr + 2
    perm = synth.words(SEED, 1 + fmt, 0, pool).argsort()[: b * ppr]
    pages = perm.reshape(b, ppr).astype(np.int32)
    paged = hp.KVCache(fmt, b, heads, cap, D, page_rows=pr, pool_pages=pool, pages=dev(pages))
    flat = hp.KVCache(fmt, b, heads, cap, D)
    pre = synth.normal_f16(SEED, 10 + fmt, (b, 150, 3 * h1))
    for kv in (paged, flat):
        hp.hp_kv_append(b, 150, h1, heads, dev(pre), 0, kv)
    rpos = np.array([150, 151, 199], np.int32)  # one more token per request, ragged rows
    tok = synth.normal_f16(SEED, 20 + fmt, (b, 1, 3 * h1))
    for kv in (paged, flat):
        hp.hp_kv_append_ragged(b, 1, h1, heads, dev(tok), dev(rpos), 200, kv)
    got = _gather(paged, pages, cap)
    for g, name in zip(got, ("k", "v", "k_sm", "v_sm")):
        if g is not None:
            assert np.array_equal(g.view(np.uint8), host(getattr(flat, name)).view(np.uint8)), name
    q = dev(tok)
    for kv_a, kv_b in ((paged, flat),):
        a = hp.hp_decode_attention_ragged(b, 1, h1, heads, q, dev(rpos), 200, kv_a)
        c = hp.hp_decode_attention_ragged(b, 1, h1, heads, q, dev(rpos), 200, kv_b)
        assert np.array_equal(host(a).view(np.uint16), host(c).view(np.uint16))
    q4 = dev(synth.normal_f16(SEED, 30 + fmt, (b, 4, 3 * h1)))
    a = hp.hp_decode_attention(b, 4, h1, heads, q4, 96, paged)
    c = hp.hp_decode_attention(b, 4, h1, heads, q4, 96, flat)
    assert np.array_equal(host(a).view(np.uint16), host(c).view(np.uint16))


@pytest.mark.parametrize("cap", [4096, 4224])
def test_paged_cache_many_pages(hp, cap):
    """Decode attention over long paged caches: 64 pages per request (the most the
    kernel holds in lanes) and 66 (table lookups instead), against the contiguous
    cache bit for bit."""
    fmt, heads, h1, b, pr = 1, 2, 256, 2, 64
    D = h1 // heads
    ppr = cap // pr
    pool = b * ppr + 3
    perm = synth.words(SEED, 40 + cap, 0, pool).argsort()[: b * ppr]
    pages = perm.reshape(b, ppr).astype(np.int32)
    paged = hp.KVCache(fmt, b, heads, cap, D, page_rows=pr, pool_pages=pool, pages=dev(pages))
    flat = hp.KVCache(fmt, b, heads, cap, D)
    T = cap - 70
    pre = synth.normal_f16(SEED, 50 + cap, (b, T, 3 * h1))
    for kv in (paged, flat):
        hp.hp_kv_append(b, T, h1, heads, dev(pre), 0, kv)
    q = dev(synth.normal_f16(SEED, 60 + cap, (b, 1, 3 * h1)))
    rpos = np.array([T - 1, T - 1000], np.int32)
    a = hp.hp_decode_attention_ragged(b, 1, h1, heads, q, dev(rpos), T - 1, paged)
    c = hp.hp_decode_attention_ragged(b, 1, h1, heads, q, dev(rpos), T - 1, flat)
    assert np.array_equal(host(a).view(np.uint16), host(c).view(np.uint16))
    assert np.isfinite(host(a).astype(np.float32)).all()


def test_paged_cache_refused_where_unsupported(hp):
    from decode_step_transformer_amd.hp import HPError
    b, heads, h1, cap, pr = 2, 2, 256, 128, 64
    pages = dev(np.arange(b * 2, dtype=np.int32).reshape(b, 2))
    kv = hp.KVCache(1, b, heads, cap, h1 // heads, page_rows=pr, pool_pages=4, pages=pages)
    q = dev(synth.normal_f16(SEED, 40, (b, 16, 3 * h1)))
    with pytest.raises(HPError):  # int4 with q >= 16 runs on the multi-query kernel
        hp.hp_decode_attention(b, 16, h1, heads, q, 32, kv)
    # page sizes are powers of two (a multiple of 64 that is not one is refused)
    odd = hp.KVCache(1, b, heads, 384, h1 // heads, page_rows=192, pool_pages=4,
                     pages=dev(np.arange(b * 2, dtype=np.int32).reshape(b, 2)))
    with pytest.raises(HPError):
        hp.hp_kv_append(b, 1, h1, heads, q[:, :1].contiguous(), 0, odd)


@pytest.mark.parametrize("fmt", [1, 0])
@pytest.mark.parametrize("cap,T", [(256, 200), (4224, 4000)])
def test_paged_topk_matches_contiguous(hp, fmt, cap, T):
    """Top-K sparse attention through a shuffled page table (4 pages per request:
    page numbers held in lanes; 66: table lookups) against the contiguous cache:
    the same kept rows and the same outputs, bit for bit."""
    heads, h1, b, pr = 2, 256, 3, 64
    D = h1 // heads
    ppr = cap // pr
    pool = b * ppr + 3
    perm = synth.words(SEED, 70 + cap + fmt, 0, pool).argsort()[: b * ppr]
    pages = perm.reshape(b, ppr).astype(np.int32)
    paged = hp.KVCache(fmt, b, heads, cap, D, page_rows=pr, pool_pages=pool, pages=dev(pages))
    flat = hp.KVCache(fmt, b, heads, cap, D)
    pre = synth.normal_f16(SEED, 80 + cap + fmt, (b, T, 3 * h1))
    for kv in (paged, flat):
        hp.hp_kv_append(b, T, h1, heads, dev(pre), 0, kv)
    q = dev(synth.normal_f16(SEED, 90 + cap + fmt, (b, 3 * h1)))
    for topk in (0, 7):
        oa, ia = hp.hp_topk_attention(b, h1, heads, q, T - 1, paged, topk=topk, idx=True)
        oc, ic = hp.hp_topk_attention(b, h1, heads, q, T - 1, flat, topk=topk, idx=True)
        assert np.array_equal(host(ia), host(ic))
        assert np.array_equal(host(oa).view(np.uint16), host(oc).view(np.uint16))
        assert np.isfinite(host(oa).astype(np.float32)).all()


def _block(hp, d, l, seed, fmt=1):
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    h1, h2 = d.h1, d.h2
    shp = {"wq": (h1, h1), "wk": (h1, h1), "wv": (h1, h1), "wo": (h1, h1), "w1": (h1, h2),
           "w2": (h2, h1)}
    layers = [hp.make_layer({k: (torch.randn(v, generator=g, device="cuda") * 0.02).half()
                             for k, v in shp.items()}, fmt) for _ in range(l)]
    x = torch.randn((d.b, d.s, h1), generator=g, device="cuda").half()
    t = torch.randn((d.n, d.b, h1), generator=g, device="cuda").half()
    return layers, x, t


def _run(hp, d, layers, x, t, kvs, flags):
    import torch
    ws = torch.empty(hp.hp_workspace_bytes(d), dtype=torch.uint8, device="cuda")
    xo = torch.empty_like(x)
    to = torch.empty_like(t)
    hp.hp_run_block(d, layers, x, t, kvs, xo, to, ws, flags)
    torch.cuda.synchronize()
    return xo, to


@pytest.mark.parametrize("b,s,n,gbs", [(512, 32, 480, 1), (60, 40, 9, 4)])
def test_diagonal_paged_pool(hp, b, s, n, gbs):
    """The diagonal schedule with page pools of exactly hp_diagonal_pages pages gives
    the contiguous-slot diagonal schedule's outputs bit for bit.  At the n >> s shape
    (512 requests, prompt 32, 480 steps) the pool holds 0.5-0.6 of the rows the same
    live requests would hold at full length s + n: about twice the requests in the
    same memory (the page's peak-memory formula for the diagonal schedule)."""
    import torch
    h1, h2, heads, l, pr = 128, 256, 2, 1, 64
    D = h1 // heads
    d = hp.dims(b, s, n, h1, h2, l, heads, gbs)
    layers, x, t = _block(hp, d, l, 7)
    nb = b // gbs
    nslot = min(nb, n + 1)
    slots = [hp.KVCache(1, nslot * gbs, heads, s + n, D) for _ in range(l)]
    sx, st = _run(hp, d, layers, x, t, slots, hp.HP_DIAGONAL)
    pages = hp.hp_diagonal_pages(d, pr)
    cap = -(-(s + n) // pr) * pr
    pools = [hp.KVCache(1, b, heads, cap, D, page_rows=pr, pool_pages=pages) for _ in range(l)]
    px, pt = _run(hp, d, layers, x, t, pools, hp.HP_DIAGONAL)
    assert torch.equal(px.view(torch.int16), sx.view(torch.int16))
    assert torch.equal(pt.view(torch.int16), st.view(torch.int16))
    assert bool(torch.isfinite(pt.float()).all())
    live = min(nb, n + 1) * gbs
    ratio = pages * pr / (live * (s + n))
    print(f"b={b} s={s} n={n}: pool {pages} pages of {pr} rows = {ratio:.3f} of the live "
          f"requests at full length")
    if n > 10 * s:
        assert 0.5 < ratio < 0.6
    # one page fewer is refused on the host
    small = [hp.KVCache(1, b, heads, cap, D, page_rows=pr, pool_pages=pages - 1) for _ in range(l)]
    from decode_step_transformer_amd.hp import HPError
    with pytest.raises(HPError) as e:
        _run(hp, d, layers, x, t, small, hp.HP_DIAGONAL)
    assert e.value.status == -3


@pytest.mark.parametrize("b,s,n,gbs", [(60, 40, 9, 4), (48, 100, 40, 2)])
def test_diagonal_paged_pool_topk(hp, b, s, n, gbs):
    """HP_DIAGONAL | HP_TOPK10 with page pools (Top-K attention over each live
    request's own rows, through the pool's page table) gives the contiguous-slot
    schedule's outputs bit for bit."""
    import torch
    h1, h2, heads, l, pr = 128, 256, 2, 2, 64
    D = h1 // heads
    d = hp.dims(b, s, n, h1, h2, l, heads, gbs)
    layers, x, t = _block(hp, d, l, 11)
    nb = b // gbs
    nslot = min(nb, n + 1)
    slots = [hp.KVCache(1, nslot * gbs, heads, s + n, D) for _ in range(l)]
    sx, st = _run(hp, d, layers, x, t, slots, hp.HP_DIAGONAL | hp.HP_TOPK10)
    pages = hp.hp_diagonal_pages(d, pr)
    cap = -(-(s + n) // pr) * pr
    pools = [hp.KVCache(1, b, heads, cap, D, page_rows=pr, pool_pages=pages) for _ in range(l)]
    px, pt = _run(hp, d, layers, x, t, pools, hp.HP_DIAGONAL | hp.HP_TOPK10)
    assert torch.equal(px.view(torch.int16), sx.view(torch.int16))
    assert torch.equal(pt.view(torch.int16), st.view(torch.int16))
    assert bool(torch.isfinite(pt.float()).all())
    # and the dense-attention schedule differs (Top-K drops rows)
    _, dt = _run(hp, d, layers, x, t, pools, hp.HP_DIAGONAL)
    assert not torch.equal(dt.view(torch.int16), pt.view(torch.int16))
