"""GPU Top-K sparse decode attention against the oracle ([FlexGen] section 5,
sparse attention), through the C ABI.

The kept rows are an integer decision taken from floating-point scores: the
kernel ranks its fp32 scores (exact code * scale + min, fp32 sums), the
oracle ranks exact double scores of the fp16 K values.  Per row the two
differ by at most a stated bound, so the test requires the GPU's set to be a
valid Top-K under those bounds (no dropped row can beat a kept one by more
than the bounds allow), to hold every row that every valid Top-K holds and
none that none holds, and the undecided band to be narrow; the output must
match the oracle's attention over the GPU's set (within the parity
tolerance), and the oracle's own output where the sets agree.  Zero queries
(all scores equal) pin the tie rule bit-exactly.
"""
import numpy as np
import pytest

import synth
from helpers import TOL, assert_close, dev, host

pytestmark = pytest.mark.gpu
SEED = synth.seed_for(81)


@pytest.fixture(scope="module")
def hp():
    import torch
    from decode_step_transformer_amd import hp as _hp
    assert torch.cuda.is_available()
    assert _hp.hp_device_check() == 0, _hp.hp_last_error()
    return _hp


def _setup(hp, orc, fmt, b, heads, D, T, stream, zero_q=False):
    """Cache rows [0, T) appended from seeded rows; the query is row T-1's."""
    h1 = heads * D
    rows = synth.normal_f16(SEED, stream, (b, T, 3 * h1))
    kv = hp.KVCache(fmt, b, heads, T + 2, D)
    hp.hp_kv_append(b, T, h1, heads, dev(rows), 0, kv)
    qkv = rows[:, T - 1].copy()
    if zero_q:
        qkv[:, :h1] = 0
    ok = orc.KV(fmt, b, heads, T + 2, D)
    for name, oname in (("k", "k"), ("v", "v")) + ((("k_sm", "ksm"), ("v_sm", "vsm")) if fmt else ()):
        setattr(ok, oname, host(getattr(kv, name)).copy())
    return kv, qkv, ok.values("k", T), ok.values("v", T), ok


def _score_bound(fmt, q, Krows, sm):
    """Per-row bound on |GPU score - exact score of the fp16 K values|.
    fp16 cache: fp16 products are exact, the kernel sums at most 2d terms in
    fp32.  int4 cache: the kernel scores the exact code * scale + min (fp32
    sums of at most 4d terms (64 + c) q, times the group scale, plus min * sum q)
    while the oracle scores that value rounded to fp16 (half an ulp: 2^-11 of
    it, or 2^-25 below the normal range)."""
    qa = np.abs(q.astype(np.float64))
    ka = np.abs(Krows.astype(np.float64))
    u, d = 2.0 ** -24, q.shape[0]
    if fmt == 0:
        return 2 * d * u * (ka @ qa) + 1e-30
    f16 = lambda x: x.astype(np.uint16).view(np.float16).astype(np.float64)
    scale, mn = np.abs(f16(sm[..., 0])), np.abs(f16(sm[..., 1]))  # [T][G]
    return (2.0 ** -11 * 1.001 * (ka @ qa) + 2.0 ** -25 * qa.sum()
            + 4 * d * u * (80 * scale.max(axis=1) + mn.max(axis=1)) * qa.sum())


def _certain(z, eps, K):
    """Rows every valid Top-K keeps (fewer than K rows can outscore them within
    the bounds) and rows none keeps (at least K rows surely outscore them)."""
    hi, lo = np.sort(z + eps), np.sort(z - eps)
    T = z.shape[0]
    could_beat = T - np.searchsorted(hi, z - eps, side="left")  # rows j with z_j + eps_j >= z_i - eps_i
    could_beat -= 1                                             # (row i itself)
    surely_beat = T - np.searchsorted(lo, z + eps, side="right")  # rows j with z_j - eps_j > z_i + eps_i
    return could_beat < K, surely_beat >= K


def _check_pair(out, sel, q, Kr, Vr, sm, fmt, K, T, orc, what):
    """Returns (GPU set == oracle set, rows in the ambiguous band)."""
    assert np.all(np.diff(sel) > 0) and sel[0] >= 0 and sel[-1] < T, sel
    z = Kr.astype(np.float64) @ q.astype(np.float64)
    eps = _score_bound(fmt, q, Kr, sm)
    drop = np.setdiff1d(np.arange(T), sel)
    if drop.size:  # every kept row scores at least every dropped row, within the bounds
        assert (z[sel] + eps[sel]).min() >= (z[drop] - eps[drop]).max(), what
    keep_sure, drop_sure = _certain(z, eps, K)
    kept = np.zeros(T, bool)
    kept[sel] = True
    assert kept[keep_sure].all() and not kept[drop_sure].any(), what
    ref_out, ref_sel = orc.topk_attention(q, Kr, Vr, K)
    want = orc.attention(q[None], Kr[sel], Vr[sel], [K])[0]
    assert_close(out, want, what=what)
    same = np.array_equal(sel, ref_sel)
    if same:
        assert_close(out, ref_out, what="oracle " + what)
    return same, int(T - keep_sure.sum() - drop_sure.sum())


def _check(hp, orc, fmt, b, heads, D, T, topk, stream, zero_q=False):
    h1 = heads * D
    kv, qkv, Kc, Vc, ok = _setup(hp, orc, fmt, b, heads, D, T, stream, zero_q)
    out, idx = hp.hp_topk_attention(b, h1, heads, dev(qkv), T - 1, kv, topk=topk, idx=True)
    out, idx = host(out), host(idx)
    K = min(topk, T) if topk > 0 else orc.topk_count(T)
    assert idx.shape == (b, heads, K)
    amb = 0
    for r in range(b):
        for h in range(heads):
            _, a = _check_pair(out[r, h * D:(h + 1) * D], idx[r, h].astype(np.int64),
                               qkv[r, h * D:(h + 1) * D], Kc[r, h], Vc[r, h],
                               ok.ksm[r, h, :T] if fmt else None, fmt, K, T, orc, f"r{r} h{h}")
            amb = max(amb, a)
    return amb, idx


@pytest.mark.parametrize("fmt", [1, 0])
@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("T", [1, 63, 64, 65, 200, 528])
def test_topk_matches_oracle(hp, orc, fmt, D, T):
    amb, _ = _check(hp, orc, fmt, 3, 2, D, T, 0, 100 + T + D + fmt)
    assert amb <= max(4, T // 32), amb  # the bounds leave only a narrow band undecided


@pytest.mark.parametrize("T,topk", [(1100, 0), (2112, 0), (3000, 17), (4096, 0), (300, 1), (50, 50),
                                    (40, 1000)])
def test_topk_sizes(hp, orc, T, topk):
    _check(hp, orc, 1, 2, 2, 128, T, topk, 200 + T + topk)


@pytest.mark.parametrize("fmt", [1, 0])
def test_topk_ties_go_to_lower_rows(hp, orc, fmt):
    """A zero query scores every row 0: the first K rows are kept, and the
    output is their mean."""
    T = 333
    K = orc.topk_count(T)
    _, idx = _check(hp, orc, fmt, 2, 2, 128, T, 0, 300 + fmt, zero_q=True)
    assert np.array_equal(idx, np.broadcast_to(np.arange(K, dtype=np.int32), idx.shape))


def test_topk_all_rows_is_dense(hp, orc):
    """topk = T keeps every row: the result matches dense decode attention."""
    b, heads, D, T = 2, 4, 128, 257
    h1 = heads * D
    kv, qkv, Kc, Vc, ok = _setup(hp, orc, 1, b, heads, D, T, 400)
    out = host(hp.hp_topk_attention(b, h1, heads, dev(qkv), T - 1, kv, topk=T))
    qkv3 = np.ascontiguousarray(qkv[:, None, :])
    dense = host(hp.hp_decode_attention(b, 1, h1, heads, dev(qkv3), T - 1, kv))[:, 0]
    assert_close(out, dense, what="topk = T vs dense")


def test_topk_full_size_sampled(hp, orc):
    """The benchmark's shape (OPT-30B decode: b = 144, 56 heads, d = 128, T = 528,
    K = 53), every request on the GPU, sampled (request, head) pairs checked."""
    import torch
    b, heads, D, T = 144, 56, 128, 528
    h1 = heads * D
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    rows = (torch.randn((b, T, 3 * h1), generator=g, device="cuda")).half()
    samp = [0, 77, 143]
    for r in samp:  # sampled requests take seeded synth rows (the same bits go to the oracle)
        rows[r] = dev(synth.normal_f16(SEED, 500 + r, (T, 3 * h1)))
    kv = hp.KVCache(1, b, heads, T, D)
    hp.hp_kv_append(b, T, h1, heads, rows, 0, kv)
    qkv = rows[:, T - 1].contiguous()
    out, idx = hp.hp_topk_attention(b, h1, heads, qkv, T - 1, kv, idx=True)
    out, idx, qh = host(out), host(idx), host(qkv)
    K = orc.topk_count(T)
    kc, vc = host(kv.k), host(kv.v)
    ks, vs = host(kv.k_sm), host(kv.v_sm)
    for r in samp:
        for h in (0, 31, 55):
            Kr = orc.dequantize_g64(kc[r, h], ks[r, h])
            Vr = orc.dequantize_g64(vc[r, h], vs[r, h])
            _, amb = _check_pair(out[r, h * D:(h + 1) * D], idx[r, h].astype(np.int64),
                                 qh[r, h * D:(h + 1) * D], Kr, Vr, ks[r, h], 1, K, T, orc,
                                 f"r{r} h{h}")
            assert amb <= T // 32, amb
    assert np.isfinite(out.astype(np.float32)).all()


def test_topk_rejects_bad_sizes(hp):
    import torch
    kv = hp.KVCache(1, 1, 1, 5000, 128)
    qkv = torch.zeros((1, 384), dtype=torch.float16, device="cuda")
    with pytest.raises(hp.HPError):
        hp.hp_topk_attention(1, 128, 1, qkv, 4096, kv)  # 4097 rows
    with pytest.raises(hp.HPError):
        hp.hp_topk_attention(1, 128, 1, qkv, 10, kv, topk=-1)
    small = hp.KVCache(1, 1, 1, 8, 128)
    with pytest.raises(hp.HPError):
        hp.hp_topk_attention(1, 128, 1, qkv, 8, small)  # row 8 is past the capacity


def _tiny_block(hp, flags, kv_fmt):
    """The Tiny configuration's block (int4 weights) on the GPU."""
    import torch
    from configs import CONFIGS, decode_inputs, layer_weights, prompt
    c = CONFIGS[1]
    l, h1, h2, heads, b, s, n = c["l"], c["h1"], c["h2"], c["heads"], c["b"], c["s"], c["n"]
    Ws = [layer_weights(1, j, h1, h2) for j in range(l)]
    layers = [hp.make_layer({k: dev(v) for k, v in W.items()}, 1) for W in Ws]
    x, t = prompt(1, b, s, h1), decode_inputs(1, n, b, h1)
    d = hp.dims(b, s, n, h1, h2, l, heads, b)
    ws = torch.empty(hp.hp_workspace_bytes(d), dtype=torch.uint8, device="cuda")
    kvs = [hp.KVCache(kv_fmt, b, heads, s + n, h1 // heads) for _ in layers]
    xo = torch.empty((b, s, h1), dtype=torch.float16, device="cuda")
    to = torch.empty((n, b, h1), dtype=torch.float16, device="cuda")
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        hp.hp_run_block(d, layers, dev(x), dev(t), kvs, xo, to, ws, flags, stream=stream)
    stream.synchronize()
    return c, Ws, x, t, host(xo), host(to)


def _min_gap_over_block(orc, c, Wo, x, t, kv_fmt):
    """Runs the oracle's sparse block and returns, over every decode step, layer,
    request and head, the smallest (K-th - (K+1)-th score) / (score bound)."""
    l, h1, heads, b, s, n = c["l"], c["h1"], c["heads"], c["b"], c["s"], c["n"]
    d = h1 // heads
    kvs = [orc.KV(kv_fmt, b, heads, s + n, d) for _ in range(l)]
    cur = x
    for j in range(l):
        cur = orc.layer_prefill(cur, Wo[j], kvs[j], heads)
    worst = np.inf
    for i in range(n):
        tc = t[i].reshape(b, 1, h1)
        for j in range(l):
            tb = tc.reshape(b, h1)
            q, kn = orc.gemm(tb, Wo[j]["wq"]), orc.gemm(tb, Wo[j]["wk"])
            T = s + i + 1
            K = orc.topk_count(T)
            prev = kvs[j].values("k", s + i)
            for r in range(b):
                for h in range(heads):
                    keys = np.concatenate([prev[r, h], kn[r, h * d:(h + 1) * d][None]])
                    qq = q[r, h * d:(h + 1) * d]
                    z = np.sort(keys.astype(np.float64) @ qq.astype(np.float64))[::-1]
                    eps = _score_bound(0, qq, keys, None).max()
                    worst = min(worst, (z[K - 1] - z[K]) / (2 * eps))
            tc = orc.layer_decode_topk(tc, Wo[j], kvs[j], heads, s + i)
    return worst


def test_tiny_block_topk10_vs_oracle(hp, orc):
    """Decode columns with 10% Top-K attention (K = ceil(T / 10) of T = 33..40
    rows), graph-replayed and eager: bitwise equal to each other and within
    the tolerance of the oracle's block with the same attention.  The cache is
    fp16 here, where the kernel's and the oracle's scores differ only by fp32
    rounding, and the test checks that every kept set of the run is unique at
    that resolution; the int4 cache's selection is checked kernel by kernel
    above (its scores differ by up to half an fp16 ulp per key, within which
    near-equal scores may legitimately be ranked either way)."""
    from configs import oracle_weights
    c, Ws, x, t, xo, to = _tiny_block(hp, hp.HP_GRAPH | hp.HP_TOPK10, 0)
    _, _, _, _, _, to2 = _tiny_block(hp, hp.HP_TOPK10, 0)
    assert np.array_equal(to.view(np.uint16), to2.view(np.uint16))
    Wo = [oracle_weights(orc, W, 1) for W in Ws]
    assert _min_gap_over_block(orc, c, Wo, x, t, 0) > 1.0  # every Top-K set is unique
    kref = [orc.KV(0, c["b"], c["heads"], c["s"] + c["n"], c["h1"] // c["heads"]) for _ in Ws]
    rx, rt = orc.run_block_topk(x, t, Wo, kref, c["heads"])
    assert_close(xo, rx, what="tiny prefill output")
    assert_close(to, rt, what="tiny decode outputs, Top-K attention")
    _, _, _, _, _, dense = _tiny_block(hp, hp.HP_GRAPH, 0)
    assert not np.array_equal(dense.view(np.uint16), to.view(np.uint16))  # the flag took effect


def test_tiny_block_topk10_int4_runs(hp):
    """The int4-cache block with Top-K attention: graph replay equals eager
    launches bit for bit, and every output is finite."""
    _, _, _, _, _, to = _tiny_block(hp, hp.HP_GRAPH | hp.HP_TOPK10, 1)
    _, _, _, _, _, to2 = _tiny_block(hp, hp.HP_TOPK10, 1)
    assert np.array_equal(to.view(np.uint16), to2.view(np.uint16))
    assert np.isfinite(to.astype(np.float32)).all()
