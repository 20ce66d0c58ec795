"""GPU parity of the individual HIP kernels against the CPU oracle, through
the C ABI.  Inputs come from the seeded generator (synth); expected values
come only from the oracle.

FlexGen paper notes: section 5 (group-wise int4 quantisation of weights
along output channels and of the KV cache along the hidden dimension),
background section (products x·w, attention softmax(q k^T / sqrt(d)) v).
SpecPipe article 2.2.1: tree masks.
"""
import numpy as np
import pytest

import synth
from helpers import TOL, assert_close, dev, host, unpack_f16_weight, unpack_nibbles, unpack_q4_weight

pytestmark = pytest.mark.gpu
SEED = synth.seed_for(99)


@pytest.fixture(scope="module")
def hp():
    import torch
    from decode_step_transformer_amd import hp as _hp
    assert torch.cuda.is_available()
    assert _hp.hp_device_check() == 0, _hp.hp_last_error()
    return _hp


def _edge_groups():
    g = np.zeros((8, 64), np.float16)
    g[0] = 2.5
    g[1] = np.where(np.arange(64) % 2, -0.0, 0.0)
    g[2] = np.where(np.arange(64) % 3, 1.0, -2.0)
    g[3] = np.linspace(-1, 1, 64)
    g[3, 5] = np.nan
    g[4] = np.nan
    g[5] = np.linspace(-3, 3, 64)
    g[5, 7] = np.inf
    g[6] = (np.arange(64) % 16) * 0.125 - 1
    g[7] = 65504.0
    g[7, ::2] = -65504.0
    return g


@pytest.mark.parametrize("rows,cols,sigma", [(1, 64, 1.0), (1000, 256, 1.0), (777, 4096, 0.02),
                                             (3, 12288, 1.0)])
def test_quantize_bit_exact(hp, orc, rows, cols, sigma):
    x = synth.normal_f16(SEED, 10 + cols, (rows, cols), sigma)
    codes, sm = hp.hp_quantize_g64(dev(x))
    rc, rs = orc.quantize_g64(x)
    assert np.array_equal(host(codes), rc)
    assert np.array_equal(host(sm), rs)


def test_quantize_edge_groups(hp, orc):
    x = _edge_groups()
    codes, sm = hp.hp_quantize_g64(dev(x))
    rc, rs = orc.quantize_g64(x)
    assert np.array_equal(host(codes), rc)
    assert np.array_equal(host(sm), rs)


def test_quantize_empty(hp):
    import torch
    x = torch.empty((0, 128), dtype=torch.float16, device="cuda")
    codes, sm = hp.hp_quantize_g64(x)
    assert codes.numel() == 0


def test_dequantize_bit_exact(hp, orc):
    x = synth.normal_f16(SEED, 20, (333, 512), 0.5)
    rc, rs = orc.quantize_g64(x)
    y = hp.hp_dequantize_g64(dev(rc), dev(rs.view(np.int16)))
    assert np.array_equal(host(y).view(np.uint16), orc.dequantize_g64(rc, rs).view(np.uint16))


@pytest.mark.parametrize("k,n", [(128, 64), (256, 768), (384, 1024)])
def test_pack_q4_layout(hp, orc, k, n):
    w = synth.normal_f16(SEED, 30 + k + n, (k, n), 0.02)
    codes, sm = hp.hp_quantize_g64(dev(w))
    m = hp.hp_pack_weight_q4(codes, sm, k, n)
    rc, rs = orc.quantize_g64(w)
    assert np.array_equal(unpack_q4_weight(host(m.data), k, n), unpack_nibbles(rc))
    assert np.array_equal(host(m.scale).view(np.uint16), rs[:, :, 0].T)
    assert np.array_equal(host(m.minv).view(np.uint16), rs[:, :, 1].T)


@pytest.mark.parametrize("k,n", [(128, 64), (256, 768), (384, 1024)])
def test_pack_f16_layout(hp, k, n):
    """hp_pack_weight_f16 writes the fragment-major layout the header documents,
    moving every value unchanged; shapes off the 128 x 64 grid are refused."""
    w = synth.normal_f16(SEED, 40 + k + n, (k, n), 0.02)
    m = hp.hp_pack_weight_f16(dev(w))
    assert np.array_equal(unpack_f16_weight(host(m.data).view(np.uint16), k, n), w.view(np.uint16))
    with pytest.raises(hp.HPError):
        hp.hp_pack_weight_f16(dev(w[:, : n - 32]))


def _ref_gemm(orc, x, w, fmt, res=None, relu=False):
    if fmt == 1:
        rc, rs = orc.quantize_g64(w)
        w = orc.dequantize_g64(rc, rs)
    return orc.gemm(x, w, res, relu)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("M,K,N,epi", [
    (1, 128, 64, ""), (4, 256, 768, "res"), (37, 384, 320, "relu"), (64, 512, 1024, "res"),
    (144, 1024, 512, "relu"), (145, 256, 256, "res"), (300, 640, 576, ""), (1000, 256, 1280, "relu"),
])
def test_gemm(hp, orc, fmt, M, K, N, epi):
    x = synth.normal_f16(SEED, 40 + M, (M, K))
    w = synth.normal_f16(SEED, 41 + N, (K, N), 0.05)
    res = synth.normal_f16(SEED, 42 + M, (M, N)) if epi == "res" else None
    m = hp.make_weight(dev(w), fmt)
    y = hp.hp_gemm(dev(x), m, res=dev(res) if res is not None else None, relu=epi == "relu")
    ref = _ref_gemm(orc, x, w, fmt, res, epi == "relu")
    assert_close(host(y), ref, what=f"gemm fmt={fmt} M={M}")


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("KB", range(5, 17))
def test_gemm_split_counts(hp, orc, fmt, KB):
    """Skinny products with one column tile and k = 128 KB: both split rules
    give KB split-K partial sums (every count the sum kernels are built for
    beyond those of test_gemm), with the residual epilogue."""
    M, K, N = 64 if KB % 2 else 144, 128 * KB, 256
    x = synth.normal_f16(SEED, 60 + KB, (M, K))
    w = synth.normal_f16(SEED, 61 + KB, (K, N), 0.05)
    res = synth.normal_f16(SEED, 62 + KB, (M, N))
    m = hp.make_weight(dev(w), fmt)
    y = hp.hp_gemm(dev(x), m, res=dev(res))
    ref = _ref_gemm(orc, x, w, fmt, res, False)
    assert_close(host(y), ref, what=f"gemm fmt={fmt} K={K}")


@pytest.mark.parametrize("fmt", [0, 1])
def test_gemm_rows_do_not_depend_on_m(hp, fmt):
    """Skinny products reduce k in an order fixed by (k, n): any row subset of
    a batch of up to 144 rows gives bitwise the same rows."""
    x = synth.normal_f16(SEED, 50, (144, 1024))
    w = synth.normal_f16(SEED, 51, (1024, 768), 0.05)
    m = hp.make_weight(dev(w), fmt)
    y = host(hp.hp_gemm(dev(x), m))
    for lo, hi in ((0, 48), (48, 96), (100, 101)):
        ys = host(hp.hp_gemm(dev(x[lo:hi]), m))
        assert np.array_equal(ys.view(np.uint16), y[lo:hi].view(np.uint16))


def _qkv(seed, b, q, h1):
    return synth.normal_f16(SEED, seed, (b, q, 3 * h1))


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("b,q,h1,heads,pos,cap", [
    (2, 5, 256, 4, 0, 8), (3, 1, 256, 2, 7, 9), (1, 64, 512, 4, 100, 170),
    # d = 128, rows from a multiple of 16 (the tiled int4 append: 16 tokens x 4 heads
    # per workgroup): whole chunks and head blocks; a ragged last chunk with a partial
    # head block; fewer heads than a block
    (2, 48, 1024, 8, 0, 64), (3, 37, 768, 6, 16, 64), (1, 16, 256, 2, 32, 48)])
def test_kv_append_bit_exact(hp, orc, fmt, b, q, h1, heads, pos, cap):
    qkv = _qkv(60 + q, b, q, h1)
    D = h1 // heads
    kv = hp.KVCache(fmt, b, heads, cap, D)
    hp.hp_kv_append(b, q, h1, heads, dev(qkv), pos, kv)
    for which, col in (("k", 1), ("v", 2)):
        rows = qkv[:, :, col * h1:(col + 1) * h1].reshape(b, q, heads, D).transpose(0, 2, 1, 3)
        got = host(getattr(kv, which))
        if fmt == 0:
            assert np.array_equal(got[:, :, pos:pos + q].view(np.uint16), rows.view(np.uint16))
        else:
            rc, rs = orc.quantize_g64(np.ascontiguousarray(rows))
            assert np.array_equal(got[:, :, pos:pos + q], rc)
            assert np.array_equal(host(getattr(kv, which + "_sm"))[:, :, pos:pos + q], rs)
        assert not got[:, :, :pos].any() and not got[:, :, pos + q:].any()


def _fill_cache(hp, orc, fmt, b, heads, cap, D, rows, seed):
    """Seeded K/V rows [0, rows) written through the KV append kernel."""
    h1 = heads * D
    kvq = synth.normal_f16(SEED, seed, (b, rows, 3 * h1))
    kv = hp.KVCache(fmt, b, heads, cap, D)
    if rows:
        hp.hp_kv_append(b, rows, h1, heads, dev(kvq), 0, kv)
    return kv


def _cache_values(orc, kv, T):
    k, v = host(kv.k)[:, :, :T], host(kv.v)[:, :, :T]
    if kv.fmt == 0:
        return k.view(np.float16), v.view(np.float16)
    return (orc.dequantize_g64(k, host(kv.k_sm)[:, :, :T]),
            orc.dequantize_g64(v, host(kv.v_sm)[:, :, :T]))


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("P,q,tree", [(0, 1, False), (1, 1, False), (63, 1, False), (200, 1, False),
                                      (70, 7, False), (130, 64, True), (0, 5, True),
                                      # q >= 16: the multi-query MFMA path for int4 caches
                                      (0, 16, True), (37, 16, False), (300, 33, True),
                                      (129, 64, False), (1000, 20, True), (64, 48, True)])
def test_decode_attention(hp, orc, fmt, D, P, q, tree):
    import torch
    b, heads = 3, 2
    h1 = heads * D
    cap = P + q + 3
    kv = _fill_cache(hp, orc, fmt, b, heads, cap, D, P, 70 + P)
    qkv = synth.normal_f16(SEED, 71 + q, (b, q, 3 * h1))
    hp.hp_kv_append(b, q, h1, heads, dev(qkv), P, kv)
    masks = None
    if tree:
        parents = np.stack([synth.bfs_parents(SEED, 72 + r, q) for r in range(b)])
        masks = np.stack([orc.tree_masks(p) for p in parents])
    out = hp.hp_decode_attention(b, q, h1, heads, dev(qkv), P, kv,
                                 masks=dev(masks.view(np.int64)) if tree else None)
    K, V = _cache_values(orc, kv, P + q)
    ref = np.zeros((b, q, h1), np.float16)
    for r in range(b):
        for h in range(heads):
            Q = qkv[r, :, h * D:(h + 1) * D]
            if tree:
                o = orc.attention(Q, K[r, h], V[r, h], [P] * q, masks[r], P)
            else:
                o = orc.attention(Q, K[r, h], V[r, h], P + 1 + np.arange(q))
            ref[r, :, h * D:(h + 1) * D] = o
    assert_close(host(out), ref, what="decode attention")


@pytest.mark.parametrize("b", [2, 5])
@pytest.mark.parametrize("D,s", [(64, 1), (64, 37), (128, 64), (128, 150)])
def test_prefill_attention(hp, orc, D, s, b):
    """b = 5 gives 15 or 20 (request, head) pairs: whole groups of 8 pairs share
    an XCD's L2 turn by turn, the remainder runs in plain order."""
    heads = 3
    h1 = heads * D
    if h1 % 128:
        heads, h1 = 4, 4 * D
    qkv = synth.normal_f16(SEED, 80 + s + b, (b, s, 3 * h1))
    out = hp.hp_prefill_attention(b, s, h1, heads, dev(qkv))
    ref = np.zeros((b, s, h1), np.float16)
    for r in range(b):
        for h in range(heads):
            sl = slice(h * D, (h + 1) * D)
            Q = qkv[r, :, sl]
            K = qkv[r, :, h1 + h * D:h1 + (h + 1) * D]
            V = qkv[r, :, 2 * h1 + h * D:2 * h1 + (h + 1) * D]
            ref[r, :, sl] = orc.attention(Q, K, V, np.arange(1, s + 1))
    assert_close(host(out), ref, what="prefill attention")


def _ramp_keys(qkv, h1, up):
    """qkv [b, s, 3 h1] with key row j scaled by 1 + j / 8 (or the reverse order), in binary16."""
    f = 1.0 + np.arange(qkv.shape[1]) / 8.0
    if not up:
        f = f[::-1]
    out = qkv.copy()
    out[:, :, h1:2 * h1] = (out[:, :, h1:2 * h1].astype(np.float32) * f[None, :, None]).astype(np.float16)
    return out


@pytest.mark.parametrize("up", [True, False])
@pytest.mark.parametrize("D", [64, 128])
def test_prefill_attention_moving_maximum(hp, orc, D, up):
    """Scores that rise block after block by far more than 2^8 in the exponent (the
    block step's running maximum moves, rescaling l and O, at every block), or fall
    (it never moves after the first block)."""
    b, s, heads = 2, 300, 2
    h1 = heads * D
    qkv = _ramp_keys(synth.normal_f16(SEED, 95, (b, s, 3 * h1)), h1, up)
    out = hp.hp_prefill_attention(b, s, h1, heads, dev(qkv))
    ref = np.zeros((b, s, h1), np.float16)
    for r in range(b):
        for h in range(heads):
            sl = slice(h * D, (h + 1) * D)
            K = qkv[r, :, h1 + h * D:h1 + (h + 1) * D]
            V = qkv[r, :, 2 * h1 + h * D:2 * h1 + (h + 1) * D]
            ref[r, :, sl] = orc.attention(qkv[r, :, sl], K, V, np.arange(1, s + 1))
    assert_close(host(out), ref, what="prefill attention, moving maximum")


@pytest.mark.parametrize("up", [True, False])
def test_tree_attention_moving_maximum(hp, orc, up):
    """The multi-query MFMA path (int4 cache, tree masks) over a prefix whose scores
    rise or fall across its 64-row blocks as in the prefill case."""
    b, heads, D, P, q = 2, 2, 128, 300, 64
    h1 = heads * D
    pre = _ramp_keys(synth.normal_f16(SEED, 96, (b, P, 3 * h1)), h1, up)
    kv = hp.KVCache(1, b, heads, P + q, D)
    hp.hp_kv_append(b, P, h1, heads, dev(pre), 0, kv)
    qkv = synth.normal_f16(SEED, 97, (b, q, 3 * h1))
    hp.hp_kv_append(b, q, h1, heads, dev(qkv), P, kv)
    parents = np.stack([synth.bfs_parents(SEED, 98 + r, q) for r in range(b)])
    masks = np.stack([orc.tree_masks(p) for p in parents])
    out = hp.hp_decode_attention(b, q, h1, heads, dev(qkv), P, kv, masks=dev(masks.view(np.int64)))
    K, V = _cache_values(orc, kv, P + q)
    ref = np.zeros((b, q, h1), np.float16)
    for r in range(b):
        for h in range(heads):
            ref[r, :, h * D:(h + 1) * D] = orc.attention(qkv[r, :, h * D:(h + 1) * D], K[r, h],
                                                         V[r, h], [P] * q, masks[r], P)
    assert_close(host(out), ref, what="tree attention, moving maximum")


def test_tree_masks(hp, orc):
    import torch
    b, q = 8, 64
    parents = np.stack([synth.bfs_parents(SEED, 90 + r, q) for r in range(b)])
    parents[7] = np.arange(-1, q - 1)                                       # chain
    masks, err = hp.hp_tree_masks(dev(parents.astype(np.int32)))
    ref = np.stack([orc.tree_masks(p) for p in parents])
    assert np.array_equal(host(masks).view(np.uint64), ref)
    assert int(host(err)[0]) == 0
    bad = parents.copy()
    bad[0, 5] = 9      # parent after child
    bad[1, 0] = 0      # root with a parent
    masks, err = hp.hp_tree_masks(dev(bad.astype(np.int32)))
    assert int(host(err)[0]) == 2
    assert int(host(masks).view(np.uint64)[0, 5]) == 1 << 5


def test_peak_probes_run(hp):
    """The measurement probes run and report rates in the range of the hardware
    (loose floors: a stream of 1 GiB above 2 TB/s, MFMA chains above 0.8 PFLOP/s)."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    x = torch.ones(1 << 29, dtype=torch.float16, device="cuda")
    sink = torch.zeros(64 * cus, dtype=torch.int32, device="cuda")

    def ms(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(3):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / 3

    t_read = ms(lambda: hp.hp_peak_read(x, 8 * cus, sink))
    assert (1 << 30) / (t_read / 1e3) > 2e12
    t_mfma = ms(lambda: hp.hp_peak_mfma(2000, cus, sink))
    assert cus * 8 * 16 * 2000 * 16384 / (t_mfma / 1e3) > 0.8e15
    assert not sink.any()  # the probes' folded values never match their store condition
