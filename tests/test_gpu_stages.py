"""Stage-wise, teacher-forced parity of one layer at the full OPT shapes.

The layer stores binary16 at every stage boundary (FlexGen paper notes,
background section: Q/K/V, the attention output, x_Out, the MLP hidden, the
output; section 5: the K/V rows are quantised from the stored fp16 values).
hp_layer_prefill / hp_layer_decode run on the whole batch in the launch
configuration the block benchmark times, with hp_debug_set_capture copying
out those fp16 tensors.  The oracle then recomputes every stage of sampled
requests from the GPU's previous-stage fp16 output, so errors never
compound and each stage is held to |gpu - ref| <= 2e-2 max(1, |ref|) per
element at its real shape:

  QKV   = x [wQ | wK | wV]                      (sampled rows)
  codes = quantise(the GPU's own K, V rows)     (bit-exact, every head)
  attn  = softmax(Q K^T / sqrt(d)) V            (every query row, every head)
  x_out = attn wO + x                           (sampled rows)
  hid   = relu(x_out w1)                        (sampled rows)
  out   = hid w2 + x_out                        (sampled rows)

Prefill checks all s = 512 query rows of every head of two requests (every
query block, the diagonal and the off-diagonal ones); the products are
checked on rows spread over all query blocks.  Decode checks two requests
per GPU batch of the block.  The layers sampled across the cases are 0, 1,
l/2 and l - 1 of their stacks.  The sampled requests take seeded synth
inputs (the same bits on both sides); the other requests get device draws
that only fill the launch to its full shape.  Each case also prints the
free-running code flip rate: the codes the oracle quantises from its own
K/V (computed from x, not from the GPU's) against the GPU's codes.
"""
import concurrent.futures as cf
import math

import numpy as np
import pytest

import synth
from configs import CONFIGS, layer_weights, oracle_weights
from helpers import assert_close, dev, host, unpack_nibbles

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

# (config, kind, layer index)
CASES = [(2, "prefill", 0), (2, "decode", 31), (3, "prefill", 1), (3, "decode", 24),
         (4, "prefill", 95), (4, "decode", 0)]
PREFILL_REQ = {2: (0, 63), 3: (0, 143), 4: (5, 140)}
DECODE_REQ = {2: (0, 63), 3: (0, 47, 48, 95, 96, 143), 4: (0, 47, 48, 95, 96, 143)}
# prefill rows checked in the products: both ends of every 64-row query block region
ROWS = np.array([0, 1, 63, 64, 130, 255, 256, 390, 448, 511])


@pytest.fixture(scope="module")
def hp():
    import torch
    from decode_step_transformer_amd import hp as _hp
    assert torch.cuda.is_available()
    assert _hp.hp_device_check() == 0, _hp.hp_last_error()
    return _hp


_cache = {}


def _layer(hp, orc, cid, j):
    """Layer j of configuration cid: the oracle's weight values and the GPU layer."""
    if (cid, j) not in _cache:
        _cache.clear()
        c = CONFIGS[cid]
        W = layer_weights(cid, j, c["h1"], c["h2"])
        layer = hp.make_layer({k: dev(v) for k, v in W.items()}, c["w_fmt"])
        Wo = oracle_weights(orc, W, c["w_fmt"])
        del W
        Wo["wqkv"] = np.concatenate([Wo["wq"], Wo["wk"], Wo["wv"]], axis=1)
        _cache[(cid, j)] = (Wo, layer)
    return _cache[(cid, j)]


def _sampled(kind, cid, rows, shape, sigma=1.0):
    seed = synth.seed_for(cid)
    return np.stack([synth.normal_f16(seed, synth.stream_request(kind, r), shape, sigma)
                     for r in rows])


def _filled(shape, sigma, rows, values, seed):
    """Device tensor of N(0, sigma^2) fp16 draws with requests `rows` replaced by `values`."""
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    t = torch.randn(shape, generator=g, device="cuda", dtype=torch.float16).mul_(sigma)
    for i, r in enumerate(rows):
        t[r].copy_(dev(values[i]))
    return t


def _captures(hp, M, h1, h2):
    import torch
    bufs = dict(qkv=torch.empty((M, 3 * h1), dtype=torch.float16, device="cuda"),
                attn=torch.empty((M, h1), dtype=torch.float16, device="cuda"),
                x_out=torch.empty((M, h1), dtype=torch.float16, device="cuda"),
                hidden=torch.empty((M, h2), dtype=torch.float16, device="cuda"))
    return bufs


def _head_rows(x, heads):
    """[T][h1] -> [heads][T][d] (the cache's head-major order)."""
    T, h1 = x.shape
    return np.ascontiguousarray(x.reshape(T, heads, h1 // heads).transpose(1, 0, 2))


def _check_codes(orc, fmt, g_codes, g_sm, rows_f16, what):
    """The GPU's cache rows against the oracle's coding of the GPU's own fp16 K or V
    rows (head-major [heads][T][d]): bit-exact codes and {scale, min} (fp16 caches:
    the same bits)."""
    if fmt == 0:
        assert np.array_equal(g_codes.view(np.uint16), rows_f16.view(np.uint16)), what
        return
    rc, rs = orc.quantize_g64(rows_f16)
    assert np.array_equal(g_codes, rc), f"{what}: codes differ"
    assert np.array_equal(g_sm.view(np.uint16), rs), f"{what}: scale/min differ"


def _flips(orc, g_codes, ref_rows_f16):
    """Fraction of 4-bit codes that differ between the GPU's cache rows and the
    oracle's coding of its own (free-running) K or V rows."""
    rc, _ = orc.quantize_g64(ref_rows_f16)
    a, b = unpack_nibbles(g_codes), unpack_nibbles(rc)
    return float((a != b).mean()), int(np.abs(a.astype(int) - b.astype(int)).max())


def _stage(name, gpu, ref, stats):
    stats[name] = assert_close(gpu, ref, what=name)


def _attn_heads(orc, pool, q, k, v, lim, heads):
    """Oracle attention of every head: q [nq][h1], k, v [T][h1] (fp16 values)."""
    D = q.shape[1] // heads
    out = np.zeros(q.shape, np.float16)

    def one(h):
        sl = slice(h * D, (h + 1) * D)
        out[:, sl] = orc.attention(np.ascontiguousarray(q[:, sl]), np.ascontiguousarray(k[:, sl]),
                                   np.ascontiguousarray(v[:, sl]), lim)

    list(pool.map(one, range(heads)))
    return out


def _prefill(hp, orc, cid, j):
    import torch
    c = CONFIGS[cid]
    b, s, n, h1, h2, heads = c["b"], c["s"], c["n"], c["h1"], c["h2"], c["heads"]
    D = h1 // heads
    fmt = c["kv_fmt"]
    Wo, layer = _layer(hp, orc, cid, j)
    req = PREFILL_REQ[cid]
    d = hp.dims(b, s, n, h1, h2, 1, heads, c["gbs"])
    ws = torch.empty(hp.hp_workspace_bytes(d), dtype=torch.uint8, device="cuda")
    kv = hp.KVCache(fmt, b, heads, s + n, D)
    xs = _sampled("prompt", cid, req, (s, h1))
    x = _filled((b, s, h1), 1.0, req, xs, 100 + cid)
    y = torch.empty((b, s, h1), dtype=torch.float16, device="cuda")
    cap = _captures(hp, b * s, h1, h2)
    hp.hp_debug_set_capture(**cap)
    try:
        hp.hp_layer_prefill(d, layer, x, kv, y, ws)
    finally:
        hp.hp_debug_set_capture(off=True)
    torch.cuda.synchronize()
    stats = {}
    with cf.ThreadPoolExecutor(16) as pool:
        for i, r in enumerate(req):
            rows = slice(r * s, (r + 1) * s)
            Q = host(cap["qkv"][rows])
            A = host(cap["attn"][rows])
            XO = host(cap["x_out"][rows])
            HID = host(cap["hidden"][rows])
            Y = host(y[r])
            w = f"config {cid} layer {j} prefill r{r}"
            qkv_ref = orc.gemm(xs[i][ROWS], Wo["wqkv"])
            _stage(f"{w} QKV", Q[ROWS], qkv_ref, stats)
            for t, col in (("k", 1), ("v", 2)):
                rows_f16 = _head_rows(Q[:, col * h1:(col + 1) * h1], heads)
                g = host(getattr(kv, t)[r])[:, :s]
                gs = host(getattr(kv, t + "_sm")[r])[:, :s] if fmt == 1 else None
                _check_codes(orc, fmt, g, gs, rows_f16, f"{w} {t} codes")
            ref_a = _attn_heads(orc, pool, Q[:, :h1], Q[:, h1:2 * h1], Q[:, 2 * h1:],
                                np.arange(1, s + 1, dtype=np.int32), heads)
            _stage(f"{w} attention (all {s} rows, {heads} heads)", A, ref_a, stats)
            _stage(f"{w} x_out", XO[ROWS], orc.gemm(A[ROWS], Wo["wo"], res=xs[i][ROWS]), stats)
            _stage(f"{w} hidden", HID[ROWS], orc.gemm(XO[ROWS], Wo["w1"], relu=True), stats)
            _stage(f"{w} output", Y[ROWS], orc.gemm(HID[ROWS], Wo["w2"], res=XO[ROWS]), stats)
            if fmt == 1:  # free-running: the oracle's own K/V from x
                for t, col in (("k", 1), ("v", 2)):
                    g = host(getattr(kv, t)[r])[:, ROWS]
                    fr, mx = _flips(orc, g, _head_rows(qkv_ref[:, col * h1:(col + 1) * h1], heads))
                    stats[f"{w} free-running {t} code flip rate"] = fr
                    assert mx <= 1, f"{w}: a free-running {t} code moved by {mx} levels"
    for k, v in stats.items():
        print(f"{k}: {v:.3g}")


def _decode(hp, orc, cid, j):
    import torch
    c = CONFIGS[cid]
    b, s, n, h1, h2, heads = c["b"], c["s"], c["n"], c["h1"], c["h2"], c["heads"]
    D = h1 // heads
    fmt = c["kv_fmt"]
    Wo, layer = _layer(hp, orc, cid, j)
    req = DECODE_REQ[cid]
    d = hp.dims(b, s, n, h1, h2, 1, heads, c["gbs"])
    ws = torch.empty(hp.hp_workspace_bytes(d), dtype=torch.uint8, device="cuda")
    kv = hp.KVCache(fmt, b, heads, s + n, D)
    T = s + n // 2  # the block's mean cache length; the new token goes to row T
    sig_kv = 0.02 * math.sqrt(h1)  # scale of x w for x ~ N(0,1), w ~ N(0, 0.02^2)
    ks = _sampled("cache_k", cid, req, (T, h1), sig_kv)
    vs = _sampled("cache_v", cid, req, (T, h1), sig_kv)
    qkv = _filled((b, T, 3 * h1), sig_kv, [], [], 200 + cid)
    for i, r in enumerate(req):
        qkv[r, :, h1:2 * h1].copy_(dev(ks[i]))
        qkv[r, :, 2 * h1:].copy_(dev(vs[i]))
    hp.hp_kv_append(b, T, h1, heads, qkv, 0, kv)
    del qkv
    ts = _sampled("token", cid, req, (1, h1))
    t = _filled((b, 1, h1), 1.0, req, ts, 300 + cid)
    to = torch.empty((b, 1, h1), dtype=torch.float16, device="cuda")
    cap = _captures(hp, b, h1, h2)
    hp.hp_debug_set_capture(**cap)
    try:
        hp.hp_layer_decode(d, layer, t, T, 1, kv, to, ws)
    finally:
        hp.hp_debug_set_capture(off=True)
    torch.cuda.synchronize()
    # every request of the batch: the layer's four products against the
    # standalone product on the same fp16 inputs, bit for bit (a row's result
    # depends neither on the caller nor on the workspace it runs in)
    t0, o0 = t[:, 0], to[:, 0]
    for xin, mat, res, relu, got, name in (
            (t0, layer.wqkv, None, False, cap["qkv"], "QKV"),
            (cap["attn"], layer.wo, t0, False, cap["x_out"], "x_out"),
            (cap["x_out"], layer.w1, None, True, cap["hidden"], "hidden"),
            (cap["hidden"], layer.w2, cap["x_out"], False, o0, "output")):
        ref = hp.hp_gemm(xin, mat, res=res, relu=relu)
        assert torch.equal(ref.view(torch.int16), got.view(torch.int16)), \
            f"config {cid} layer {j} decode {name}: the layer's product differs from hp_gemm"
    ridx = list(req)
    Q, A = host(cap["qkv"])[ridx], host(cap["attn"])[ridx]
    XO, HID, Y = host(cap["x_out"])[ridx], host(cap["hidden"])[ridx], host(to)[ridx, 0]
    x0 = ts[:, 0]
    w = f"config {cid} layer {j} decode"
    stats = {}
    kv_ref = orc.gemm(x0, Wo["wqkv"])
    _stage(f"{w} QKV", Q, kv_ref, stats)
    with cf.ThreadPoolExecutor(16) as pool:
        for i, r in enumerate(req):
            Kc, Vc = [], []
            for t_, col, hist in (("k", 1, ks), ("v", 2, vs)):
                g = host(getattr(kv, t_)[r])[:, :T + 1]
                gs = host(getattr(kv, t_ + "_sm")[r])[:, :T + 1] if fmt == 1 else None
                # history rows: appended from the same fp16 values on both sides
                _check_codes(orc, fmt, g[:, :T], None if gs is None else gs[:, :T],
                             _head_rows(hist[i], heads), f"{w} r{r} {t_} history")
                # the new row: coded from the GPU's own K/V (teacher forced)
                new = _head_rows(Q[i:i + 1, col * h1:(col + 1) * h1], heads)
                _check_codes(orc, fmt, g[:, T:], None if gs is None else gs[:, T:], new,
                             f"{w} r{r} {t_} new row")
                if fmt == 1:
                    fr, mx = _flips(orc, g[:, T:],
                                    _head_rows(kv_ref[i:i + 1, col * h1:(col + 1) * h1], heads))
                    stats[f"{w} r{r} free-running {t_} code flip rate"] = fr
                    assert mx <= 1, f"{w}: a free-running {t_} code moved by {mx} levels"
                    vals = orc.dequantize_g64(g, gs.view(np.uint16))
                else:
                    vals = g.view(np.float16)
                (Kc if t_ == "k" else Vc).append(vals.transpose(1, 0, 2).reshape(T + 1, h1))
            ref_a = _attn_heads(orc, pool, Q[i:i + 1, :h1], Kc[0], Vc[0],
                                np.array([T + 1], np.int32), heads)
            _stage(f"{w} r{r} attention ({heads} heads, T = {T + 1})", A[i:i + 1], ref_a, stats)
    _stage(f"{w} x_out", XO, orc.gemm(A, Wo["wo"], res=x0), stats)
    _stage(f"{w} hidden", HID, orc.gemm(XO, Wo["w1"], relu=True), stats)
    _stage(f"{w} output", Y, orc.gemm(HID, Wo["w2"], res=XO), stats)
    for k, v in stats.items():
        print(f"{k}: {v:.3g}")


@pytest.mark.parametrize("cid,kind,j", CASES)
def test_layer_stages_teacher_forced(hp, orc, cid, kind, j):
    (_prefill if kind == "prefill" else _decode)(hp, orc, cid, j)
