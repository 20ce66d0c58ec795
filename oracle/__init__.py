"""Python access to the CPU oracle (oracle.cpp) -- test infrastructure only.

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product path never does.  Arrays are numpy; binary16 data
travels as numpy float16 (the oracle reads the raw bits).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c++17", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
          "-fPIC", "-shared", "-Wall"]


def build(force: bool = True) -> str:
    """Compile oracle.cpp into liboracle.so with g++ (no GPU toolchain)."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        subprocess.check_call(["g++", *CFLAGS, _SRC, "-o", tmp])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None
_p = C.c_void_p
_i64 = C.c_int64
_int = C.c_int


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = C.CDLL(LIB_PATH)
        L.or_h2f.restype = C.c_float
        L.or_h2f.argtypes = [C.c_uint16]
        L.or_d2h.restype = C.c_uint16
        L.or_d2h.argtypes = [C.c_double]
        L.or_f2h.restype = C.c_uint16
        L.or_f2h.argtypes = [C.c_float]
        for name in ("or_h2f_array", "or_f2h_array", "or_d2h_array"):
            getattr(L, name).argtypes = [_p, _p, _i64]
        L.or_threads.restype = _int
        L.or_quantize_g64.argtypes = [_p, _i64, _i64, _p, _p]
        L.or_dequantize_g64.argtypes = [_p, _p, _i64, _i64, _p]
        L.or_gemm.argtypes = [_p, _i64, _p, _i64, _i64, _i64, _p, _i64, _int, _p, _i64]
        L.or_attention.argtypes = [_int, _int, _p, _p, _p, _p, _p, _int, _p]
        L.or_layer_prefill.argtypes = [_int] * 5 + [_p] * 7 + [_int, _int, _p, _p, _p, _p, _int, _p]
        L.or_layer_decode.argtypes = [_int] * 6 + [_p] * 8 + [_int, _int, _p, _p, _p, _p, _p]
        L.or_kv_append.argtypes = [_int] * 5 + [_p, _p, _int, _int, _p, _p, _p, _p]
        L.or_tree_masks.restype = _int
        L.or_tree_masks.argtypes = [_p, _int, _p]
        L.or_tree_prune.restype = _int
        L.or_tree_prune.argtypes = [_p, _int, _int, _p, _p, _p]
        L.or_run_block.argtypes = [_int] * 9 + [_p, _p, _p, _int, _int, _p, _p, _p, _p, _p, _p]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


F16, Q4 = 0, 1


def threads() -> int:
    return int(lib().or_threads())


# --------------------------------------------------------------- binary16
def h2f(h: np.ndarray) -> np.ndarray:
    h = _c(h, np.uint16)
    out = np.empty(h.shape, np.float32)
    lib().or_h2f_array(_ptr(h), _ptr(out), h.size)
    return out


def f2h(f: np.ndarray) -> np.ndarray:
    f = _c(f, np.float32)
    out = np.empty(f.shape, np.uint16)
    lib().or_f2h_array(_ptr(f), _ptr(out), f.size)
    return out


def d2h(d: np.ndarray) -> np.ndarray:
    d = _c(d, np.float64)
    out = np.empty(d.shape, np.uint16)
    lib().or_d2h_array(_ptr(d), _ptr(out), d.size)
    return out


def _bits(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        return a.view(np.uint16)
    assert a.dtype == np.uint16, a.dtype
    return a


# ---------------------------------------------------------- quantisation
def quantize_g64(x: np.ndarray):
    """x[..., cols] fp16 -> (codes uint8[..., cols/2], sm uint16[..., cols/64, 2])."""
    xb = _bits(x)
    cols = xb.shape[-1]
    assert cols % 64 == 0
    rows = xb.size // cols
    codes = np.empty(xb.shape[:-1] + (cols // 2,), np.uint8)
    sm = np.empty(xb.shape[:-1] + (cols // 64, 2), np.uint16)
    lib().or_quantize_g64(_ptr(xb), rows, cols, _ptr(codes), _ptr(sm))
    return codes, sm


def dequantize_g64(codes: np.ndarray, sm: np.ndarray) -> np.ndarray:
    codes = _c(codes, np.uint8)
    sm = _c(sm, np.uint16)
    cols = codes.shape[-1] * 2
    rows = codes.size // (cols // 2)
    y = np.empty(codes.shape[:-1] + (cols,), np.uint16)
    lib().or_dequantize_g64(_ptr(codes), _ptr(sm), rows, cols, _ptr(y))
    return y.view(np.float16)


# --------------------------------------------------------------- products
def gemm(x, w, res=None, relu=False) -> np.ndarray:
    """fp16 y = act(x @ w) + res with double sums (x[M][K], w[K][N])."""
    xb, wb = _bits(x), _bits(w)
    M, K = xb.shape
    K2, N = wb.shape
    assert K == K2
    rb = None if res is None else _bits(res)
    y = np.empty((M, N), np.uint16)
    lib().or_gemm(_ptr(xb), K, _ptr(wb), M, K, N, _ptr(rb), N, int(relu), _ptr(y), N)
    return y.view(np.float16)


def attention(q, k, v, lim, mask=None, tbase=0) -> np.ndarray:
    """One head: q[nq][d], k, v [T][d]; query i sees keys j < lim[i] and tbase+u for bits u of mask[i]."""
    qb, kb, vb = _bits(q), _bits(k), _bits(v)
    nq, d = qb.shape
    lim = _c(lim, np.int32)
    m = None if mask is None else _c(mask, np.uint64)
    out = np.empty((nq, d), np.uint16)
    lib().or_attention(d, nq, _ptr(qb), _ptr(kb), _ptr(vb), _ptr(lim), _ptr(m), tbase, _ptr(out))
    return out.view(np.float16)


def topk_count(T: int) -> int:
    """[FlexGen] section 5 (sparse attention): the top 10% of the T cached tokens,
    read as ceil(T / 10), at least one."""
    return max(1, -(-int(T) // 10))


def topk_attention(q, k, v, topk: int):
    """[FlexGen] section 5, sparse attention: one query q[d] against the cached keys
    k[T][d] and values v[T][d] (binary16 values, dequantised where the cache is int4).
    Scores z_j = q . k_j (double; the 1/sqrt(d) scale does not change the order); the
    topk largest are kept, ties going to the lower index; the other tokens are dropped
    and the output is the attention over the kept keys alone (the softmax renormalised
    over them).  Returns (out binary16 [d], kept indices in ascending order)."""
    qb, kb, vb = _bits(q).reshape(-1), _bits(k), _bits(v)
    T = kb.shape[0]
    if not 1 <= topk <= T:
        raise ValueError("topk must be in [1, T]")
    z = h2f(kb).astype(np.float64) @ h2f(qb).astype(np.float64)
    order = np.argsort(-z, kind="stable")  # descending; equal scores keep index order
    kept = np.sort(order[:topk])
    out = attention(qb.reshape(1, -1), kb[kept], vb[kept], [topk])[0]
    return out, kept


def tree_masks(parent) -> np.ndarray:
    p = _c(parent, np.int32)
    m = np.zeros(p.shape[0], np.uint64)
    rc = lib().or_tree_masks(_ptr(p), p.shape[0], _ptr(m))
    if rc != 0:
        raise ValueError("invalid parent array")
    return m


def tree_prune(parent, u: int):
    """[SpecPipe] sub-tree pruning for verified token u: (new_parent [nq], src [nq], kept,
    depth).  kept = size of u's subtree (the new tree, u at index 0); depth = length of
    the verified path above u (cache rows committed to the prefix); src[j], j < depth +
    kept, = old index of the token whose row goes to position j after the old prefix."""
    p = _c(parent, np.int32)
    new_parent = np.zeros(p.shape[0], np.int32)
    src = np.zeros(p.shape[0], np.int32)
    depth = np.zeros(1, np.int32)
    kept = lib().or_tree_prune(_ptr(p), p.shape[0], int(u), _ptr(new_parent), _ptr(src),
                               _ptr(depth))
    if kept < 0:
        raise ValueError("invalid parent array or verified index")
    return new_parent, src, kept, int(depth[0])


def kv_compact(kv, pos: int, src, count):
    """Moves the rows that survive pruning into place: for request r, rows pos + j
    (j < count[r]) of every head take rows pos + src[r][j] (K and V, codes and
    scale/min); other rows untouched."""
    for r in range(kv.b):
        idx = pos + np.asarray(src[r][:count[r]], np.int64)
        dst = slice(pos, pos + int(count[r]))
        for arr in (kv.k, kv.v, kv.ksm, kv.vsm):
            if arr is not None:
                arr[r][:, dst] = arr[r][:, idx].copy()


# ----------------------------------------------------------------- layers
class KV:
    """One layer's cache in the oracle's layout (see oracle.cpp)."""

    def __init__(self, fmt: int, b: int, heads: int, cap: int, d: int):
        self.fmt, self.b, self.heads, self.cap, self.d = fmt, b, heads, cap, d
        if fmt == F16:
            self.k = np.zeros((b, heads, cap, d), np.uint16)
            self.v = np.zeros((b, heads, cap, d), np.uint16)
            self.ksm = self.vsm = None
        else:
            self.k = np.zeros((b, heads, cap, d // 2), np.uint8)
            self.v = np.zeros((b, heads, cap, d // 2), np.uint8)
            self.ksm = np.zeros((b, heads, cap, d // 64, 2), np.uint16)
            self.vsm = np.zeros((b, heads, cap, d // 64, 2), np.uint16)

    def args(self):
        return (self.fmt, self.cap, _ptr(self.k), _ptr(self.v), _ptr(self.ksm), _ptr(self.vsm))

    def values(self, which: str, T: int) -> np.ndarray:
        """Rows [0, T) as fp16 values [b][heads][T][d] (dequantised for int4)."""
        if self.fmt == F16:
            return getattr(self, which)[:, :, :T].copy().view(np.float16)
        codes = getattr(self, which)[:, :, :T]
        sm = getattr(self, which + "sm")[:, :, :T]
        return dequantize_g64(codes, sm)


def kv_append(kv: KV, k_rows, v_rows, pos: int) -> None:
    """Stores k_rows, v_rows [b][nq][h1] (fp16) as cache rows [pos, pos + nq)."""
    kb, vb = _bits(k_rows), _bits(v_rows)
    b, nq, h1 = kb.shape
    assert vb.shape == kb.shape and b == kv.b and pos + nq <= kv.cap
    lib().or_kv_append(b, nq, h1, kv.heads, pos, _ptr(kb), _ptr(vb), *kv.args())


def _w6(W):
    return [_bits(W[n]) for n in ("wq", "wk", "wv", "wo", "w1", "w2")]


def layer_prefill(x, W, kv: KV, heads: int, causal: bool = True) -> np.ndarray:
    """x[b][s][h1] -> next-layer activations; fills cache rows [0, s)."""
    xb = _bits(x)
    b, s, h1 = xb.shape
    w = _w6(W)
    h2 = w[4].shape[1]
    y = np.empty_like(xb)
    lib().or_layer_prefill(b, s, h1, h2, heads, _ptr(xb), *[_ptr(a) for a in w], *kv.args(),
                           int(causal), _ptr(y))
    return y.view(np.float16)


def layer_decode(t, W, kv: KV, heads: int, pos: int, masks=None) -> np.ndarray:
    """t[b][nq][h1] at cache rows [pos, pos+nq) -> next-layer activations."""
    tb = _bits(t)
    b, nq, h1 = tb.shape
    w = _w6(W)
    h2 = w[4].shape[1]
    m = None if masks is None else _c(masks, np.uint64)
    y = np.empty_like(tb)
    lib().or_layer_decode(b, nq, h1, h2, heads, pos, _ptr(m), _ptr(tb), *[_ptr(a) for a in w],
                          *kv.args(), _ptr(y))
    return y.view(np.float16)


def layer_decode_topk(t, W, kv: KV, heads: int, pos: int, topk: int = 0) -> np.ndarray:
    """The decode step of layer_decode (one new token per request, t[b][1][h1] at cache
    row pos) with the Top-K sparse attention of [FlexGen] section 5 in place of the
    attention: K = topk (at most pos + 1) kept rows per (request, head), or
    ceil((pos + 1) / 10) for topk 0.  Same steps and fp16 rounding points as
    layer_decode: Q, K, V products, append, attention, then the output projection with
    the residual and the ReLU MLP with the residual."""
    tb = _bits(t)
    b, nq, h1 = tb.shape
    assert nq == 1
    d = h1 // heads
    x = tb.reshape(b, h1)
    q, k, v = gemm(x, W["wq"]), gemm(x, W["wk"]), gemm(x, W["wv"])
    kv_append(kv, k.reshape(b, 1, h1), v.reshape(b, 1, h1), pos)
    T = pos + 1
    K = min(topk, T) if topk > 0 else topk_count(T)
    Kc, Vc = kv.values("k", T), kv.values("v", T)
    a = np.empty((b, h1), np.float16)
    for r in range(b):
        for h in range(heads):
            cols = slice(h * d, (h + 1) * d)
            a[r, cols] = topk_attention(q[r, cols], Kc[r, h], Vc[r, h], K)[0]
    x_out = gemm(a, W["wo"], res=x)
    hid = gemm(x_out, W["w1"], relu=True)
    return gemm(hid, W["w2"], res=x_out).reshape(b, 1, h1)


def run_block_topk(x, t_in, layers, kvs, heads: int, topk: int = 0):
    """run_block (zig-zag order; requests never interact, so the order does not change
    the result) with layer_decode_topk in every decode column."""
    b, s, h1 = _bits(x).shape
    n = _bits(t_in).shape[0]
    cur = np.asarray(x)
    for j, W in enumerate(layers):
        cur = layer_prefill(cur, W, kvs[j], heads)
    t_out = np.empty((n, b, h1), np.float16)
    for i in range(n):
        tcur = np.asarray(t_in)[i].reshape(b, 1, h1)
        for j, W in enumerate(layers):
            tcur = layer_decode_topk(tcur, W, kvs[j], heads, s + i, topk)
        t_out[i] = tcur.reshape(b, h1)
    return cur, t_out


def run_block(x, t_in, layers, kvs, heads: int, gbs: int, order: int = 0):
    """Whole block: prefill column then n decode columns over all layers.

    layers: list of dicts of fp16 weights; kvs: list of KV; order 0 zig-zag, 1 row-by-row,
    2 diagonal (the KV arrays then need only min(b/gbs, n+1) GPU batches of requests).
    Returns (x_out[b][s][h1], t_out[n][b][h1])."""
    xb, tb = _bits(x), _bits(t_in)
    b, s, h1 = xb.shape
    n = tb.shape[0]
    l = len(layers)
    ws = [a for W in layers for a in _w6(W)]
    h2 = ws[4].shape[1]
    wp = (C.c_void_p * (6 * l))(*[a.ctypes.data for a in ws])
    kp = (C.c_void_p * l)(*[kv.k.ctypes.data for kv in kvs])
    vp = (C.c_void_p * l)(*[kv.v.ctypes.data for kv in kvs])
    fmt = kvs[0].fmt
    ksp = (C.c_void_p * l)(*[(kv.ksm.ctypes.data if fmt == Q4 else 0) for kv in kvs])
    vsp = (C.c_void_p * l)(*[(kv.vsm.ctypes.data if fmt == Q4 else 0) for kv in kvs])
    x_out = np.empty_like(xb)
    t_out = np.empty_like(tb)
    lib().or_run_block(b, s, n, h1, h2, l, heads, gbs, order, _ptr(xb), _ptr(tb), wp, fmt,
                       kvs[0].cap, kp, vp, ksp, vsp, _ptr(x_out), _ptr(t_out))
    return x_out.view(np.float16), t_out.view(np.float16)
