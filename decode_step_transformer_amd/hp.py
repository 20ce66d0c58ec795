"""ctypes binding of libhp (include/hp.h): argument marshalling only.

Every function named hp_* here calls the C entry point of the same name.
Tensors are torch CUDA (HIP) tensors; the binding passes their device
pointers, sizes and the current stream, and raises HPError on a non-zero
status.  Nothing here computes any part of the layer: if libhp.so is missing
the import fails loudly (there is no fallback path).
"""
from __future__ import annotations

import ctypes as C
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhp.so")

HP_F16, HP_Q4 = 0, 1
HP_GRAPH, HP_ROW_BY_ROW, HP_MICROBATCH, HP_TOPK10, HP_DIAGONAL = 1, 2, 4, 8, 16


class HPError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"hp status {status}: {msg}")
        self.status = status


class hp_mat(C.Structure):
    _fields_ = [("fmt", C.c_int32), ("k", C.c_int32), ("n", C.c_int32),
                ("data", C.c_void_p), ("scale", C.c_void_p), ("minv", C.c_void_p)]


class hp_layer(C.Structure):
    _fields_ = [("wqkv", hp_mat), ("wo", hp_mat), ("w1", hp_mat), ("w2", hp_mat)]


class hp_kv(C.Structure):
    _fields_ = [("fmt", C.c_int32), ("cap", C.c_int32), ("k", C.c_void_p), ("v", C.c_void_p),
                ("k_sm", C.c_void_p), ("v_sm", C.c_void_p), ("pages", C.c_void_p),
                ("page_rows", C.c_int32), ("pool_pages", C.c_int32)]


class hp_capture(C.Structure):
    _fields_ = [("qkv", C.c_void_p), ("attn", C.c_void_p), ("x_out", C.c_void_p),
                ("hidden", C.c_void_p)]


class hp_dims(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("b", "s", "n", "h1", "h2", "l", "heads", "gbs")]


EXPORTS = [
    "hp_last_error", "hp_device_check", "hp_quantize_g64", "hp_dequantize_g64",
    "hp_pack_weight_q4", "hp_pack_weight_f16", "hp_gemm_workspace_bytes", "hp_gemm",
    "hp_gemm_noalloc",
    "hp_kv_append", "hp_prefill_attention", "hp_decode_attention", "hp_decode_attention_ragged",
    "hp_topk_attention",
    "hp_tree_masks",
    "hp_tree_prune", "hp_kv_compact",
    "hp_workspace_bytes", "hp_layer_prefill", "hp_layer_decode", "hp_run_block",
    "hp_release_graphs", "hp_weight_bytes", "hp_kv_bytes", "hp_profile", "hp_profile_read",
    "hp_debug_set_capture", "hp_kv_append_ragged", "hp_diagonal_pages",
    "hp_peak_read", "hp_peak_mfma",
]

_lib = None
_p, _i32, _i64, _sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t


def lib():
    """Loads libhp.so (built by __graft_entry__.build()); raises if it is absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: run __graft_entry__.build() first")
        L = C.CDLL(LIB_PATH)
        L.hp_last_error.restype = C.c_char_p
        L.hp_device_check.restype = _i32
        sigs = {
            "hp_quantize_g64": [_p, _i64, _i64, _p, _p, _p],
            "hp_dequantize_g64": [_p, _p, _i64, _i64, _p, _p],
            "hp_pack_weight_q4": [_p, _p, _i32, _i32, _p, _p, _p, _p],
            "hp_pack_weight_f16": [_p, _i32, _i32, _p, _p],
            "hp_gemm": [_p, _i64, C.POINTER(hp_mat), _i64, _p, _i64, _i32, _p, _i64, _p, _sz, _p],
            "hp_gemm_noalloc": [_p, _i64, C.POINTER(hp_mat), _i64, _p, _i64, _i32, _p, _i64, _p],
            "hp_kv_append": [_i32, _i32, _i32, _i32, _p, _i32, C.POINTER(hp_kv), _p],
            "hp_kv_append_ragged": [_i32, _i32, _i32, _i32, _p, _p, _i32, C.POINTER(hp_kv), _p],
            "hp_prefill_attention": [_i32, _i32, _i32, _i32, _p, _p, _p],
            "hp_decode_attention": [_i32, _i32, _i32, _i32, _p, _i32, _p, C.POINTER(hp_kv), _p, _p],
            "hp_topk_attention": [_i32, _i32, _i32, _p, _i32, _i32, C.POINTER(hp_kv), _p, _p, _p],
            "hp_tree_masks": [_i32, _i32, _p, _p, _p, _p],
            "hp_decode_attention_ragged": [_i32, _i32, _i32, _i32, _p, _p, _i32, _p,
                                           C.POINTER(hp_kv), _p, _p],
            "hp_tree_prune": [_i32, _i32, _p, _p, _i32, _p, _p, _p, _p, _p, _p],
            "hp_kv_compact": [_i32, _i32, _i32, _i32, _i32, _p, _p, _p, C.POINTER(hp_kv), _p],
            "hp_layer_prefill": [C.POINTER(hp_dims), C.POINTER(hp_layer), _p, C.POINTER(hp_kv), _p,
                                 _p, _sz, _p],
            "hp_layer_decode": [C.POINTER(hp_dims), C.POINTER(hp_layer), _p, _i32, _i32, _p,
                                C.POINTER(hp_kv), _p, _p, _sz, _p],
            "hp_run_block": [C.POINTER(hp_dims), C.POINTER(hp_layer), _p, _p, C.POINTER(hp_kv), _p,
                             _p, _p, _sz, C.c_uint32, C.POINTER(C.c_float), _p],
            "hp_peak_read": [_p, C.c_uint64, _i32, _p, _p],
            "hp_peak_mfma": [_i32, _i32, _p, _p],
        }
        for name, args in sigs.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = _i32
        L.hp_gemm_workspace_bytes.argtypes = [_i64, _i32, _i32, _i32]
        L.hp_gemm_workspace_bytes.restype = _sz
        L.hp_workspace_bytes.argtypes = [C.POINTER(hp_dims)]
        L.hp_workspace_bytes.restype = _sz
        L.hp_weight_bytes.argtypes = [C.POINTER(hp_dims), _i32]
        L.hp_weight_bytes.restype = C.c_uint64
        L.hp_kv_bytes.argtypes = [C.POINTER(hp_dims), _i32]
        L.hp_kv_bytes.restype = C.c_uint64
        L.hp_release_graphs.restype = None
        L.hp_diagonal_pages.argtypes = [C.POINTER(hp_dims), _i32]
        L.hp_diagonal_pages.restype = C.c_int64
        L.hp_debug_set_capture.argtypes = [C.POINTER(hp_capture)]
        L.hp_debug_set_capture.restype = _i32
        L.hp_profile.argtypes = [_i32]
        L.hp_profile.restype = _i32
        L.hp_profile_read.argtypes = [C.c_char_p, _sz]
        L.hp_profile_read.restype = _i32
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise HPError(status, lib().hp_last_error().decode())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _need(t, dtype, name):
    if t.dtype != dtype or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name}: need a contiguous {dtype} device tensor")


# ------------------------------------------------------------ diagnostics
def hp_device_check() -> int:
    return int(lib().hp_device_check())


def hp_last_error() -> str:
    return lib().hp_last_error().decode()


# ------------------------------------------------------------ compression
def hp_quantize_g64(x: torch.Tensor, stream=None):
    """x fp16 [..., cols] -> (codes uint8 [..., cols/2], sm int16 [..., cols/64, 2] = scale, min bits)."""
    _need(x, torch.float16, "x")
    cols = x.shape[-1]
    rows = x.numel() // cols if cols else 0
    codes = torch.empty(x.shape[:-1] + (cols // 2,), dtype=torch.uint8, device=x.device)
    sm = torch.empty(x.shape[:-1] + (cols // 64, 2), dtype=torch.int16, device=x.device)
    _check(lib().hp_quantize_g64(_ptr(x), rows, cols, _ptr(codes), _ptr(sm), _stream(stream)))
    return codes, sm


def hp_dequantize_g64(codes: torch.Tensor, sm: torch.Tensor, stream=None) -> torch.Tensor:
    _need(codes, torch.uint8, "codes")
    cols = codes.shape[-1] * 2
    rows = codes.numel() // (cols // 2)
    y = torch.empty(codes.shape[:-1] + (cols,), dtype=torch.float16, device=codes.device)
    _check(lib().hp_dequantize_g64(_ptr(codes), _ptr(sm), rows, cols, _ptr(y), _stream(stream)))
    return y


class Mat:
    """A weight in the GEMM layout (keeps its device tensors alive)."""

    def __init__(self, fmt, k, n, data, scale=None, minv=None):
        self.fmt, self.k, self.n = fmt, k, n
        self.data, self.scale, self.minv = data, scale, minv

    def c(self) -> hp_mat:
        return hp_mat(self.fmt, self.k, self.n, _ptr(self.data), _ptr(self.scale), _ptr(self.minv))

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.data, self.scale, self.minv)
                   if t is not None)


def hp_pack_weight_q4(codes: torch.Tensor, sm: torch.Tensor, k: int, n: int, stream=None) -> Mat:
    dev = codes.device
    packed = torch.empty(n * k // 2, dtype=torch.uint8, device=dev)
    scale = torch.empty((n // 64, k), dtype=torch.float16, device=dev)
    minv = torch.empty((n // 64, k), dtype=torch.float16, device=dev)
    _check(lib().hp_pack_weight_q4(_ptr(codes), _ptr(sm), k, n, _ptr(packed), _ptr(scale),
                                   _ptr(minv), _stream(stream)))
    return Mat(HP_Q4, k, n, packed, scale, minv)


def hp_pack_weight_f16(w: torch.Tensor, stream=None) -> Mat:
    _need(w, torch.float16, "w")
    k, n = w.shape
    wt = torch.empty(n * k, dtype=torch.float16, device=w.device)  # fragment-major tiles
    _check(lib().hp_pack_weight_f16(_ptr(w), k, n, _ptr(wt), _stream(stream)))
    return Mat(HP_F16, k, n, wt)


def make_weight(w: torch.Tensor, fmt: int, stream=None) -> Mat:
    """fp16 w[k][n] (page orientation) -> GEMM-layout weight in format fmt."""
    if fmt == HP_F16:
        return hp_pack_weight_f16(w, stream)
    codes, sm = hp_quantize_g64(w, stream)
    return hp_pack_weight_q4(codes, sm, w.shape[0], w.shape[1], stream)


# ---------------------------------------------------------- layer stages
def hp_gemm_workspace_bytes(M: int, k: int, n: int, fmt: int) -> int:
    return int(lib().hp_gemm_workspace_bytes(M, k, n, fmt))


def hp_gemm(x: torch.Tensor, w: Mat, res=None, relu=False, out=None, ws=None, stream=None):
    M = x.shape[0]
    y = out if out is not None else torch.empty((M, w.n), dtype=torch.float16, device=x.device)
    need = hp_gemm_workspace_bytes(M, w.k, w.n, w.fmt)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=x.device)
    mc = w.c()
    _check(lib().hp_gemm(_ptr(x), x.stride(0), C.byref(mc), M, _ptr(res),
                         res.stride(0) if res is not None else 0, int(relu), _ptr(y), y.stride(0),
                         _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream)))
    return y


def hp_gemm_noalloc(x: torch.Tensor, w: Mat, res=None, relu=False, out=None, stream=None):
    """hp_gemm without a workspace: split partials go to the library's static scratch."""
    M = x.shape[0]
    y = out if out is not None else torch.empty((M, w.n), dtype=torch.float16, device=x.device)
    mc = w.c()
    _check(lib().hp_gemm_noalloc(_ptr(x), x.stride(0), C.byref(mc), M, _ptr(res),
                                 res.stride(0) if res is not None else 0, int(relu), _ptr(y),
                                 y.stride(0), _stream(stream)))
    return y


class KVCache:
    """One layer's cache tensors in the library layout (see hp_kv).

    Contiguous: [b][heads][cap][row].  Paged (page_rows > 0): a pool of
    pool_pages pages [page][heads][page_rows][row]; `pages` (device int32
    [b][cap / page_rows], or None when hp_run_block assigns pages under
    HP_DIAGONAL) maps request rows to pages."""

    def __init__(self, fmt, b, heads, cap, d, device="cuda", page_rows=0, pool_pages=0,
                 pages=None):
        self.fmt, self.b, self.heads, self.cap, self.d = fmt, b, heads, cap, d
        self.page_rows, self.pool_pages, self.pages = page_rows, pool_pages, pages
        lead = (pool_pages, heads, page_rows) if page_rows else (b, heads, cap)
        if fmt == HP_F16:
            self.k = torch.zeros(lead + (d,), dtype=torch.float16, device=device)
            self.v = torch.zeros(lead + (d,), dtype=torch.float16, device=device)
            self.k_sm = self.v_sm = None
        else:
            self.k = torch.zeros(lead + (d // 2,), dtype=torch.uint8, device=device)
            self.v = torch.zeros(lead + (d // 2,), dtype=torch.uint8, device=device)
            self.k_sm = torch.zeros(lead + (d // 64, 2), dtype=torch.int16, device=device)
            self.v_sm = torch.zeros(lead + (d // 64, 2), dtype=torch.int16, device=device)

    def c(self) -> hp_kv:
        return hp_kv(self.fmt, self.cap, _ptr(self.k), _ptr(self.v), _ptr(self.k_sm),
                     _ptr(self.v_sm), _ptr(self.pages), self.page_rows, self.pool_pages)

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.k, self.v, self.k_sm, self.v_sm)
                   if t is not None)


def hp_kv_append(b, q, h1, heads, qkv, pos, kv: KVCache, stream=None):
    c = kv.c()
    _check(lib().hp_kv_append(b, q, h1, heads, _ptr(qkv), pos, C.byref(c), _stream(stream)))


def hp_kv_append_ragged(b, q, h1, heads, qkv, rpos, max_pos, kv: KVCache, stream=None):
    c = kv.c()
    _check(lib().hp_kv_append_ragged(b, q, h1, heads, _ptr(qkv), _ptr(rpos), max_pos, C.byref(c),
                                     _stream(stream)))


def hp_diagonal_pages(d: hp_dims, page_rows: int) -> int:
    return int(lib().hp_diagonal_pages(C.byref(d), page_rows))


def hp_prefill_attention(b, s, h1, heads, qkv, out=None, stream=None):
    out = out if out is not None else torch.empty((b, s, h1), dtype=torch.float16, device=qkv.device)
    _check(lib().hp_prefill_attention(b, s, h1, heads, _ptr(qkv), _ptr(out), _stream(stream)))
    return out


def hp_decode_attention(b, q, h1, heads, qkv, pos, kv: KVCache, masks=None, out=None, stream=None):
    out = out if out is not None else torch.empty((b, q, h1), dtype=torch.float16, device=qkv.device)
    c = kv.c()
    _check(lib().hp_decode_attention(b, q, h1, heads, _ptr(qkv), pos, _ptr(masks), C.byref(c),
                                     _ptr(out), _stream(stream)))
    return out


def hp_topk_attention(b, h1, heads, qkv, pos, kv: KVCache, topk=0, out=None, idx=False,
                      stream=None):
    """Top-K sparse decode attention; returns out [b][h1], or (out, idx [b][heads][K])
    when idx is True (K = topk, at most pos + 1, or ceil((pos + 1) / 10) for topk 0)."""
    out = out if out is not None else torch.empty((b, h1), dtype=torch.float16, device=qkv.device)
    T = pos + 1
    K = min(topk, T) if topk > 0 else -(-T // 10)
    ix = torch.empty((b, heads, K), dtype=torch.int32, device=qkv.device) if idx else None
    c = kv.c()
    _check(lib().hp_topk_attention(b, h1, heads, _ptr(qkv), pos, topk, C.byref(c), _ptr(out),
                                   _ptr(ix), _stream(stream)))
    return (out, ix) if idx else out


def hp_tree_masks(parent: torch.Tensor, stream=None):
    """parent int32 [b][q] (device) -> (masks int64 [b][q] (bit pattern), err int32 [1])."""
    b, q = parent.shape
    masks = torch.empty((b, q), dtype=torch.int64, device=parent.device)
    err = torch.empty(1, dtype=torch.int32, device=parent.device)
    _check(lib().hp_tree_masks(b, q, _ptr(parent), _ptr(masks), _ptr(err), _stream(stream)))
    return masks, err


def hp_decode_attention_ragged(b, q, h1, heads, qkv, prefix, max_prefix, kv: KVCache, masks=None,
                               out=None, stream=None):
    """hp_decode_attention with per-request prefix lengths (device int32 [b])."""
    out = out if out is not None else torch.empty((b, q, h1), dtype=torch.float16, device=qkv.device)
    c = kv.c()
    _check(lib().hp_decode_attention_ragged(b, q, h1, heads, _ptr(qkv), _ptr(prefix), max_prefix,
                                            _ptr(masks), C.byref(c), _ptr(out), _stream(stream)))
    return out


def hp_tree_prune(parent: torch.Tensor, verified: torch.Tensor, pos: int = 0, stream=None):
    """parent int32 [b][q], verified int32 [b] (device), tree rows after a prefix of pos
    rows -> (new_parent, src, prefix, kept, err), all device int32."""
    b, q = parent.shape
    new_parent = torch.empty((b, q), dtype=torch.int32, device=parent.device)
    src = torch.empty((b, q), dtype=torch.int32, device=parent.device)
    prefix = torch.empty(b, dtype=torch.int32, device=parent.device)
    kept = torch.empty(b, dtype=torch.int32, device=parent.device)
    err = torch.empty(1, dtype=torch.int32, device=parent.device)
    _check(lib().hp_tree_prune(b, q, _ptr(parent), _ptr(verified), pos, _ptr(new_parent),
                               _ptr(src), _ptr(prefix), _ptr(kept), _ptr(err), _stream(stream)))
    return new_parent, src, prefix, kept, err


def hp_kv_compact(b, q, h1, heads, pos, src, prefix, kept, kv: KVCache, stream=None):
    c = kv.c()
    _check(lib().hp_kv_compact(b, q, h1, heads, pos, _ptr(src), _ptr(prefix), _ptr(kept),
                               C.byref(c), _stream(stream)))


# ------------------------------------------------------------------ layers
def dims(b, s, n, h1, h2, l, heads, gbs=None) -> hp_dims:
    return hp_dims(b, s, n, h1, h2, l, heads, gbs if gbs else b)


def hp_workspace_bytes(d: hp_dims) -> int:
    return int(lib().hp_workspace_bytes(C.byref(d)))


class Layer:
    def __init__(self, wqkv: Mat, wo: Mat, w1: Mat, w2: Mat):
        self.wqkv, self.wo, self.w1, self.w2 = wqkv, wo, w1, w2

    def c(self) -> hp_layer:
        return hp_layer(self.wqkv.c(), self.wo.c(), self.w1.c(), self.w2.c())

    def nbytes(self) -> int:
        return sum(m.nbytes() for m in (self.wqkv, self.wo, self.w1, self.w2))


def make_layer(W: dict, fmt: int, stream=None) -> Layer:
    """W: fp16 device tensors wq, wk, wv, wo [h1][h1], w1 [h1][h2], w2 [h2][h1]."""
    wqkv = torch.cat([W["wq"], W["wk"], W["wv"]], dim=1).contiguous()
    return Layer(make_weight(wqkv, fmt, stream), make_weight(W["wo"], fmt, stream),
                 make_weight(W["w1"], fmt, stream), make_weight(W["w2"], fmt, stream))


def hp_layer_prefill(d: hp_dims, layer: Layer, x, kv: KVCache, x_out, ws, stream=None):
    lc, kc = layer.c(), kv.c()
    _check(lib().hp_layer_prefill(C.byref(d), C.byref(lc), _ptr(x), C.byref(kc), _ptr(x_out),
                                  _ptr(ws), ws.numel(), _stream(stream)))


def hp_layer_decode(d: hp_dims, layer: Layer, t, pos, q, kv: KVCache, t_out, ws, masks=None,
                    stream=None):
    lc, kc = layer.c(), kv.c()
    _check(lib().hp_layer_decode(C.byref(d), C.byref(lc), _ptr(t), pos, q, _ptr(masks),
                                 C.byref(kc), _ptr(t_out), _ptr(ws), ws.numel(), _stream(stream)))


def hp_debug_set_capture(qkv=None, attn=None, x_out=None, hidden=None, off=False):
    """Teacher-forcing diagnostics: later hp_layer_prefill / hp_layer_decode calls on
    this thread copy their stored fp16 intermediates into these device tensors
    (contiguous, M rows); off=True stops capturing."""
    if off:
        _check(lib().hp_debug_set_capture(None))
        return
    for t in (qkv, attn, x_out, hidden):
        if t is not None:
            _need(t, torch.float16, "capture buffer")
    c = hp_capture(_ptr(qkv), _ptr(attn), _ptr(x_out), _ptr(hidden))
    _check(lib().hp_debug_set_capture(C.byref(c)))


def hp_run_block(d: hp_dims, layers, x, t_in, kvs, x_out, t_out, ws, flags=0, timing=False,
                 stream=None):
    """Runs one block; returns (prefill_ms, decode_ms) when timing, else None."""
    L = (hp_layer * len(layers))(*[ly.c() for ly in layers])
    K = (hp_kv * len(kvs))(*[kv.c() for kv in kvs])
    times = (C.c_float * 2)() if timing else None
    _check(lib().hp_run_block(C.byref(d), L, _ptr(x), _ptr(t_in), K, _ptr(x_out), _ptr(t_out),
                              _ptr(ws), ws.numel(), flags, times, _stream(stream)))
    return (times[0], times[1]) if timing else None


def hp_release_graphs():
    lib().hp_release_graphs()


def hp_weight_bytes(d: hp_dims, fmt: int) -> int:
    return int(lib().hp_weight_bytes(C.byref(d), fmt))


def hp_kv_bytes(d: hp_dims, fmt: int) -> int:
    return int(lib().hp_kv_bytes(C.byref(d), fmt))


# ---------------------------------------------------------------- profiling
def hp_profile(on: bool):
    lib().hp_profile(1 if on else 0)


def hp_peak_read(x: torch.Tensor, workgroups: int, sink: torch.Tensor, stream=None):
    """Streams x once (a measurement probe, see include/hp.h)."""
    _check(lib().hp_peak_read(_ptr(x), x.numel() * x.element_size(), workgroups, _ptr(sink),
                              _stream(stream)))


def hp_peak_mfma(iters: int, workgroups: int, sink: torch.Tensor, stream=None):
    """8 * 16 * iters fp16 16x16x32 MFMAs per workgroup (a measurement probe)."""
    _check(lib().hp_peak_mfma(iters, workgroups, _ptr(sink), _stream(stream)))


def hp_profile_read() -> dict:
    """{kernel: (launches, total_ms)} of the launches recorded since hp_profile(True)."""
    buf = C.create_string_buffer(1 << 16)
    n = lib().hp_profile_read(buf, len(buf))
    if n < 0:
        raise HPError(n, hp_last_error())
    out = {}
    for ln in buf.value.decode().splitlines():
        name, cnt, ms = ln.split()
        out[name] = (int(cnt), float(ms))
    return out
