"""Seeded synthetic inputs shared by the CPU oracle's tests and the GPU path.

This module holds none of the method's arithmetic: it only draws numbers.
Every tensor is a pure function of (seed, stream, index), so any slice of any
tensor can be regenerated on its own, and the same bits reach both sides.

Generator: a counter-based SplitMix64 stream (Steele, Lea and Flood,
"Fast splittable pseudorandom number generators", OOPSLA 2014): the i-th
64-bit word of stream `stream` under seed `seed` is mix64(key + (i + 1) * G),
with key = mix64(seed * P + stream), G the golden-ratio increment
0x9E3779B97F4A7C15 and mix64 the SplitMix64 finaliser.  Normal deviates come
from the Box-Muller transform (Box and Muller, 1958) applied to pairs of
words; each is scaled by sigma and rounded to IEEE binary16 by numpy.  The
words and the normals in binary64 come from synth/gen.c (OpenMP, built on
first use), so full-size tensors take seconds; `words` below is the same
generator in numpy, kept as the reference that the C build is checked
against.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_G = np.uint64(0x9E3779B97F4A7C15)
_P = np.uint64(0xD1B54A32D192ED03)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 24


def _mix64(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def _key(seed: int, stream: int) -> np.uint64:
    with np.errstate(over="ignore"):
        s = np.array([seed], dtype=np.uint64) * _P + np.array([stream], dtype=np.uint64)
        return _mix64(s)[0]


def words(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    """64-bit words [start, start+count) of one stream (uint64 array)."""
    key = _key(seed, stream)
    idx = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix64(key + idx * _G)


_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None
_lock = threading.Lock()


def build(force: bool = False) -> str:
    """Compiles synth/gen.c into synth/libsynth.so (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + f".{os.getpid()}.tmp"
        subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
                        "-ffp-contract=off", "-Wall", os.path.join(_HERE, "gen.c"), "-lm",
                        "-o", tmp], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _native():
    global _lib
    with _lock:
        if _lib is None:
            L = ctypes.CDLL(build())
            L.syn_words.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64,
                                    ctypes.c_int64, ctypes.c_void_p]
            L.syn_normal.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64,
                                     ctypes.c_int64, ctypes.c_double, ctypes.c_void_p]
            _lib = L
    return _lib


def words_native(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    """The same words as `words`, from the C build."""
    out = np.empty(count, dtype=np.uint64)
    _native().syn_words(seed, stream, start, count, out.ctypes.data)
    return out


def normal_f16(seed: int, stream: int, shape, sigma: float = 1.0) -> np.ndarray:
    """N(0, sigma^2) samples rounded to binary16, C order, element i uses words 2i, 2i+1."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float16)
    L = _native()
    buf = np.empty(min(n, _CHUNK), dtype=np.float64)
    for lo in range(0, n, _CHUNK):
        m = min(_CHUNK, n - lo)
        L.syn_normal(seed, stream, lo, m, float(sigma), buf.ctypes.data)
        out[lo:lo + m] = buf[:m].astype(np.float16)
    return out.reshape(shape)


def normal_f64_reference(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    """Box-Muller normals (sigma 1) of elements [start, start+count) in numpy."""
    w = words(seed, stream, 2 * start, 2 * count)
    u1 = ((w[0::2] >> np.uint64(11)).astype(np.float64) + 0.5) * (2.0 ** -53)
    u2 = (w[1::2] >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)


def uniform_bits(seed: int, stream: int, count: int) -> np.ndarray:
    """`count` fair bits (uint8 0/1), bit i from word i."""
    return (words(seed, stream, 0, count) >> np.uint64(63)).astype(np.uint8)


def bfs_parents(seed: int, stream: int, q: int) -> np.ndarray:
    """A random tree of q tokens listed in breadth-first order, as a parent array.

    parent[0] = -1 (the root hangs off the prompt prefix); for i >= 2 the parent
    is parent[i-1] or parent[i-1] + 1, picked by one fair bit, and capped at
    i - 1, so parents never decrease (breadth-first order) and always precede
    their children.
    """
    p = np.full(q, -1, dtype=np.int32)
    if q > 1:
        p[1] = 0
    bits = uniform_bits(seed, stream, max(q, 1))
    for i in range(2, q):
        p[i] = min(int(p[i - 1]) + int(bits[i]), i - 1)
    return p


def codes_u8(seed: int, stream: int, count: int) -> np.ndarray:
    """Uniform random bytes (two random 4-bit codes per byte)."""
    return (words(seed, stream, 0, count) >> np.uint64(56)).astype(np.uint8)


# Stream ids, one per tensor of a configuration (seed = 0x5EED0000 + config id).
def seed_for(config_id: int) -> int:
    return 0x5EED0000 + int(config_id)


WEIGHT_NAMES = ("wq", "wk", "wv", "wo", "w1", "w2")


def weight_stream(layer: int, name: str) -> int:
    return 6 * layer + WEIGHT_NAMES.index(name)


STREAM_PREFILL_X = 1_000_000


def stream_decode_t(step: int) -> int:
    return 1_000_000 + 1 + step


def stream_tree_parents(request: int) -> int:
    return 2_000_000 + request


STREAM_TREE_Q, STREAM_TREE_K, STREAM_TREE_V = 3_000_000, 3_000_001, 3_000_002


def stream_layer_input(layer: int) -> int:
    return 4_000_000 + layer


# Per-request streams (full-size parity tests draw only the sampled requests).
_REQUEST_KINDS = {"prompt": 6_000_000, "token": 7_000_000, "cache_k": 8_000_000,
                  "cache_v": 9_000_000, "tree_qkv": 10_000_000}


def stream_request(kind: str, request: int) -> int:
    return _REQUEST_KINDS[kind] + int(request)
