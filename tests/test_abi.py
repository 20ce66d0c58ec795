"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point declared in include/hp.h, and its size helpers reproduce
the closed forms printed in the FlexGen paper notes (background section)."""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "hp.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(hp_[a-z0-9_]+)\s*\(", src)))


def test_header_matches_exports():
    from decode_step_transformer_amd import hp
    names = _declared()
    assert names, "no declarations found"
    assert sorted(hp.EXPORTS) == names
    L = hp.lib()
    for n in names:
        assert hasattr(L, n), n


def test_flexgen_size_closed_forms():
    from decode_step_transformer_amd import hp
    g = {}
    for ln in open(os.path.join(ROOT, "tests", "golden", "flexgen_sizes.txt")):
        if ln.startswith("#") or ":" not in ln:
            continue
        k, v = ln.split(":")
        g[k.strip()] = float(v)
    d = hp.dims(int(g["b"]), int(g["s"]), int(g["n"]), int(g["h1"]), int(g["h2"]), int(g["l"]), 96)
    w = hp.hp_weight_bytes(d, hp.HP_F16)
    kv = hp.hp_kv_bytes(d, hp.HP_F16)
    assert round(w / 1e9) == pytest.approx(g["weights_GB_printed"], abs=25)  # 347.9e9 B = 324 GiB
    assert round(w / 2 ** 30) == g["weights_GB_printed"] - 1
    assert round(kv / 2 ** 40, 1) == g["kv_TB_printed"]
    assert round(kv / w, 1) == g["ratio_printed"]
    # int4 group-64 packing: 4 bits per element plus 2 x fp16 per 64 elements
    elems = w // 2
    assert hp.hp_weight_bytes(d, hp.HP_Q4) == elems // 2 + elems // 64 * 4


def test_argument_errors_before_device():
    """Shape errors are reported on the host before any device work."""
    from decode_step_transformer_amd import hp
    L = hp.lib()
    assert L.hp_quantize_g64(None, 4, 100, None, None, None) == -2      # cols % 64
    assert L.hp_tree_masks(1, 65, None, None, None, None) == -4         # q > 64
    d = hp.dims(4, 32, 8, 256, 1024, 2, 3)                              # 256 % 3 != 0
    assert hp.hp_workspace_bytes(d) == 0
    d = hp.dims(4, 32, 8, 256, 1024, 2, 4, 3)                           # b % gbs != 0
    assert hp.hp_workspace_bytes(d) == 0
    d = hp.dims(4, 32, 8, 256, 1024, 2, 4)
    assert hp.hp_workspace_bytes(d) > 0


def test_gemm_host_checks():
    """hp_gemm on the host: a product with no rows is a no-op that touches no
    memory (the pointers below are never dereferenced), negative M and bad
    weight shapes are rejected, all before any device call."""
    import ctypes as C
    from decode_step_transformer_amd import hp
    L = hp.lib()
    fake = 0x100000  # aligned, never dereferenced
    m = hp.hp_mat(hp.HP_Q4, 256, 512, fake, fake, fake)
    assert L.hp_gemm(None, 256, C.byref(m), 0, None, 0, 0, None, 512, None, 0, None) == 0
    assert L.hp_gemm(None, 256, C.byref(m), -1, None, 0, 0, None, 512, None, 0, None) == -2
    bad = hp.hp_mat(hp.HP_Q4, 200, 512, fake, fake, fake)               # k % 128 != 0
    assert L.hp_gemm(None, 200, C.byref(bad), 4, None, 0, 0, None, 512, None, 0, None) == -2
    nul = hp.hp_mat(hp.HP_Q4, 256, 512, fake, None, fake)               # no scales
    assert L.hp_gemm(None, 256, C.byref(nul), 4, None, 0, 0, None, 512, None, 0, None) == -1
    assert L.hp_gemm(None, 256, None, 4, None, 0, 0, None, 512, None, 0, None) == -1


def test_gemm_noalloc_host_checks():
    """hp_gemm_noalloc refuses, on the host and before any device call, a product
    taller than the skinny limit (M > 144 needs a weight-sized buffer) and one whose
    split partials exceed its 64 MiB static scratch (k = 49152, n = 24576 at M = 144
    needs 67.5 MiB); M = 0 is a no-op.  The pointers are never dereferenced."""
    import ctypes as C
    from decode_step_transformer_amd import hp
    L = hp.lib()
    fake = 0x100000
    m = hp.hp_mat(hp.HP_Q4, 256, 512, fake, fake, fake)
    assert L.hp_gemm_noalloc(None, 256, C.byref(m), 0, None, 0, 0, None, 512, None) == 0
    assert L.hp_gemm_noalloc(fake, 256, C.byref(m), 145, None, 0, 0, fake, 512, None) == -2
    assert "M <= 144" in hp.hp_last_error()
    big = hp.hp_mat(hp.HP_Q4, 49152, 24576, fake, fake, fake)
    assert hp.hp_gemm_workspace_bytes(144, 49152, 24576, hp.HP_Q4) > 64 << 20
    assert L.hp_gemm_noalloc(fake, 49152, C.byref(big), 144, None, 0, 0, fake, 24576, None) == -5
    assert "static scratch" in hp.hp_last_error()


def _diag_pages_closed_form(b, s, n, gbs, pr):
    """Pages in use at the busiest iteration of the diagonal schedule, counted directly:
    at iteration it, GPU batch it (if any) holds its prompt rows and every batch k in
    [it - n, it - 1] holds s + (it - k) rows, each request ceil(rows / pr) pages."""
    nb = b // gbs
    best = 0
    for it in range(nb + n):
        live = [s] if it < nb else []
        live += [s + it - k for k in range(max(0, it - n), min(it - 1, nb - 1) + 1)]
        best = max(best, gbs * sum(-(-rows // pr) for rows in live))
    return best


def test_diagonal_pages():
    """[FlexGen] appendix A.2: the diagonal schedule's peak cache, in pages, from the
    library's page plan equals a direct count over the iterations; with n >> s it
    approaches half of what the same live requests hold at full length s + n (the
    page's (2s + n) / 2 against s + n)."""
    from decode_step_transformer_amd import hp
    for b, s, n, gbs, pr in ((12, 20, 7, 3, 64), (150, 16, 128, 1, 64), (144, 512, 32, 48, 64),
                             (40, 100, 300, 2, 128), (512, 32, 480, 1, 64)):
        d = hp.dims(b, s, n, 256, 512, 2, 4, gbs)
        assert hp.hp_diagonal_pages(d, pr) == _diag_pages_closed_form(b, s, n, gbs, pr), (b, s, n)
    d = hp.dims(12, 20, 7, 256, 512, 2, 4, 3)
    assert hp.hp_diagonal_pages(d, 192) == 0 and hp.hp_diagonal_pages(d, 32) == 0  # not a power of two >= 64
    d = hp.dims(512, 32, 480, 256, 512, 2, 4, 1)
    live = 481                                         # n + 1 requests in steady state
    full = live * (32 + 480)                           # their rows at full length
    paged = hp.hp_diagonal_pages(d, 64) * 64
    assert 0.5 < paged / full < 0.6
    assert hp.hp_diagonal_pages(d, 48) == 0            # page rows must be a multiple of 64


def test_peak_probes_reject_bad_arguments_on_the_host():
    """The measurement probes check their arguments before any launch."""
    import ctypes as C
    from decode_step_transformer_amd import hp
    L = hp.lib()
    assert L.hp_peak_read(None, 1024, 8, C.c_void_p(16), None) == -1
    assert L.hp_peak_read(C.c_void_p(16), 1000, 8, C.c_void_p(16), None) == -2  # bytes % 16
    assert L.hp_peak_read(C.c_void_p(8), 1024, 8, C.c_void_p(16), None) == -2   # x % 16
    assert L.hp_peak_read(C.c_void_p(16), 1024, 0, C.c_void_p(16), None) == -2
    assert L.hp_peak_mfma(10, 8, None, None) == -1
    assert L.hp_peak_mfma(0, 8, C.c_void_p(16), None) == -2
