"""The direct global-to-LDS loads set the m0 register inside inline assembly
(lds_dma.h).  m0 is a reserved register, so the compiler does not model that
write; it is only safe while no compiler-generated instruction in the same
kernels uses m0.  This compiles the sources that use those loads for gfx950
(device code only, the library's own flags) and checks their assembly: every
mention of m0 is one of the helpers' `s_mov_b32 m0, sN` writes, each followed
by the direct load it addresses, and no instruction that reads m0 implicitly
appears."""
import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from decode_step_transformer_amd import build as B

SOURCES = ("attn.hip", "gemm16.hip", "gemm_dec.hip")
# instruction families that read m0 without naming it
IMPLICIT_M0 = re.compile(r"^\s*(s_movrel|v_movrel|s_set_gpr_idx|ds_gws|ds_append|ds_consume|"
                         r"ds_ordered_count|s_sendmsg|v_interp|\S*_addtid|buffer_load\S*\s.*\blds\b)")


def _asm(src, out_dir):
    out = os.path.join(out_dir, src + ".s")
    subprocess.run([B.HIPCC, *B.FLAGS, "--cuda-device-only", "-S", os.path.join(B.CSRC, src),
                    "-o", out], check=True, capture_output=True, timeout=600)
    return out


@pytest.mark.skipif(not os.path.exists(B.HIPCC), reason="hipcc not installed")
def test_m0_written_only_by_direct_load_helpers():
    tmp = tempfile.mkdtemp()
    try:
        with cf.ThreadPoolExecutor(len(SOURCES)) as ex:
            files = list(ex.map(lambda s: _asm(s, tmp), SOURCES))
        for f in files:
            lines = [ln.split(";")[0].rstrip() for ln in open(f)]
            code = [ln for ln in lines if ln.strip() and not ln.strip().startswith(".")
                    and not ln.strip().endswith(":")]
            writes = 0
            for i, ln in enumerate(code):
                assert not IMPLICIT_M0.match(ln), (f, ln)
                if re.search(r"\bm0\b", ln):
                    assert re.fullmatch(r"\s*s_mov_b32 m0, s\d+", ln), (f, ln)
                    nxt = [c.strip() for c in code[i + 1:i + 3]]
                    assert nxt[0] == "s_nop 0" and nxt[1].startswith("global_load_lds"), (f, nxt)
                    writes += 1
            assert writes > 0, f
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
