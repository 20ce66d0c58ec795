"""No kernel of the library spills registers to scratch memory.

Every kernel is sized to its register budget (the hot ones to two or three
waves per SIMD); a spill would turn register traffic into memory traffic in
the inner loops.  This compiles every HIP source for gfx950 (device code only,
the library's own flags) and checks the compiler's report for each function:
`ScratchSize: 0`."""
import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from decode_step_transformer_amd import build as B


def _asm(src, out_dir):
    out = os.path.join(out_dir, src + ".s")
    subprocess.run([B.HIPCC, *B.FLAGS, "--cuda-device-only", "-S", os.path.join(B.CSRC, src),
                    "-o", out], check=True, capture_output=True, timeout=900)
    return src, out


@pytest.mark.skipif(not os.path.exists(B.HIPCC), reason="hipcc not installed")
def test_no_kernel_spills():
    tmp = tempfile.mkdtemp()
    try:
        with cf.ThreadPoolExecutor(min(8, len(B.SOURCES))) as ex:
            files = list(ex.map(lambda s: _asm(s, tmp), B.SOURCES))
        spills, seen = [], 0
        for src, path in files:
            name = None
            for ln in open(path):
                m = re.match(r"^(_Z\S+):", ln)
                if m:
                    name = m.group(1)
                if "; ScratchSize:" in ln:
                    seen += 1
                    if int(ln.split(":")[1]) != 0:
                        spills.append((src, name))
        assert seen >= len(B.SOURCES), "no resource reports found"
        assert not spills, f"functions with scratch (spilled registers): {spills}"
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
