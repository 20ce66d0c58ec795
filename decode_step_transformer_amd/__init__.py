"""MI355X (gfx950) hot path of the FlexGen OPT-style layer with int4 compression.

The computation lives in libhp.so (HIP kernels behind the C ABI of
include/hp.h); `decode_step_transformer_amd.hp` is its ctypes binding.
"""
from . import hp  # noqa: F401
