"""The five workload shapes (FlexGen paper notes: OPT layer shapes with prompt
512 and 32 generated tokens; SpecPipe article: 64-token trees) and their
seeded synthetic inputs."""
import numpy as np

import synth

CONFIGS = {
    1: dict(name="tiny", l=2, h1=256, h2=1024, heads=4, b=4, gbs=4, s=32, n=8, w_fmt=1, kv_fmt=1),
    2: dict(name="opt-6.7b-fp16", l=32, h1=4096, h2=16384, heads=32, b=64, gbs=64, s=512, n=32,
            w_fmt=0, kv_fmt=0),
    3: dict(name="opt-30b-int4", l=48, h1=7168, h2=28672, heads=56, b=144, gbs=48, s=512, n=32,
            w_fmt=1, kv_fmt=1),
    4: dict(name="opt-175b-int4", l=96, h1=12288, h2=49152, heads=96, b=144, gbs=48, s=512, n=32,
            w_fmt=1, kv_fmt=1),
    5: dict(name="tree-attention", b=8, h1=8192, heads=64, prefix=2048, q=64, kv_fmt=1),
}


def layer_weights(cid, j, h1, h2, sigma=0.02):
    seed = synth.seed_for(cid)
    shp = {"wq": (h1, h1), "wk": (h1, h1), "wv": (h1, h1), "wo": (h1, h1), "w1": (h1, h2),
           "w2": (h2, h1)}
    return {k: synth.normal_f16(seed, synth.weight_stream(j, k), v, sigma) for k, v in shp.items()}


def oracle_weights(orc, W, fmt):
    """The fp16 values the oracle multiplies by: w itself, or its int4 round trip."""
    if fmt == 0:
        return W
    out = {}
    for k, w in W.items():
        c, s = orc.quantize_g64(w)
        out[k] = orc.dequantize_g64(c, s)
    return out


def prompt(cid, b, s, h1):
    return synth.normal_f16(synth.seed_for(cid), synth.STREAM_PREFILL_X, (b, s, h1))


def decode_inputs(cid, n, b, h1):
    seed = synth.seed_for(cid)
    return np.stack([synth.normal_f16(seed, synth.stream_decode_t(i), (b, h1)) for i in range(n)])
