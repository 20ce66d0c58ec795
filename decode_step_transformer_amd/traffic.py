"""HBM traffic of a kernel from rocprofv3 counters, calibrated on a plain copy.

rocprofv3 reports FETCH_SIZE and WRITE_SIZE (KiB per dispatch, summed over the
L2 channels).  A copy of a known number of bytes reads and writes exactly that
many bytes of HBM, so the ratio of known bytes to the counter's value on the
copy is the counter's scale on this GPU; a kernel's traffic is its counter
value times that scale.  Each counter is collected in its own run.

Commands (from the repository root; results under gpurun_out/):

  rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/tr_copy_f -o run \\
      -- python3 decode_step_transformer_amd/traffic.py copy
  rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/tr_copy_w -o run \\
      -- python3 decode_step_transformer_amd/traffic.py copy
  rocprofv3 --pmc FETCH_SIZE --kernel-include-regex k_gemm16 --output-format csv \\
      -d gpurun_out/tr_k_f -o run \\
      -- python3 decode_step_transformer_amd/traffic.py prefill opt-30b-int4
  rocprofv3 --pmc WRITE_SIZE ... (the same with -d gpurun_out/tr_k_w)
  python3 -m decode_step_transformer_amd.traffic summarize k_gemm16 opt-30b-int4 \\
      gpurun_out/tr_copy_f gpurun_out/tr_copy_w gpurun_out/tr_k_f gpurun_out/tr_k_w

`prefill` runs one layer prefill of a bench.py configuration eagerly: the
block's prefill column issues one such call per layer (all GPU batches in one
launch), so its GEMM launches have the block's shapes.  `decode` runs one
layer decode the same way, at the cache length where bench.py times the
decode kernels (the decode GEMM and attention; select them with
--kernel-include-regex 'k_gemm_dq|k_decode_attn').  `topk` runs Top-K sparse
attention at the same cache length (k_topk_attn).  `tree` runs the
tree-masked decode attention workload (k_multi_attn) and `quant` the int4
quantiser on a weight of the 175B w1 shape (k_quantize_g64); `prefill` also
covers the KV append at the prefill shape (k_kv_append).

`summarize` writes profiles/traffic.json: per kernel, the calibrated bytes
read and written per dispatch and a hash of the sources that define the
kernel; bench.py reports the figure only while that hash still matches.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
OUT = os.path.join(ROOT, "profiles", "traffic.json")
COPY_BYTES = 1 << 30

# sources that define each measured kernel (the figure is void once they change)
KERNEL_SOURCES = {
    "k_gemm16": ["csrc/gemm16.hip", "csrc/lds_dma.h", "csrc/common.h"],
    "k_gemm_dq": ["csrc/gemm_dec.hip", "csrc/lds_dma.h", "csrc/dequant_dev.h", "csrc/common.h"],
    "k_gemm<": ["csrc/gemm.hip", "csrc/common.h"],  # the fp16 skinny product
    "k_decode_attn": ["csrc/attn.hip", "csrc/decode_dev.h", "csrc/dequant_dev.h", "csrc/common.h"],
    "k_topk_attn": ["csrc/topk.hip", "csrc/decode_dev.h", "csrc/dequant_dev.h", "csrc/common.h"],
    "k_multi_attn": ["csrc/attn.hip", "csrc/lds_dma.h", "csrc/decode_dev.h", "csrc/dequant_dev.h",
                     "csrc/common.h"],
    "k_kv_append": ["csrc/attn.hip", "csrc/quant_dev.h", "csrc/common.h"],
    "k_quantize_g64": ["csrc/quant.hip", "csrc/quant_dev.h", "csrc/common.h"],
}


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(HERE, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def copy() -> None:
    """A plain device copy of COPY_BYTES bytes (the calibration kernel)."""
    import torch

    src = torch.ones(COPY_BYTES // 2, dtype=torch.float16, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print("copied", COPY_BYTES, "bytes", flush=True)


def _one_layer(config: str, cap_extra: int):
    import torch

    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    from bench import CONFIGS
    from decode_step_transformer_amd import hp

    c = CONFIGS[config]
    h1, h2, heads, b, s = c["h1"], c["h2"], c["heads"], c["b"], c["s"]
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    W = {name: (torch.randn(shp, generator=g, device="cuda") * 0.02).half()
         for name, shp in (("wq", (h1, h1)), ("wk", (h1, h1)), ("wv", (h1, h1)),
                           ("wo", (h1, h1)), ("w1", (h1, h2)), ("w2", (h2, h1)))}
    layer = hp.make_layer(W, c["fmt"])
    del W
    x = (torch.randn((b, s, h1), generator=g, device="cuda")).half()
    kv = hp.KVCache(c["fmt"], b, heads, s + cap_extra, h1 // heads)
    d = hp.dims(b, s, max(cap_extra, 1), h1, h2, 1, heads, c["gbs"])
    ws = torch.empty(hp.hp_workspace_bytes(d), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(x)
    torch.cuda.synchronize()
    return hp, c, d, layer, x, kv, ws, out


def prefill(config: str, calls: int = 2) -> None:
    """`calls` eager hp_layer_prefill calls at the shapes of a bench.py configuration."""
    import torch

    hp, c, d, layer, x, kv, ws, out = _one_layer(config, 0)
    for i in range(calls):
        hp.hp_layer_prefill(d, layer, x, kv, out, ws)
        torch.cuda.synchronize()
        print(f"prefill call {i} done", flush=True)


def decode(config: str, calls: int = 2) -> None:
    """One prefill, then `calls` eager hp_layer_decode calls at cache length
    s + n/2 (the decode-kernel timing point of bench.py)."""
    import torch

    n = _config_n(config)
    hp, c, d, layer, x, kv, ws, out = _one_layer(config, n)
    hp.hp_layer_prefill(d, layer, x, kv, out, ws)
    t = x[:, -1].contiguous()
    t_out = torch.empty_like(t)
    pos = c["s"] + n // 2 - 1
    for i in range(calls):
        hp.hp_layer_decode(d, layer, t, pos, 1, kv, t_out, ws)
        torch.cuda.synchronize()
        print(f"decode call {i} done", flush=True)


def topk(config: str, calls: int = 2) -> None:
    """One prefill, then `calls` eager Top-K sparse attention calls at cache length
    s + n/2 (the sparse_attention timing point of bench.py)."""
    import torch

    n = _config_n(config)
    hp, c, d, layer, x, kv, ws, out = _one_layer(config, n)
    hp.hp_layer_prefill(d, layer, x, kv, out, ws)
    qkv = torch.randn((c["b"], 3 * c["h1"]), device="cuda").half()
    pos = c["s"] + n // 2 - 1
    for i in range(calls):
        hp.hp_topk_attention(c["b"], c["h1"], c["heads"], qkv, pos, kv)
        torch.cuda.synchronize()
        print(f"topk call {i} done", flush=True)


def tree(calls: int = 3) -> None:
    """The tree-masked decode attention workload of bench.py (8 requests, h1 = 8192,
    64 heads, 2048-row int4 prefix, 64 tree tokens with random BFS parents):
    `calls` hp_decode_attention calls (k_multi_attn)."""
    import torch

    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    from bench import TREE
    from decode_step_transformer_amd import hp

    b, h1, H, P, q = TREE["b"], TREE["h1"], TREE["heads"], TREE["prefix"], TREE["q"]
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    sig = 0.02 * h1 ** 0.5
    kv = hp.KVCache(1, b, H, P + q, h1 // H)
    pre = (torch.randn((b, P, 3 * h1), generator=g, device="cuda") * sig).half()
    hp.hp_kv_append(b, P, h1, H, pre, 0, kv)
    del pre
    qkv = (torch.randn((b, q, 3 * h1), generator=g, device="cuda") * sig).half()
    hp.hp_kv_append(b, q, h1, H, qkv, P, kv)
    parent = torch.arange(-1, q - 1, dtype=torch.int32).repeat(b, 1)
    parent[:, 1:] = torch.div(torch.arange(0, q - 1), 2, rounding_mode="floor").to(torch.int32)
    masks, _ = hp.hp_tree_masks(parent.cuda())
    for i in range(calls):
        hp.hp_decode_attention(b, q, h1, H, qkv, P, kv, masks=masks)
        torch.cuda.synchronize()
        print(f"tree call {i} done", flush=True)


def quant(calls: int = 3) -> None:
    """hp_quantize_g64 on an fp16 weight of the 175B w1 shape (12288 x 49152)."""
    import torch

    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    from decode_step_transformer_amd import hp

    g = torch.Generator(device="cuda")
    g.manual_seed(23)
    w = (torch.randn((12288, 49152), generator=g, device="cuda") * 0.02).half()
    torch.cuda.synchronize()
    for i in range(calls):
        hp.hp_quantize_g64(w)
        torch.cuda.synchronize()
        print(f"quantize call {i} done", flush=True)


def _config_n(config: str) -> int:
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    from bench import CONFIGS
    return CONFIGS[config]["n"]


def _per_dispatch(d: str, counter: str, name_part: str) -> list:
    """Counter values (KiB) of the dispatches whose kernel name contains name_part."""
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    vals = {}
    for row in csv.DictReader(open(files[0])):
        if row["Counter_Name"] != counter or name_part not in row["Kernel_Name"]:
            continue
        key = row.get("Dispatch_Id") or row.get("Correlation_Id") or str(len(vals))
        vals[key] = vals.get(key, 0.0) + float(row["Counter_Value"])
    return list(vals.values())


def summarize(kernel: str, workload: str, copy_f: str, copy_w: str, k_f: str,
              k_w: str) -> dict:
    cf = _per_dispatch(copy_f, "FETCH_SIZE", "copy")
    cw = _per_dispatch(copy_w, "WRITE_SIZE", "copy")
    # the largest copy dispatch is the calibration copy (torch may launch smaller ones)
    scale_f = COPY_BYTES / (max(cf) * 1024.0)
    scale_w = COPY_BYTES / (max(cw) * 1024.0)
    kf = _per_dispatch(k_f, "FETCH_SIZE", kernel)
    kw = _per_dispatch(k_w, "WRITE_SIZE", kernel)
    rec = {
        "fetch_bytes_per_dispatch": sum(kf) / len(kf) * 1024.0 * scale_f,
        "write_bytes_per_dispatch": sum(kw) / len(kw) * 1024.0 * scale_w,
        "dispatches": [len(kf), len(kw)],
        "calibration": {"copy_bytes": COPY_BYTES, "fetch_KiB": max(cf), "write_KiB": max(cw),
                        "fetch_scale": scale_f, "write_scale": scale_w},
        "source_hash": source_hash(kernel),
    }
    data = json.load(open(OUT)) if os.path.exists(OUT) else {}
    data[f"{kernel}@{workload}"] = rec
    with open(OUT, "w") as f:
        json.dump(data, f, indent=1)
    return rec


def lookup(kernel: str, workload: str):
    """Calibrated traffic (bytes per dispatch) of `kernel` in the bench.py configuration
    `workload`, if measured on the current sources, else None."""
    if not os.path.exists(OUT) or kernel not in KERNEL_SOURCES:
        return None
    rec = json.load(open(OUT)).get(f"{kernel}@{workload}")
    if not rec or rec.get("source_hash") != source_hash(kernel):
        return None
    return rec["fetch_bytes_per_dispatch"] + rec["write_bytes_per_dispatch"]


if __name__ == "__main__":
    if len(sys.argv) >= 2 and sys.argv[1] == "copy":
        copy()
    elif len(sys.argv) == 3 and sys.argv[1] == "prefill":
        prefill(sys.argv[2])
    elif len(sys.argv) == 3 and sys.argv[1] == "decode":
        decode(sys.argv[2])
    elif len(sys.argv) == 3 and sys.argv[1] == "topk":
        topk(sys.argv[2])
    elif len(sys.argv) == 2 and sys.argv[1] == "tree":
        tree()
    elif len(sys.argv) == 2 and sys.argv[1] == "quant":
        quant()
    elif len(sys.argv) == 8 and sys.argv[1] == "summarize":
        print(json.dumps(summarize(*sys.argv[2:8]), indent=1))
    else:
        raise SystemExit(__doc__)
