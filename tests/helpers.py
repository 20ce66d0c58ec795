"""Shared test helpers: device transfer, the parity tolerance, layout readers."""
import numpy as np

TOL = 2e-2  # |gpu - ref| <= TOL * max(1, |ref|) per element


def dev(a):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.float16).cuda()
    return torch.from_numpy(a.copy()).cuda()


def host(t):
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float16:
        return t.view(torch.int16).numpy().view(np.float16)
    if t.dtype == torch.int16:
        return t.numpy().view(np.uint16)
    return t.numpy()


def assert_close(gpu, ref, tol=TOL, what=""):
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite GPU values"
    err = np.abs(g - r) / np.maximum(1.0, np.abs(r))
    worst = np.unravel_index(np.argmax(err), err.shape) if err.size else None
    assert err.size == 0 or err.max() <= tol, \
        f"{what}: max rel err {err.max():.3g} at {worst}: gpu {g[worst]} ref {r[worst]}"
    return float(err.max()) if err.size else 0.0


def unpack_nibbles(codes):
    """Generic layout bytes -> codes (byte j holds c[2j] | c[2j+1] << 4)."""
    lo = codes & 15
    hi = codes >> 4
    return np.stack([lo, hi], -1).reshape(codes.shape[:-1] + (codes.shape[-1] * 2,))


def unpack_q4_weight(packed, k, n):
    """The packed GEMM layout of include/hp.h -> codes c[k][n]."""
    t = packed.reshape(n // 16, k // 128, 64, 4, 4)          # nb, kb, lane, dword j, byte
    words = t.astype(np.uint32)
    words = words[..., 0] | (words[..., 1] << 8) | (words[..., 2] << 16) | (words[..., 3] << 24)
    nib = np.stack([(words >> (4 * p)) & 15 for p in range(8)], -1)  # nb, kb, lane, j, nibble
    order = [0, 4, 1, 5, 2, 6, 3, 7]   # k-offset e sits in nibble e/2 (even) or 4 + e/2 (odd)
    e_vals = nib[..., order]                                  # nb, kb, lane, j, e
    lane = np.arange(64)
    c = np.zeros((k, n), np.uint8)
    for nb in range(n // 16):
        for kb in range(k // 128):
            blk = e_vals[nb, kb]                              # lane, j, e
            cols = 16 * nb + (lane % 16)
            for j in range(4):
                for e in range(8):
                    kk = 128 * kb + 32 * (lane // 16) + 8 * j + e
                    c[kk, cols] = blk[:, j, e]
    return c


def unpack_f16_weight(packed, k, n):
    """The fragment-major HP_F16 layout of include/hp.h -> w[k][n] (uint16 bits)."""
    t = packed.reshape(k // 128, n // 16, 4, 64, 8)            # kb, nb, j, lane, e
    w = np.zeros((k, n), np.uint16)
    lane = np.arange(64)
    for kb in range(k // 128):
        for nb in range(n // 16):
            cols = 16 * nb + (lane % 16)
            for j in range(4):
                for e in range(8):
                    w[128 * kb + 32 * j + 8 * (lane // 16) + e, cols] = t[kb, nb, j, :, e]
    return w


def check_flips(g_codes, r_codes, what, max_rate):
    """int4 cache rows that the two sides coded from K/V each computed itself (sums in
    different orders): reports the share of differing 4-bit codes (the flip rate),
    requires every code within one level and the rate at most max_rate.  Codes coded
    from the same fp16 rows are compared bit-exactly elsewhere."""
    gc = unpack_nibbles(np.asarray(g_codes)).astype(np.int32)
    rc = unpack_nibbles(np.asarray(r_codes)).astype(np.int32)
    rate = float((gc != rc).mean())
    print(f"{what}: code flip rate {rate:.3g}")
    assert np.abs(gc - rc).max() <= 1, f"{what}: a code differs by more than one level"
    assert rate <= max_rate, f"{what}: flip rate {rate:.3g} > {max_rate}"
    return rate
