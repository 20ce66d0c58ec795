"""The allocation-free product hp_gemm_noalloc against hp_gemm, through the C ABI.

hp_gemm_noalloc runs the same kernels with the split-k partial sums in the
library's static device scratch instead of a caller workspace, so its output
must equal hp_gemm's bit for bit.  Two calls in a row share the scratch; the
second is smaller than the first, so stale partials of the first call would
show if the second read any entry it did not write.
"""
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hp():
    import torch
    from decode_step_transformer_amd import hp as _hp
    assert torch.cuda.is_available()
    assert _hp.hp_device_check() == 0, _hp.hp_last_error()
    return _hp


def _weight(hp, k, n, fmt, seed):
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    w = (torch.randn((k, n), generator=g, device="cuda") * 0.02).half()
    return hp.make_weight(w, fmt)


def _inputs(M, k, n, seed):
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    x = torch.randn((M, k), generator=g, device="cuda").half()
    r = torch.randn((M, n), generator=g, device="cuda").half()
    return x, r


@pytest.mark.parametrize("fmt", [1, 0])
def test_noalloc_equals_gemm_two_calls(hp, fmt):
    import torch
    # first: the OPT-30B QKV decode product (M = 144, k = 7168, n = 21504, 3 splits);
    # second: a smaller product (M = 37, k = 1024, n = 768) on the same scratch
    for M, k, n, relu, use_res, seed in ((144, 7168, 21504, False, False, 1),
                                         (37, 1024, 768, True, True, 2)):
        w = _weight(hp, k, n, fmt, seed)
        x, r = _inputs(M, k, n, seed + 10)
        res = r if use_res else None
        assert hp.hp_gemm_workspace_bytes(M, k, n, fmt) > 0  # split k: the scratch is used
        ref = hp.hp_gemm(x, w, res=res, relu=relu)
        got = hp.hp_gemm_noalloc(x, w, res=res, relu=relu)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), (M, k, n, fmt)
        assert bool(torch.isfinite(got.float()).all())


def test_noalloc_rejects_tall(hp):
    from decode_step_transformer_amd.hp import HPError
    w = _weight(hp, 256, 512, 1, 3)
    x, _ = _inputs(145, 256, 512, 4)
    with pytest.raises(HPError) as e:
        hp.hp_gemm_noalloc(x, w)
    assert e.value.status == -2
