"""The binding's packed-batch checks on GPU tensors: each bad cu_seqlens is
refused with a Python exception before anything is launched."""
import pytest

pytestmark = pytest.mark.gpu


def _packed(T=10, Hq=2, Hkv=1, d=64):
    import torch
    q = torch.randn(T, Hq, d, device="cuda").to(torch.bfloat16)
    k = torch.randn(T, Hkv, d, device="cuda").to(torch.bfloat16)
    return q, k, k.clone()


@pytest.mark.parametrize("case", ["int64", "short_total", "long_total", "too_long", "decreasing",
                                  "nonzero_start"])
def test_bad_cu_seqlens_refused(case):
    import torch
    import exact_io_aware_12_amd as fa
    q, k, v = _packed()
    cu, mx, dt = [0, 4, 10], 6, torch.int32
    if case == "int64":
        dt = torch.int64
    elif case == "short_total":
        cu = [0, 4, 9]
    elif case == "long_total":
        cu = [0, 4, 11]
    elif case == "too_long":
        mx = 5
    elif case == "decreasing":
        cu = [0, 6, 4, 10]
    elif case == "nonzero_start":
        cu = [1, 4, 10]
    c = torch.tensor(cu, dtype=dt, device="cuda")
    with pytest.raises((TypeError, ValueError)):
        fa.flash_attn_func(q, k, v, causal=True, cu_seqlens=c, max_seqlen=mx)
    # the backward checks the same way (o, lse, dout shaped for T = 10)
    good = torch.tensor([0, 4, 10], dtype=torch.int32, device="cuda")
    o, lse = fa.flash_attn_func(q, k, v, causal=True, cu_seqlens=good, max_seqlen=6)
    with pytest.raises((TypeError, ValueError)):
        fa.flash_attn_backward(o, q, k, v, o, lse, causal=True, cu_seqlens=c, max_seqlen=mx)
    torch.cuda.synchronize()


def test_validate_false_skips_the_readback():
    """validate=False trusts the caller: a consistent batch gives the same bits."""
    import torch
    import exact_io_aware_12_amd as fa
    from parity_util import bits_equal
    q, k, v = _packed()
    c = torch.tensor([0, 4, 10], dtype=torch.int32, device="cuda")
    o1, l1 = fa.flash_attn_func(q, k, v, causal=True, cu_seqlens=c, max_seqlen=6)
    o2, l2 = fa.flash_attn_func(q, k, v, causal=True, cu_seqlens=c, max_seqlen=6, validate=False)
    torch.cuda.synchronize()
    assert bits_equal(o1, o2) and bits_equal(l1, l2)
