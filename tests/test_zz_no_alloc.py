"""fa_bwd_noalloc (the backward with its workspace in the library's fixed
device array) against fa_bwd with a caller-owned workspace, through the C ABI:
two calls in a row, the second smaller, each bitwise equal to fa_bwd and
within the gradient tolerance of the float64 oracle."""
import numpy as np
import pytest

import workloads as W
from oracle import attention_bwd
from parity_util import bits_equal, check_grad, host64, say, to_device

pytestmark = pytest.mark.gpu

CASES = [
    dict(B=2, Hq=4, Hkv=2, N=300, d=128, dtype="bf16", causal=True, seed=61),
    dict(B=0, Hq=2, Hkv=1, N=0, d=64, dtype="fp16", causal=False, seed=62, lens=[40, 0, 77]),
]


def _run(case):
    import torch
    import exact_io_aware_12_amd as fa
    w = W.custom(backward=True, **case)
    a = W.generate(w, with_grad=True)
    t = to_device(a, w.dtype)
    cu = t["cu_seqlens"] if w.varlen else None
    say(f"[fa_bwd_noalloc] B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} d={w.d} {w.dtype} "
        f"causal={w.causal} varlen={w.varlen} T={w.T}")
    kw = dict(causal=w.causal, softmax_scale=w.scale)
    if w.varlen:
        kw.update(cu_seqlens=cu, max_seqlen=w.N)
    o, lse = fa.flash_attn_func(t["q"], t["k"], t["v"], **kw) if w.varlen else \
        fa.flash_attn_func(*(t[n].view(w.B, w.N, -1, w.d) for n in ("q", "k", "v")), **kw)
    o = o.reshape(w.T, w.Hq, w.d)
    code = fa.FA_BF16 if w.dtype == "bf16" else fa.FA_FP16
    stream = torch.cuda.current_stream().cuda_stream
    outs = []
    for entry in ("fa_bwd", "fa_bwd_noalloc"):
        dq, dk, dv = (torch.full_like(t[n], float("nan")) for n in ("q", "k", "v"))
        ptrs = [t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(), o.data_ptr(),
                t["do"].data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr()]
        sizes = [w.B, w.Hq, w.Hkv, w.N, w.d, float(w.scale), int(w.causal),
                 cu.data_ptr() if cu is not None else None, code]
        if entry == "fa_bwd":
            nws = fa.fa_bwd_workspace_size(w.B, w.Hq, w.Hkv, w.N, w.d)
            ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
            st = fa.fa_bwd(*ptrs, *sizes, ws.data_ptr(), nws, stream)
        else:
            st = fa.fa_bwd_noalloc(*ptrs, *sizes, stream)
        assert st == fa.FA_OK, fa.fa_status_string(st)
        torch.cuda.synchronize()
        outs.append((dq, dk, dv))
    for x, y, n in zip(*outs, ("dQ", "dK", "dV")):
        assert bits_equal(x, y), f"{n}: fa_bwd_noalloc differs from fa_bwd"
    ref = attention_bwd(host64(t["q"]), host64(t["k"]), host64(t["v"]), host64(t["do"]),
                        w.scale, w.causal, t["cu_seqlens"].cpu().numpy())
    for g, r, n in zip(outs[1], ref, ("dQ", "dK", "dV")):
        check_grad(host64(g), r, n)
    return outs[1]


def test_noalloc_matches_fa_bwd_twice_second_smaller():
    first = _run(CASES[0])
    second = _run(CASES[1])
    assert second[0].numel() < first[0].numel()


def test_noalloc_rejects_what_the_scratch_cannot_hold():
    import exact_io_aware_12_amd as fa
    P = 0x1000
    st = fa.fa_bwd_noalloc(*([P] * 9), 4, 64, 8, 65536, 128, 0.088, 1, None, fa.FA_BF16, None)
    assert st == fa.FA_ERR_WORKSPACE
