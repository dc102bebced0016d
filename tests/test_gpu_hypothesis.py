"""Property-based shapes for the training path (fa_fwd + fa_bwd through the C
ABI), against the float64 oracle and inside guard bands.

Hypothesis draws the shape: batch 1-3 of fixed length 1-300 or a packed batch
of 1-4 sequences of length 0-300 (at least one token), 1 or 2 KV heads with
1, 2 or 4 query heads each, d = 64/128/256, fp16 or bf16, causal or not, and
the seed of the N(0, 1) inputs. Every output must meet the parity tolerances
of parity_util on every element, and no guard band may change. The cases are
derandomized (the same 40 every run) so that a failure names a reproducible
shape; the shape is printed before each case runs.
"""
import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import workloads as W
from oracle import attention_bwd, attention_fwd
from parity_util import check_grad, check_lse, check_o, host64, say, to_device
from test_gpu_guard_bands import Guarded

pytestmark = pytest.mark.gpu


@st.composite
def shapes(draw):
    d = draw(st.sampled_from([64, 128, 256]))
    hkv = draw(st.sampled_from([1, 2]))
    hq = hkv * draw(st.sampled_from([1, 2, 4]))
    dtype = draw(st.sampled_from(["fp16", "bf16"]))
    causal = draw(st.booleans())
    seed = draw(st.integers(0, 2 ** 20))
    if draw(st.booleans()):
        lens = draw(st.lists(st.integers(0, 300), min_size=1, max_size=4).filter(lambda l: sum(l) > 0))
        return W.custom(B=0, Hq=hq, Hkv=hkv, N=0, d=d, dtype=dtype, causal=causal, seed=seed,
                        lens=lens, backward=True)
    return W.custom(B=draw(st.integers(1, 3)), Hq=hq, Hkv=hkv, N=draw(st.integers(1, 300)), d=d,
                    dtype=dtype, causal=causal, seed=seed, backward=True)


def _stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


@settings(max_examples=40, deadline=None, derandomize=True, database=None,
          suppress_health_check=list(HealthCheck))
@given(w=shapes())
def test_random_shapes_match_oracle(w):
    import torch
    import exact_io_aware_12_amd as fa
    say(f"[hypothesis] B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} d={w.d} {w.dtype} causal={w.causal} "
        f"lens={w.lens} seed={w.seed}")
    a = W.generate(w, with_grad=True)
    t = to_device(a, w.dtype)
    td = t["q"].dtype
    code = fa.FA_BF16 if w.dtype == "bf16" else fa.FA_FP16
    cu = t["cu_seqlens"].data_ptr() if w.varlen else None
    o = Guarded((w.T, w.Hq, w.d), td)
    lse = Guarded((w.Hq, w.T), torch.float32)
    st_ = fa.fa_fwd(t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(), o.ptr(), lse.ptr(),
                    w.B, w.Hq, w.Hkv, w.N, w.d, float(w.scale), int(w.causal), cu, code, _stream())
    assert st_ == fa.FA_OK, fa.fa_status_string(st_)
    dq = Guarded((w.T, w.Hq, w.d), td)
    dk = Guarded((w.T, w.Hkv, w.d), td)
    dv = Guarded((w.T, w.Hkv, w.d), td)
    nws = fa.fa_bwd_workspace_size(w.B, w.Hq, w.Hkv, w.N, w.d)
    ws = Guarded((max(nws, 1),), torch.uint8)
    st_ = fa.fa_bwd(t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(), o.ptr(),
                    t["do"].data_ptr(), lse.ptr(), dq.ptr(), dk.ptr(), dv.ptr(), w.B, w.Hq, w.Hkv,
                    w.N, w.d, float(w.scale), int(w.causal), cu, code, ws.ptr(), nws, _stream())
    assert st_ == fa.FA_OK, fa.fa_status_string(st_)
    torch.cuda.synchronize()
    for g, n in ((o, "O"), (lse, "LSE"), (dq, "dQ"), (dk, "dK"), (dv, "dV"), (ws, "workspace")):
        g.check(n)
    h = {n: host64(t[n]) for n in ("q", "k", "v", "do")}
    cus = a["cu_seqlens"]   # B+1 offsets, for fixed-length batches too
    o_ref, lse_ref = attention_fwd(h["q"], h["k"], h["v"], w.scale, w.causal, cus)
    check_o(host64(o.body), o_ref, w.dtype)
    check_lse(host64(lse.body), lse_ref)
    g_ref = attention_bwd(h["q"], h["k"], h["v"], h["do"], w.scale, w.causal, cus)
    for g, r, n in zip((dq, dk, dv), g_ref, ("dQ", "dK", "dV")):
        if np.abs(r).max(initial=0.0) > 0:
            check_grad(host64(g.body), r, n)


@st.composite
def masked(draw):
    """A shape plus options for fa_fwd_ex / fa_bwd_ex: a mask (none, causal, or a
    window with each bound unbounded or 0-300 positions) and a soft cap (none or
    1-60)."""
    w = draw(shapes())
    kind = draw(st.sampled_from(["none", "causal", "window"]))
    cap = draw(st.one_of(st.just(0.0), st.floats(1.0, 60.0)))
    bound = st.one_of(st.just(-1), st.integers(0, 300))
    window = (draw(bound), draw(bound)) if kind == "window" else (-1, -1)
    return w, kind, window, cap


@settings(max_examples=30, deadline=None, derandomize=True, database=None,
          suppress_health_check=list(HealthCheck))
@given(case=masked())
def test_random_masks_and_caps_match_oracle(case):
    """The options-struct entry points on drawn shapes, masks and soft caps, against
    the oracle's window and soft-cap arguments, inside guard bands."""
    import ctypes
    import torch
    import exact_io_aware_12_amd as fa
    w, kind, window, cap = case
    mask = {"none": fa.FA_MASK_NONE, "causal": fa.FA_MASK_CAUSAL, "window": fa.FA_MASK_WINDOW}[kind]
    say(f"[hypothesis-ex] B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} d={w.d} {w.dtype} lens={w.lens} "
        f"seed={w.seed} mask={kind} window={window} softcap={cap}")
    opts = fa.attn_options(mask=mask, window=window, softcap=cap)
    a = W.generate(w, with_grad=True)
    t = to_device(a, w.dtype)
    td = t["q"].dtype
    code = fa.FA_BF16 if w.dtype == "bf16" else fa.FA_FP16
    cu = t["cu_seqlens"].data_ptr() if w.varlen else None
    o = Guarded((w.T, w.Hq, w.d), td)
    lse = Guarded((w.Hq, w.T), torch.float32)
    st_ = fa.fa_fwd_ex(t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(), o.ptr(), lse.ptr(),
                       w.B, w.Hq, w.Hkv, w.N, w.d, float(w.scale), ctypes.addressof(opts), cu, code,
                       _stream())
    assert st_ == fa.FA_OK, fa.fa_status_string(st_)
    dq = Guarded((w.T, w.Hq, w.d), td)
    dk = Guarded((w.T, w.Hkv, w.d), td)
    dv = Guarded((w.T, w.Hkv, w.d), td)
    nws = fa.fa_bwd_workspace_size(w.B, w.Hq, w.Hkv, w.N, w.d)
    ws = Guarded((max(nws, 1),), torch.uint8)
    st_ = fa.fa_bwd_ex(t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(), o.ptr(),
                       t["do"].data_ptr(), lse.ptr(), dq.ptr(), dk.ptr(), dv.ptr(), w.B, w.Hq,
                       w.Hkv, w.N, w.d, float(w.scale), ctypes.addressof(opts), cu, code,
                       ws.ptr(), nws, _stream())
    assert st_ == fa.FA_OK, fa.fa_status_string(st_)
    torch.cuda.synchronize()
    for g, n in ((o, "O"), (lse, "LSE"), (dq, "dQ"), (dk, "dK"), (dv, "dV"), (ws, "workspace")):
        g.check(n)
    h = {n: host64(t[n]) for n in ("q", "k", "v", "do")}
    cus = a["cu_seqlens"]
    causal = kind == "causal"
    win = window if kind == "window" else None
    sc = cap if cap else None
    o_ref, lse_ref = attention_fwd(h["q"], h["k"], h["v"], w.scale, causal, cus, window=win,
                                   softcap=sc)
    check_o(host64(o.body), o_ref, w.dtype)
    check_lse(host64(lse.body), lse_ref)
    g_ref = attention_bwd(h["q"], h["k"], h["v"], h["do"], w.scale, causal, cus, window=win,
                          softcap=sc)
    for g, r, n in zip((dq, dk, dv), g_ref, ("dQ", "dK", "dV")):
        if np.abs(r).max(initial=0.0) > 0:
            check_grad(host64(g.body), r, n)
