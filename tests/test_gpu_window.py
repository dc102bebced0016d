"""GPU parity of the sliding-window (band) entry points against the oracle.

fa_fwd_window / fa_bwd_window (through the binding's window_size) on small
shapes that span several tiles on both sides of the band, ragged ends, GQA and
varlen, compared element by element with the float64 oracle's band mask; the
two bands that select the plain kernels are checked bit for bit against
fa_fwd / fa_bwd.
"""
import numpy as np
import pytest

import workloads as W
from oracle import attention_bwd, attention_fwd
from parity_util import bits_equal, check_grad, check_lse, check_o, host64, say, to_device

pytestmark = pytest.mark.gpu

WINDOWS = [(0, 0), (1, 0), (5, 3), (64, 0), (63, 65), (127, -1), (-1, 37), (200, 0), (300, 300)]


def _fa():
    import exact_io_aware_12_amd as fa   # raises if libfa.so is missing: no fallback
    return fa


def _views(w, t):
    if w.varlen:
        return t["q"], t["k"], t["v"], dict(cu_seqlens=t["cu_seqlens"], max_seqlen=w.N)
    shp = (w.B, w.N)
    return (t["q"].view(*shp, w.Hq, w.d), t["k"].view(*shp, w.Hkv, w.d),
            t["v"].view(*shp, w.Hkv, w.d), {})


def run_fwd(w, window, arrays=None):
    import torch
    fa = _fa()
    arrays = W.generate(w, with_grad=False) if arrays is None else arrays
    t = to_device(arrays, w.dtype)
    say(f"[fa_fwd_window] {window} B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} d={w.d} {w.dtype} "
        f"causal={w.causal} varlen={w.varlen}")
    q, k, v, kw = _views(w, t)
    o, lse = fa.flash_attn_func(q, k, v, causal=w.causal, softmax_scale=w.scale,
                                window_size=window, **kw)
    torch.cuda.synchronize()
    return o.reshape(w.T, w.Hq, w.d), lse, t


def _oracle_window(w, window):
    wl, wr = window
    if w.causal:
        wr = 0 if wr < 0 else min(wr, 0)
    return (wl, wr)


def compare_fwd(w, window, arrays=None):
    o, lse, t = run_fwd(w, window, arrays)
    cu = t["cu_seqlens"].cpu().numpy()
    o_ref, lse_ref = attention_fwd(host64(t["q"]), host64(t["k"]), host64(t["v"]), w.scale, False,
                                   cu, window=_oracle_window(w, window))
    e, _, _ = check_o(host64(o), o_ref, w.dtype)
    el = check_lse(host64(lse), lse_ref)
    say(f"   max|dO|={e:.2e} max|dLSE|={el:.2e}")


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("window", WINDOWS)
def test_forward(dtype, d, window):
    N = 333 if d < 256 else 200
    compare_fwd(W.custom(B=2, Hq=2, Hkv=1, N=N, d=d, dtype=dtype, causal=False,
                         seed=600 + d + WINDOWS.index(window)), window)


@pytest.mark.parametrize("N", [1, 64, 65, 700])
def test_forward_lengths(N):
    compare_fwd(W.custom(B=1, Hq=4, Hkv=2, N=N, d=128, dtype="bf16", causal=False, seed=610 + N),
                (100, 20))


def test_forward_causal_flag_with_window():
    """causal=True with a window keeps the left bound and closes the right side."""
    compare_fwd(W.custom(B=1, Hq=2, Hkv=2, N=500, d=128, dtype="fp16", causal=True, seed=620),
                (90, 40))


def test_forward_varlen_gqa():
    w = W.custom(B=0, Hq=8, Hkv=2, N=0, d=128, dtype="bf16", causal=False, seed=621,
                 lens=[300, 0, 1, 129, 64, 513])
    compare_fwd(w, (70, 10))


def test_forward_long():
    """Several interior tiles between the two masked edges."""
    compare_fwd(W.custom(B=1, Hq=2, Hkv=2, N=2100, d=128, dtype="bf16", causal=False, seed=622),
                (512, 256))


@pytest.mark.parametrize("window,causal", [((-1, 0), True), ((-1, -1), False)])
def test_plain_bands_match_the_plain_calls(window, causal):
    """(−1, 0) and (−1, −1) run the causal and unmasked kernels: identical bits."""
    import torch
    fa = _fa()
    w = W.custom(B=2, Hq=4, Hkv=2, N=300, d=128, dtype="fp16", causal=False, seed=623)
    t = to_device(W.generate(w, with_grad=False), w.dtype)
    q, k, v, _ = _views(w, t)
    o1, l1 = fa.flash_attn_func(q, k, v, causal=causal, softmax_scale=w.scale)
    o2, l2 = fa.flash_attn_func(q, k, v, causal=False, softmax_scale=w.scale, window_size=window)
    torch.cuda.synchronize()
    assert bits_equal(o1, o2) and bits_equal(l1, l2)


# ---- backward -----------------------------------------------------------------
def compare_bwd(w, window):
    import torch
    fa = _fa()
    t = to_device(W.generate(w, with_grad=True), w.dtype)
    say(f"[fa_bwd_window] {window} B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} d={w.d} {w.dtype} "
        f"varlen={w.varlen}")
    q, k, v, kw = _views(w, t)
    do = t["do"].view(q.shape)
    o, lse = fa.flash_attn_func(q, k, v, softmax_scale=w.scale, window_size=window, **kw)
    dq, dk, dv = fa.flash_attn_backward(do, q, k, v, o, lse, softmax_scale=w.scale,
                                        window_size=window, **kw)
    torch.cuda.synchronize()
    cu = t["cu_seqlens"].cpu().numpy()
    ref = attention_bwd(host64(t["q"]), host64(t["k"]), host64(t["v"]), host64(t["do"]), w.scale,
                        False, cu, window=window)
    T = w.T
    got = (dq.reshape(T, w.Hq, w.d), dk.reshape(T, w.Hkv, w.d), dv.reshape(T, w.Hkv, w.d))
    res = [check_grad(host64(g), r, n) for g, r, n in zip(got, ref, ("dQ", "dK", "dV"))]
    say("   " + " ".join(f"{n}: rel {a:.2e}" for n, (a, _) in zip(("dQ", "dK", "dV"), res)))


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("window", WINDOWS)
def test_backward(dtype, d, window):
    compare_bwd(W.custom(B=2, Hq=2, Hkv=1, N=333, d=d, dtype=dtype, causal=False,
                         seed=700 + d + WINDOWS.index(window), backward=True), window)


def test_backward_varlen_gqa():
    w = W.custom(B=0, Hq=8, Hkv=2, N=0, d=128, dtype="bf16", causal=False, seed=720,
                 lens=[300, 0, 1, 129, 64, 513], backward=True)
    compare_bwd(w, (70, 10))


@pytest.mark.parametrize("window", [(70, 10), (4095, 0), (130, 200)])
def test_backward_d256_varlen_gqa(window):
    """d = 256 (two-pass dK/dV): varlen with GQA, empty and one-token sequences,
    windows narrower and wider than the 128-key block and a causal-style band."""
    w = W.custom(B=0, Hq=8, Hkv=2, N=0, d=256, dtype="bf16", causal=False, seed=722,
                 lens=[300, 0, 1, 129, 64, 513], backward=True)
    compare_bwd(w, window)


def test_backward_long():
    compare_bwd(W.custom(B=1, Hq=2, Hkv=2, N=1500, d=128, dtype="fp16", causal=False, seed=721,
                         backward=True), (400, 130))


def test_window_deterministic():
    import torch
    fa = _fa()
    w = W.custom(B=1, Hq=2, Hkv=2, N=600, d=128, dtype="bf16", causal=False, seed=722,
                 backward=True)
    t = to_device(W.generate(w, with_grad=True), w.dtype)
    q, k, v, _ = _views(w, t)
    do = t["do"].view(q.shape)
    outs = []
    for _ in range(2):
        o, lse = fa.flash_attn_func(q, k, v, softmax_scale=w.scale, window_size=(77, 33))
        grads = fa.flash_attn_backward(do, q, k, v, o, lse, softmax_scale=w.scale,
                                       window_size=(77, 33))
        outs.append((o, lse) + tuple(grads))
    torch.cuda.synchronize()
    assert all(bits_equal(a, b) for a, b in zip(*outs))
