"""GPU parity of the dropout entry points (fa_fwd_dropout, fa_bwd_dropout through
the binding's dropout_p / dropout_seed) against the oracle.

Two read-outs check the keep decisions bit for bit against the oracle's
Philox4x32-10 mask: with Q = 0 every visible weight is 1/n, so with one-hot
value rows O_ic · n · t/256 is the keep bit of (query i, key c) (forward and dQ
kernels' layout); with one-hot dO rows, dV_jc · n_c · t/256 is the keep bit of
(query c, key j) (the dK/dV kernel's layout). Random inputs then check O, LSE
and the gradients with the plain path's tolerances, across both masks, d 64 and
128, fp16 and bf16, varlen with GQA and ragged lengths; dropout_p = 0 must run
the plain kernels bit for bit.
"""
import numpy as np
import pytest

import workloads as W
from oracle import attention_bwd_dropout, attention_fwd_dropout, keep_mask, keep_threshold
from parity_util import bits_equal, check_grad, check_lse, check_o, host64, say, to_device

pytestmark = pytest.mark.gpu

SEED = 0x0123456789ABCDEF


def _fa():
    import exact_io_aware_12_amd as fa   # raises if libfa.so is missing: no fallback
    return fa


def _tdt(dtype):
    import torch
    return {"fp16": torch.float16, "bf16": torch.bfloat16}[dtype]


def _readout_inputs(B, H, L, dtype):
    import torch
    td = _tdt(dtype)
    q = torch.zeros((B, L, H, 128), dtype=td, device="cuda")
    k = torch.randn((B, L, H, 128), generator=torch.Generator().manual_seed(1)).to(td).cuda()
    eye = torch.eye(L, 128, dtype=td, device="cuda")      # V_j = e_j, dO_i = e_i
    v = eye[None, :, None, :].expand(B, L, H, 128).contiguous()
    return q, k, v


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("p", [0.3, 0.75])
def test_forward_keep_bits(dtype, causal, p):
    import torch
    fa = _fa()
    B, H, L = 2, 3, 128
    q, k, v = _readout_inputs(B, H, L, dtype)
    say(f"[fa_fwd_dropout readout] {dtype} causal={causal} p={p}")
    o, _ = fa.flash_attn_func(q, k, v, causal=causal, dropout_p=p, dropout_seed=SEED)
    torch.cuda.synchronize()
    t = keep_threshold(p)
    o = o.double().cpu().numpy()
    n = (np.arange(L) + 1.0) if causal else np.full(L, float(L))
    for b in range(B):
        for h in range(H):
            got = np.rint(o[b, :, h, :L] * n[:, None] * t / 256.0)
            ref = keep_mask(SEED, b, h, np.arange(L), np.arange(L), t).astype(float)
            if causal:
                ref = np.tril(ref)
            assert np.array_equal(got, ref), f"(b={b}, h={h}): {int((got != ref).sum())} bits differ"


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_keep_bits(dtype, causal):
    import torch
    fa = _fa()
    B, H, L, p = 2, 3, 128, 0.3
    q, k, v = _readout_inputs(B, H, L, dtype)
    do = v.clone()   # dO_i = e_i
    say(f"[fa_bwd_dropout readout] {dtype} causal={causal} p={p}")
    o, lse = fa.flash_attn_func(q, k, v, causal=causal, dropout_p=p, dropout_seed=SEED)
    dq, dk, dv = fa.flash_attn_backward(do, q, k, v, o, lse, causal=causal, dropout_p=p,
                                        dropout_seed=SEED)
    torch.cuda.synchronize()
    t = keep_threshold(p)
    dv = dv.double().cpu().numpy()
    n = (np.arange(L) + 1.0) if causal else np.full(L, float(L))   # visible keys of query c
    for b in range(B):
        for h in range(H):
            got = np.rint(dv[b, :, h, :L] * n[None, :] * t / 256.0)   # [key j, query c]
            ref = keep_mask(SEED, b, h, np.arange(L), np.arange(L), t).astype(float)
            if causal:
                ref = np.tril(ref)
            assert np.array_equal(got, ref.T), f"(b={b}, h={h}): {int((got != ref.T).sum())} differ"
    # dQ of the same call against the oracle (its dS carries Z on the diagonal)
    ref = attention_bwd_dropout(host64(q.view(B * L, H, 128)), host64(k.view(B * L, H, 128)),
                                host64(v.view(B * L, H, 128)), host64(do.view(B * L, H, 128)),
                                128 ** -0.5, causal, np.arange(B + 1) * L, p, SEED)
    check_grad(host64(dq.view(B * L, H, 128)), ref[0], "dQ")


# ---- random inputs --------------------------------------------------------------
def _views(w, t):
    if w.varlen:
        return t["q"], t["k"], t["v"], dict(cu_seqlens=t["cu_seqlens"], max_seqlen=w.N)
    shp = (w.B, w.N)
    return (t["q"].view(*shp, w.Hq, w.d), t["k"].view(*shp, w.Hkv, w.d),
            t["v"].view(*shp, w.Hkv, w.d), {})


def compare(w, p, seed, backward=True):
    import torch
    fa = _fa()
    t = to_device(W.generate(w, with_grad=True), w.dtype)
    say(f"[fa_fwd/bwd_dropout] p={p} seed={seed:#x} B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} "
        f"d={w.d} {w.dtype} causal={w.causal} varlen={w.varlen}")
    q, k, v, kw = _views(w, t)
    o, lse = fa.flash_attn_func(q, k, v, causal=w.causal, dropout_p=p, dropout_seed=seed, **kw)
    if backward:
        do = t["do"].view(q.shape)
        dq, dk, dv = fa.flash_attn_backward(do, q, k, v, o, lse, causal=w.causal, dropout_p=p,
                                            dropout_seed=seed, **kw)
    torch.cuda.synchronize()
    cu = t["cu_seqlens"].cpu().numpy()
    args = (host64(t["q"]), host64(t["k"]), host64(t["v"]))
    o_ref, lse_ref = attention_fwd_dropout(*args, w.scale, w.causal, cu, p, seed)
    e, _, _ = check_o(host64(o.reshape(w.T, w.Hq, w.d)), o_ref, w.dtype)
    el = check_lse(host64(lse), lse_ref)
    msg = f"   max|dO|={e:.2e} max|dLSE|={el:.2e}"
    if backward:
        ref = attention_bwd_dropout(*args, host64(t["do"]), w.scale, w.causal, cu, p, seed)
        T = w.T
        got = (dq.reshape(T, w.Hq, w.d), dk.reshape(T, w.Hkv, w.d), dv.reshape(T, w.Hkv, w.d))
        res = [check_grad(host64(g), r, n) for g, r, n in zip(got, ref, ("dQ", "dK", "dV"))]
        msg += " " + " ".join(f"{n}: rel {a:.2e}" for n, (a, _) in zip(("dQ", "dK", "dV"), res))
    say(msg)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("p", [0.1, 0.5])
def test_dropout_parity(dtype, d, causal, p):
    compare(W.custom(B=2, Hq=2, Hkv=1, N=333, d=d, dtype=dtype, causal=causal,
                     seed=950 + d + int(10 * p), backward=True), p, SEED + d)


@pytest.mark.parametrize("N", [1, 65, 700])
def test_dropout_lengths(N):
    compare(W.custom(B=1, Hq=4, Hkv=2, N=N, d=128, dtype="bf16", causal=True, seed=960 + N,
                     backward=True), 0.2, 77)


def test_dropout_varlen_gqa():
    w = W.custom(B=0, Hq=8, Hkv=2, N=0, d=128, dtype="bf16", causal=True, seed=965,
                 lens=[300, 0, 1, 129, 64, 513], backward=True)
    compare(w, 0.15, 2 ** 64 - 1)


def test_dropout_varlen_gqa_d256():
    """d = 256 (the two-pass dK/dV kernel draws the same decisions in both passes)."""
    w = W.custom(B=0, Hq=8, Hkv=4, N=0, d=256, dtype="bf16", causal=True, seed=967,
                 lens=[300, 0, 1, 200, 129], backward=True)
    compare(w, 0.2, 0xDEADBEEF)


def test_dropout_long():
    compare(W.custom(B=1, Hq=2, Hkv=2, N=1500, d=128, dtype="fp16", causal=False, seed=966,
                     backward=True), 0.1, 12345)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_dropout_runs_the_plain_kernels(causal):
    import torch
    fa = _fa()
    w = W.custom(B=2, Hq=4, Hkv=2, N=300, d=128, dtype="fp16", causal=causal, seed=967,
                 backward=True)
    t = to_device(W.generate(w, with_grad=True), w.dtype)
    q, k, v, _ = _views(w, t)
    do = t["do"].view(q.shape)
    o1, l1 = fa.flash_attn_func(q, k, v, causal=causal)
    o2, l2 = fa.flash_attn_func(q, k, v, causal=causal, dropout_p=0.0, dropout_seed=5)
    g1 = fa.flash_attn_backward(do, q, k, v, o1, l1, causal=causal)
    g2 = fa.flash_attn_backward(do, q, k, v, o2, l2, causal=causal, dropout_p=0.0,
                                dropout_seed=5)
    torch.cuda.synchronize()
    assert bits_equal(o1, o2) and bits_equal(l1, l2)
    assert all(bits_equal(a, b) for a, b in zip(g1, g2))


def test_dropout_deterministic_and_seeded():
    import torch
    fa = _fa()
    w = W.custom(B=1, Hq=2, Hkv=2, N=600, d=128, dtype="bf16", causal=True, seed=968,
                 backward=True)
    t = to_device(W.generate(w, with_grad=True), w.dtype)
    q, k, v, _ = _views(w, t)
    do = t["do"].view(q.shape)
    outs = []
    for seed in (11, 11, 12):
        o, lse = fa.flash_attn_func(q, k, v, causal=True, dropout_p=0.3, dropout_seed=seed)
        grads = fa.flash_attn_backward(do, q, k, v, o, lse, causal=True, dropout_p=0.3,
                                       dropout_seed=seed)
        outs.append((o, lse) + tuple(grads))
    torch.cuda.synchronize()
    assert all(bits_equal(a, b) for a, b in zip(outs[0], outs[1]))
    assert not bits_equal(outs[0][0], outs[2][0])        # another seed, other decisions
    assert bits_equal(outs[0][1], outs[2][1])            # the LSE ignores dropout
