"""GPU parity of fa_bwd against the float64 oracle (through the C ABI).

The GPU backward consumes the GPU forward's O and LSE, exactly as a training
step does; the oracle recomputes everything from Q, K, V, dO by definition.
"""
import numpy as np
import pytest

import workloads as W
from oracle import attention_bwd, attention_bwd_rows
from parity_util import (bits_equal, check_grad, host32, host64, map_units, say,
                         tile_rows, to_device)

pytestmark = pytest.mark.gpu


def run_fwd_bwd(w: W.Workload, arrays=None):
    import torch
    import exact_io_aware_12_amd as fa
    arrays = W.generate(w, with_grad=True) if arrays is None else arrays
    t = to_device(arrays, w.dtype)
    say(f"[fa_fwd+fa_bwd] {w.name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} d={w.d} {w.dtype} "
        f"causal={w.causal} varlen={w.varlen} T={w.T}")
    kw = dict(causal=w.causal, softmax_scale=w.scale)
    if w.varlen:
        kw.update(cu_seqlens=t["cu_seqlens"], max_seqlen=w.N)
        q, k, v, do = t["q"], t["k"], t["v"], t["do"]
    else:
        shp = (w.B, w.N)
        q, k, v = (t[n].view(*shp, -1, w.d) for n in ("q", "k", "v"))
        do = t["do"].view(*shp, w.Hq, w.d)
    o, lse = fa.flash_attn_func(q, k, v, **kw)
    dq, dk, dv = fa.flash_attn_backward(do, q, k, v, o, lse, **kw)
    torch.cuda.synchronize()
    T = w.T
    return (dq.view(T, w.Hq, w.d), dk.view(T, w.Hkv, w.d), dv.view(T, w.Hkv, w.d)), t


def compare_whole(w, arrays=None):
    (dq, dk, dv), t = run_fwd_bwd(w, arrays)
    cu = t["cu_seqlens"].cpu().numpy()
    ref = attention_bwd(host64(t["q"]), host64(t["k"]), host64(t["v"]), host64(t["do"]), w.scale,
                        w.causal, cu)
    res = [check_grad(host64(g), r, n) for g, r, n in zip((dq, dk, dv), ref, ("dQ", "dK", "dV"))]
    say("   " + " ".join(f"{n}: rel {a:.2e} frob {b:.2e}" for n, (a, b) in
                         zip(("dQ", "dK", "dV"), res)))
    return (dq, dk, dv), t


def test_tiny_backward():
    w = W.WORKLOADS["tiny"]
    compare_whole(W.custom(B=w.B, Hq=w.Hq, Hkv=w.Hkv, N=w.N, d=w.d, dtype=w.dtype,
                           causal=w.causal, seed=w.seed, backward=True))


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 33, 64, 129, 300])
def test_ragged_lengths(dtype, d, causal, N):
    compare_whole(W.custom(B=2, Hq=2, Hkv=2, N=N, d=d, dtype=dtype, causal=causal,
                           seed=200 + N, backward=True))


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_varlen(causal):
    w = W.custom(B=0, Hq=8, Hkv=2, N=0, d=128, dtype="bf16", causal=causal, seed=21,
                 lens=[0, 1, 77, 128, 200, 64], backward=True)
    compare_whole(w)


def test_causal_d64_shape_backward():
    compare_whole(W.custom(B=1, Hq=16, Hkv=16, N=2048, d=64, dtype="fp16", causal=True, seed=2,
                           backward=True))


def test_identities_on_gpu():
    """Σ_j dV_j = Σ_i dO_i and Σ_j dK_j = 0 per (sequence, head), up to rounding."""
    w = W.custom(B=2, Hq=4, Hkv=4, N=500, d=128, dtype="fp16", causal=True, seed=22, backward=True)
    (dq, dk, dv), t = run_fwd_bwd(w)
    dk64, dv64, do64 = host64(dk), host64(dv), host64(t["do"])
    for b in range(2):
        sl = slice(b * 500, (b + 1) * 500)
        np.testing.assert_allclose(dv64[sl].sum(0), do64[sl].sum(0), rtol=1e-2, atol=0.05)
        bound = 2e-3 * np.abs(dk64[sl]).sum(0) + 1e-3
        assert (np.abs(dk64[sl].sum(0)) <= bound).all()


def test_deterministic():
    w = W.custom(B=1, Hq=4, Hkv=2, N=700, d=128, dtype="bf16", causal=True, seed=23, backward=True)
    a = W.generate(w)
    (g1, _), (g2, _) = run_fwd_bwd(w, a), run_fwd_bwd(w, a)
    for x, y in zip(g1, g2):
        assert bits_equal(x, y)


def test_train_16k_backward_every_unit():
    """The training-step workload at full size: every (sequence, KV head) unit,
    dQ on query rows and dK, dV on keys from each unit's first, one inner and
    last tile, against the oracle's selected-row backward."""
    w = W.WORKLOADS["train_16k"]
    (dq, dk, dv), t = run_fwd_bwd(w)
    cu = w.cu_seqlens()
    rng = np.random.default_rng(55)
    q, k, v, do = (host32(t[n]) for n in ("q", "k", "v", "do"))
    g = w.Hq // w.Hkv
    units = [(s, kvh) for s in range(w.B) for kvh in range(w.Hkv)]
    sel = {u: (tile_rows(rng, w.N, 128), tile_rows(rng, w.N, 128)) for u in units}
    refs = map_units(lambda u: attention_bwd_rows(q, k, v, do, w.scale, w.causal, cu, u[0], u[1],
                                                  *sel[u]), units)
    dq_h, dk_h, dv_h = host64(dq), host64(dk), host64(dv)
    worst = [0.0, 0.0, 0.0]
    for u, (rq, rk, rv) in zip(units, refs):
        (s, kvh), (qr, kr) = u, sel[u]
        tq, tk = cu[s] + np.array(qr), cu[s] + np.array(kr)
        res = (check_grad(dq_h[tq, kvh * g:(kvh + 1) * g], rq, f"dQ unit {u}"),
               check_grad(dk_h[tk, kvh], rk, f"dK unit {u}"),
               check_grad(dv_h[tk, kvh], rv, f"dV unit {u}"))
        worst = [max(a, r[0]) for a, r in zip(worst, res)]
    say(f"   every unit ({len(units)}): worst rel dQ {worst[0]:.2e} dK {worst[1]:.2e} "
        f"dV {worst[2]:.2e}")


def test_gqa_varlen_backward_every_unit():
    """The GQA packed-batch workload (Hq 32, Hkv 8, 8 sequences of 1024-8192
    tokens, causal) through the backward at full size: for every (sequence, KV
    head) unit, dQ of the unit's 4 query heads on query rows and dK, dV on keys
    from the first, one inner and the last tile of the sequence, against the
    oracle's selected-row backward. The dK/dV kernel's loop over the query heads
    of a group and its ragged last tiles run here at their full-size form."""
    w = W.WORKLOADS["gqa_varlen"]
    (dq, dk, dv), t = run_fwd_bwd(w)
    cu = w.cu_seqlens()
    rng = np.random.default_rng(56)
    q, k, v, do = (host32(t[n]) for n in ("q", "k", "v", "do"))
    g = w.Hq // w.Hkv
    units = [(s, kvh) for s in range(w.B) for kvh in range(w.Hkv)]
    lens = np.diff(cu)
    sel = {u: (tile_rows(rng, int(lens[u[0]]), 128), tile_rows(rng, int(lens[u[0]]), 128))
           for u in units}
    refs = map_units(lambda u: attention_bwd_rows(q, k, v, do, w.scale, w.causal, cu, u[0], u[1],
                                                  *sel[u]), units)
    dq_h, dk_h, dv_h = host64(dq), host64(dk), host64(dv)
    worst = [0.0, 0.0, 0.0]
    for u, (rq, rk, rv) in zip(units, refs):
        (s, kvh), (qr, kr) = u, sel[u]
        tq, tk = cu[s] + np.array(qr), cu[s] + np.array(kr)
        res = (check_grad(dq_h[tq, kvh * g:(kvh + 1) * g], rq, f"dQ unit {u}"),
               check_grad(dk_h[tk, kvh], rk, f"dK unit {u}"),
               check_grad(dv_h[tk, kvh], rv, f"dV unit {u}"))
        worst = [max(a, r[0]) for a, r in zip(worst, res)]
    say(f"   every unit ({len(units)}): worst rel dQ {worst[0]:.2e} dK {worst[1]:.2e} "
        f"dV {worst[2]:.2e}")
