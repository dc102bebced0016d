"""Parity at the full sizes the benchmark times, for the workloads beyond the
training step: the sliding window (window_16k), the soft cap (softcap_16k, and
softcap_d256 at head dimension 256), dropout (dropout_16k) and head dimension
256 (train_d256). Each runs forward
and backward through the same entry points bench.py times, at the same shape;
the oracle then computes sampled query rows of the forward one by one and whole
(sequence, head) units of the backward.
"""
import numpy as np
import pytest

import workloads as W
from oracle import attention_bwd_sampled, attention_fwd_rows, head_bwd_dropout, head_fwd_dropout
from parity_util import check_grad, check_lse, check_o, host64, say, to_device

pytestmark = pytest.mark.gpu


def _rows(rng, L, n=10):
    fixed = [0, 1, 63, 64, 127, 128, L // 2, L - 65, L - 1]
    return sorted(set(r for r in fixed if 0 <= r < L) | set(int(x) for x in rng.integers(0, L, n)))


def _run(w):
    import torch
    import exact_io_aware_12_amd as fa
    t = to_device(W.generate(w, with_grad=True), w.dtype)
    say(f"[full size] {w.name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} d={w.d} causal={w.causal} "
        f"window={w.window} softcap={w.softcap} dropout={w.dropout_p}")
    shp = (w.B, w.N)
    q = t["q"].view(*shp, w.Hq, w.d)
    k, v = (t[n].view(*shp, w.Hkv, w.d) for n in ("k", "v"))
    do = t["do"].view(*shp, w.Hq, w.d)
    kw = dict(causal=w.causal, softmax_scale=w.scale)
    if w.window is not None:
        kw["window_size"] = w.window
    if w.softcap:
        kw["softcap"] = w.softcap
    if w.dropout_p:
        kw.update(dropout_p=w.dropout_p, dropout_seed=w.dropout_seed)
    o, lse = fa.flash_attn_func(q, k, v, **kw)
    dq, dk, dv = fa.flash_attn_backward(do, q, k, v, o, lse, **kw)
    torch.cuda.synchronize()
    T = w.T
    return (o.reshape(T, w.Hq, w.d), lse, dq.reshape(T, w.Hq, w.d), dk.reshape(T, w.Hkv, w.d),
            dv.reshape(T, w.Hkv, w.d), t)


def _check(w, fwd_units, bwd_units, seed):
    import torch
    o, lse, dq, dk, dv, t = _run(w)
    cu = w.cu_seqlens()
    rng = np.random.default_rng(seed)
    g = w.Hq // w.Hkv
    for s, h in fwd_units:
        rows = _rows(rng, w.N)
        sl = slice(int(cu[s]), int(cu[s + 1]))
        if w.dropout_p:
            o_ref, l_ref = head_fwd_dropout(t["q"][sl, h], t["k"][sl, h // g], t["v"][sl, h // g],
                                            w.scale, w.causal, s, h, w.dropout_p,
                                            w.dropout_seed, rows=rows)
        else:
            o_ref, l_ref = attention_fwd_rows(t["q"], t["k"], t["v"], w.scale, w.causal, cu, s, h,
                                              rows, window=w.window, softcap=w.softcap or None)
        gi = torch.as_tensor(cu[s] + np.array(rows), device=o.device)
        check_o(host64(o[gi, h]), o_ref, w.dtype, f"O seq {s} head {h}")
        check_lse(host64(lse[h, gi]), l_ref, f"LSE seq {s} head {h}")
    for s, kvh in bwd_units:
        sl = slice(int(cu[s]), int(cu[s + 1]))
        if w.dropout_p:
            rq = []
            rk = rv = 0.0
            for r in range(g):
                h = kvh * g + r
                a, b, c = head_bwd_dropout(t["q"][sl, h], t["k"][sl, kvh], t["v"][sl, kvh],
                                           t["do"][sl, h], w.scale, w.causal, s, h, w.dropout_p,
                                           w.dropout_seed)
                rq.append(a)
                rk, rv = rk + b, rv + c
            rq = np.stack(rq, axis=1)
        else:
            ref = attention_bwd_sampled(t["q"], t["k"], t["v"], t["do"], w.scale, w.causal, cu,
                                        [(s, kvh)], window=w.window, softcap=w.softcap or None)
            rq, rk, rv = ref[(s, kvh)]
        check_grad(host64(dq[sl, kvh * g:(kvh + 1) * g]), rq, f"dQ seq {s} kv head {kvh}")
        check_grad(host64(dk[sl, kvh]), rk, f"dK seq {s} kv head {kvh}")
        r = check_grad(host64(dv[sl, kvh]), rv, f"dV seq {s} kv head {kvh}")
        say(f"   backward unit ({s}, {kvh}) ok; dV rel {r[0]:.2e}")


def test_window_16k_full_size():
    _check(W.WORKLOADS["window_16k"], [(0, 0), (1, 13)], [(1, 7)], seed=31)


def test_softcap_16k_full_size():
    _check(W.WORKLOADS["softcap_16k"], [(0, 2), (1, 15)], [(0, 9)], seed=32)


def test_dropout_16k_full_size():
    _check(W.WORKLOADS["dropout_16k"], [(0, 4), (1, 11)], [(1, 3)], seed=33)


def test_train_d256_full_size():
    _check(W.WORKLOADS["train_d256"], [(0, 0), (3, 15), (2, 7)], [(1, 5), (3, 0)], seed=34)


def test_softcap_d256_full_size():
    """Soft cap 50 at d = 256 with GQA 16/8 (the Gemma-2 setting) at the benchmark's size."""
    _check(W.WORKLOADS["softcap_d256"], [(0, 0), (3, 15), (1, 6)], [(2, 3), (0, 7)], seed=35)
