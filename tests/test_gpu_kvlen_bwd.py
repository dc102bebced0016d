"""GPU parity of fa_bwd_kvlen (the backward for queries and keys of different
lengths) against the float64 oracle (oracle.decode.kvlen_bwd), through the
C ABI. The GPU backward consumes the GPU forward's O and LSE (fa_fwd_kvlen),
as a training step does.

Cases: fixed length with Nq < Nk (a chunk over a longer context), Nq = Nk
(bitwise equal to fa_bwd), Nq > Nk (causal rows before every key: dq = 0),
Nk = 0 (dq = 0) and Nq = 0 (dk = dv = 0); head dims 64/128, fp16/bf16, causal
or not, GQA; varlen with ragged lengths on both sides including empty
sequences; the chunked-prefill workload at full size on sampled units.
"""
import numpy as np
import pytest

from oracle.decode import kvlen_bwd, kvlen_head_bwd
from parity_util import bits_equal, check_grad, host64, map_units, say, torch_dtype

pytestmark = pytest.mark.gpu


def _fa():
    import exact_io_aware_12_amd as fa   # raises if libfa.so is missing: no fallback
    return fa


def _randn(rng, shape, dtype):
    import torch
    return torch.from_numpy(rng.standard_normal(shape, dtype=np.float32)).to(
        torch_dtype(dtype)).cuda()


def _check(g, r, what):
    """Gradient tolerance; an all-zero reference (no query or no key) needs exact zeros."""
    g = host64(g)
    if not np.abs(r).max(initial=0.0) > 0:
        assert (g == 0).all(), f"{what}: must be exactly 0"
        return 0.0
    return check_grad(g, r, what)[0]


def run_fixed(B, Hq, Hkv, Nq, Nk, d, dtype, causal, seed):
    import torch
    fa = _fa()
    rng = np.random.default_rng(seed)
    q = _randn(rng, (B, Nq, Hq, d), dtype)
    k = _randn(rng, (B, Nk, Hkv, d), dtype)
    v = _randn(rng, (B, Nk, Hkv, d), dtype)
    do = _randn(rng, (B, Nq, Hq, d), dtype)
    say(f"[fa_bwd_kvlen] B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} {dtype} causal={causal}")
    o, lse = fa.flash_attn_kvlen_func(q, k, v, causal=causal)
    dq, dk, dv = fa.flash_attn_kvlen_backward(do, q, k, v, o, lse, causal=causal)
    torch.cuda.synchronize()
    return (q, k, v, do), (dq, dk, dv)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Nq,Nk", [(200, 700), (130, 130), (300, 77), (64, 0), (0, 90),
                                   (1, 513), (257, 1000)])
def test_fixed_length(dtype, d, causal, Nq, Nk):
    B, Hq, Hkv = 2, 4, 2
    (q, k, v, do), (dq, dk, dv) = run_fixed(B, Hq, Hkv, Nq, Nk, d, dtype, causal,
                                            900 + d + Nq + Nk)
    cq, ck = np.arange(B + 1) * Nq, np.arange(B + 1) * Nk
    ref = kvlen_bwd(host64(q).reshape(B * Nq, Hq, d), host64(k).reshape(B * Nk, Hkv, d),
                    host64(v).reshape(B * Nk, Hkv, d), host64(do).reshape(B * Nq, Hq, d),
                    1.0 / np.sqrt(d), causal, cq, ck)
    rel = [_check(g.reshape(r.shape), r, n) for g, r, n in zip((dq, dk, dv), ref, ("dQ", "dK", "dV"))]
    say(f"   rel dQ {rel[0]:.2e} dK {rel[1]:.2e} dV {rel[2]:.2e}")


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_equal_lengths_match_fa_bwd_bitwise(dtype, causal):
    """With Lq = Lk the kernels run fa_bwd's arithmetic: identical bits."""
    import torch
    fa = _fa()
    (q, k, v, do), (dq, dk, dv) = run_fixed(2, 8, 2, 333, 333, 128, dtype, causal, 91)
    o, lse = fa.flash_attn_func(q, k, v, causal=causal)
    g2 = fa.flash_attn_backward(do, q, k, v, o, lse, causal=causal)
    torch.cuda.synchronize()
    for x, y in zip((dq, dk, dv), g2):
        assert bits_equal(x, y)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_varlen(causal, d):
    import torch
    fa = _fa()
    lq = [0, 37, 300, 128, 5, 64, 0]
    lk = [19, 0, 900, 128, 200, 33, 0]
    cq = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    rng = np.random.default_rng(93 + d)
    Hq, Hkv = 8, 2
    q = _randn(rng, (int(cq[-1]), Hq, d), "bf16")
    k = _randn(rng, (int(ck[-1]), Hkv, d), "bf16")
    v = _randn(rng, (int(ck[-1]), Hkv, d), "bf16")
    do = _randn(rng, (int(cq[-1]), Hq, d), "bf16")
    tq, tk = torch.from_numpy(cq).cuda(), torch.from_numpy(ck).cuda()
    say(f"[fa_bwd_kvlen] varlen lq={lq} lk={lk} d={d} causal={causal}")
    kw = dict(causal=causal, cu_seqlens_q=tq, cu_seqlens_k=tk, max_seqlen_q=max(lq),
              max_seqlen_k=max(lk))
    o, lse = fa.flash_attn_kvlen_func(q, k, v, **kw)
    dq, dk, dv = fa.flash_attn_kvlen_backward(do, q, k, v, o, lse, **kw)
    torch.cuda.synchronize()
    ref = kvlen_bwd(host64(q), host64(k), host64(v), host64(do), 1.0 / np.sqrt(d), causal, cq, ck)
    for g, r, n in zip((dq, dk, dv), ref, ("dQ", "dK", "dV")):
        _check(g, r, n)


def test_prefill_chunk_sampled():
    """The chunked-prefill shape at full size (B4 Hq32 Hkv8, 2048 queries over
    8192 keys, bf16, causal): every batch entry and KV head, one query head of
    each group, against the oracle."""
    import torch
    fa = _fa()
    import workloads as W
    w = W.KVLEN_WORKLOADS["prefill_chunk"]
    a = W.generate_kvlen(w)
    td = torch_dtype(w.dtype)
    q, k, v = (torch.from_numpy(a[n]).to(td).cuda() for n in ("q", "k", "v"))
    rng = np.random.default_rng(97)
    do = _randn(rng, tuple(q.shape), w.dtype)
    say(f"[fa_bwd_kvlen] prefill_chunk B={w.B} Nq={w.Nq} Nk={w.Nk}")
    o, lse = fa.flash_attn_kvlen_func(q, k, v, causal=True)
    dq, dk, dv = fa.flash_attn_kvlen_backward(do, q, k, v, o, lse, causal=True)
    torch.cuda.synchronize()
    g = w.Hq // w.Hkv
    units = [(b, kvh) for b in range(w.B) for kvh in range(w.Hkv)]
    qh = {u: u[1] * g + (u[0] + u[1]) % g for u in units}   # one query head per group
    qf, kf, vf, dof = (x.float().cpu().numpy() for x in (q, k, v, do))

    def ref(u):
        b, kvh = u
        return kvlen_head_bwd(qf[b, :, qh[u]], kf[b, :, kvh], vf[b, :, kvh], dof[b, :, qh[u]],
                              w.scale, True)
    refs = map_units(ref, units)
    dq_h = host64(dq)
    for u, (rq, _, _) in zip(units, refs):
        check_grad(dq_h[u[0], :, qh[u]], rq, f"dQ unit {u}")
    # dK, dV sum over the group's query heads: compare the group sums of the oracle
    dk_h, dv_h = host64(dk), host64(dv)
    for b, kvh in units[:4]:
        rk = np.zeros((w.Nk, w.d))
        rv = np.zeros((w.Nk, w.d))
        for r in range(g):
            _, rkr, rvr = kvlen_head_bwd(qf[b, :, kvh * g + r], kf[b, :, kvh], vf[b, :, kvh],
                                         dof[b, :, kvh * g + r], w.scale, True)
            rk += rkr
            rv += rvr
        check_grad(dk_h[b, :, kvh], rk, f"dK unit {(b, kvh)}")
        check_grad(dv_h[b, :, kvh], rv, f"dV unit {(b, kvh)}")
    say(f"   dQ on {len(units)} units, dK/dV on 4 units ok")
