"""Pins for the oracle's backward: dQ, dK, dV.

The pages give no gradient formulas (only that the backward recomputes S
rather than storing it: FlashAttention guide, cxbdf.cn, part 2, item 3), so
the oracle's backward is the chain rule of the forward definition. It is
pinned by hand-worked values, central finite differences of the forward,
exact identities of softmax attention, a pure-Python brute force and torch's
CPU float64 autograd.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import attention_fwd, attention_bwd, attention_bwd_sampled, bruteforce

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")))


def _rand(rng, *shape):
    return rng.standard_normal(shape)


@pytest.mark.parametrize("case", ["full", "causal"])
def test_worked_example(case):
    c = GOLD["cases"][case]
    q = np.array([0.0, 1.0]).reshape(2, 1, 1)
    k = np.array([0.0, math.log(3.0)]).reshape(2, 1, 1)
    v = np.array([4.0, 8.0]).reshape(2, 1, 1)
    do = np.ones((2, 1, 1))
    dq, dk, dv = attention_bwd(q, k, v, do, 1.0, c["causal"])
    np.testing.assert_allclose(dq[:, 0, 0], c["dq"]["values"], atol=1e-14)
    np.testing.assert_allclose(dk[:, 0, 0], c["dk"]["values"], atol=1e-14)
    np.testing.assert_allclose(dv[:, 0, 0], c["dv"]["values"], atol=1e-14)


def test_single_token():
    rng = np.random.default_rng(0)
    q, k, v, do = (_rand(rng, 1, 2, 4) for _ in range(4))
    dq, dk, dv = attention_bwd(q, k, v, do, 0.5, False)
    np.testing.assert_allclose(dq, 0.0, atol=1e-15)
    np.testing.assert_allclose(dk, 0.0, atol=1e-15)
    np.testing.assert_allclose(dv, do, atol=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_constant_values_zero_grads(causal):
    rng = np.random.default_rng(1)
    T, d = 21, 6
    q, k, do = _rand(rng, T, 2, d), _rand(rng, T, 2, d), _rand(rng, T, 2, d)
    v = np.broadcast_to(_rand(rng, 2, d), (T, 2, d)).copy()
    dq, dk, _ = attention_bwd(q, k, v, do, 0.4, causal)
    np.testing.assert_allclose(dq, 0.0, atol=1e-12)
    np.testing.assert_allclose(dk, 0.0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (4, 1)])
def test_identities(causal, Hq, Hkv):
    """Σ_j dK_j = 0, Σ_j dV_j = Σ_i dO_i (per sequence, summed over the group),
    and Σ⟨dQ, Q⟩ = Σ⟨dK, K⟩ (S is unchanged by Q→tQ, K→K/t)."""
    rng = np.random.default_rng(2)
    lens = [9, 14]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, d = int(cu[-1]), 8
    q, k, v = _rand(rng, T, Hq, d), _rand(rng, T, Hkv, d), _rand(rng, T, Hkv, d)
    do = _rand(rng, T, Hq, d)
    dq, dk, dv = attention_bwd(q, k, v, do, 0.3, causal, cu)
    g = Hq // Hkv
    for a, b in zip(cu[:-1], cu[1:]):
        np.testing.assert_allclose(dk[a:b].sum(axis=0), 0.0, atol=1e-12)
        want = do[a:b].reshape(b - a, Hkv, g, d).sum(axis=(0, 2))
        np.testing.assert_allclose(dv[a:b].sum(axis=0), want, atol=1e-12)
        lhs = np.einsum("thc,thc->", dq[a:b], q[a:b])
        rhs = np.einsum("tgc,tgc->", dk[a:b], k[a:b])
        np.testing.assert_allclose(lhs, rhs, atol=1e-11)


@pytest.mark.parametrize("causal", [False, True])
def test_finite_differences(causal):
    """Central differences of L = Σ O∘dO in float64 (h = 1e-6)."""
    rng = np.random.default_rng(3)
    lens = [4, 6]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, Hq, Hkv, d = 10, 2, 1, 3
    q, k, v = _rand(rng, T, Hq, d), _rand(rng, T, Hkv, d), _rand(rng, T, Hkv, d)
    do = _rand(rng, T, Hq, d)
    scale = 0.6
    dq, dk, dv = attention_bwd(q, k, v, do, scale, causal, cu)

    def loss(q_, k_, v_):
        o, _ = attention_fwd(q_, k_, v_, scale, causal, cu)
        return float((o * do).sum())

    h = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = loss(args["q"], args["k"], args["v"])
            args[name] = xm
            lm = loss(args["q"], args["k"], args["v"])
            num[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-8, err_msg=name)


@pytest.mark.parametrize("causal", [False, True])
def test_bruteforce_agrees(causal):
    rng = np.random.default_rng(4)
    lens = [3, 0, 7, 1]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, Hq, Hkv, d = int(cu[-1]), 4, 2, 5
    q, k, v = _rand(rng, T, Hq, d), _rand(rng, T, Hkv, d), _rand(rng, T, Hkv, 4)
    do = _rand(rng, T, Hq, 4)
    dq, dk, dv = attention_bwd(q, k, v, do, 0.5, causal, cu)
    seqs = [(int(cu[i]), int(cu[i + 1])) for i in range(len(lens))]
    bq, bk, bv = bruteforce.backward(q.tolist(), k.tolist(), v.tolist(), do.tolist(), 0.5,
                                     causal, seqs)
    np.testing.assert_allclose(dq, np.array(bq), atol=1e-12)
    np.testing.assert_allclose(dk, np.array(bk), atol=1e-12)
    np.testing.assert_allclose(dv, np.array(bv), atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_torch_cpu_autograd(causal):
    """Library special case: autograd through torch's CPU float64 SDPA."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    T, H, d = 40, 2, 16
    q, k, v, do = (_rand(rng, T, H, d) for _ in range(4))
    dq, dk, dv = attention_bwd(q, k, v, do, d ** -0.5, causal)
    tq, tk, tv = (torch.from_numpy(x).permute(1, 0, 2).unsqueeze(0).requires_grad_()
                  for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal)
    out.backward(torch.from_numpy(do).permute(1, 0, 2).unsqueeze(0))
    for mine, t in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(mine, t.grad[0].permute(1, 0, 2).numpy(), atol=1e-11)


def test_gqa_group_sum():
    """dK/dV of a KV head = sum over its query heads of MHA gradients on repeated K/V."""
    rng = np.random.default_rng(6)
    T, Hq, Hkv, d = 15, 6, 3, 4
    q, k, v, do = _rand(rng, T, Hq, d), _rand(rng, T, Hkv, d), _rand(rng, T, Hkv, d), \
        _rand(rng, T, Hq, d)
    dq, dk, dv = attention_bwd(q, k, v, do, 0.3, True)
    g = Hq // Hkv
    dq2, dk2, dv2 = attention_bwd(q, np.repeat(k, g, axis=1), np.repeat(v, g, axis=1), do,
                                  0.3, True)
    np.testing.assert_allclose(dq, dq2, atol=1e-13)
    np.testing.assert_allclose(dk, dk2.reshape(T, Hkv, g, d).sum(axis=2), atol=1e-13)
    np.testing.assert_allclose(dv, dv2.reshape(T, Hkv, g, d).sum(axis=2), atol=1e-13)


def test_sampled_matches_whole():
    rng = np.random.default_rng(7)
    lens = [11, 19]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, Hq, Hkv, d = 30, 4, 2, 8
    q, k, v, do = _rand(rng, T, Hq, d), _rand(rng, T, Hkv, d), _rand(rng, T, Hkv, d), \
        _rand(rng, T, Hq, d)
    dq, dk, dv = attention_bwd(q, k, v, do, 0.3, True, cu)
    res = attention_bwd_sampled(q, k, v, do, 0.3, True, cu, [(1, 1), (0, 0)])
    sq, sk, sv = res[(1, 1)]
    np.testing.assert_allclose(sq, dq[11:, 2:4], atol=1e-14)
    np.testing.assert_allclose(sk, dk[11:, 1], atol=1e-14)
    np.testing.assert_allclose(sv, dv[11:, 1], atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (4, 1)])
@pytest.mark.parametrize("opt", ["plain", "window", "softcap"])
def test_rows_match_whole(monkeypatch, causal, Hq, Hkv, opt):
    """attention_bwd_rows at selected query rows and key columns equals those rows
    and columns of the whole-tensor backward (itself pinned above), across
    several row blocks (a tiny block size) and two sequences of a packed batch."""
    import oracle.attention as A
    monkeypatch.setattr(A, "_BLOCK_ELEMS", 40)   # blocks of one to a few rows
    rng = np.random.default_rng(11 + Hq)
    lens = [9, 23]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, d = int(cu[-1]), 6
    q, k, v, do = _rand(rng, T, Hq, d), _rand(rng, T, Hkv, d), _rand(rng, T, Hkv, d), \
        _rand(rng, T, Hq, d)
    kw = {"plain": {}, "window": {"window": (4, 2)}, "softcap": {"softcap": 1.5}}[opt]
    dq, dk, dv = attention_bwd(q, k, v, do, 0.45, causal, cu, **kw)
    g = Hq // Hkv
    for s in range(2):
        a, L = int(cu[s]), lens[s]
        qr, kr = [0, L // 2, L - 1], [L - 1, 0, 3]
        for kvh in range(Hkv):
            rq, rk, rv = A.attention_bwd_rows(q, k, v, do, 0.45, causal, cu, s, kvh, qr, kr, **kw)
            np.testing.assert_allclose(rq, dq[a + np.array(qr), kvh * g:(kvh + 1) * g],
                                       atol=1e-13)
            np.testing.assert_allclose(rk, dk[a + np.array(kr), kvh], atol=1e-13)
            np.testing.assert_allclose(rv, dv[a + np.array(kr), kvh], atol=1e-13)


def test_rows_torch_autograd():
    """attention_bwd_rows against torch's CPU float64 autograd of plain causal GQA
    attention (an implementation that shares nothing with the oracle)."""
    torch = pytest.importorskip("torch")
    from oracle import attention_bwd_rows
    rng = np.random.default_rng(5)
    L, Hq, Hkv, d = 37, 4, 2, 8
    q, k, v, do = _rand(rng, L, Hq, d), _rand(rng, L, Hkv, d), _rand(rng, L, Hkv, d), \
        _rand(rng, L, Hq, d)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    kk = tk.repeat_interleave(Hq // Hkv, dim=1)
    vv = tv.repeat_interleave(Hq // Hkv, dim=1)
    s = torch.einsum("ihc,jhc->hij", tq, kk) * 0.3
    mask = torch.ones(L, L, dtype=torch.bool).tril()
    s = s.masked_fill(~mask, float("-inf"))
    o = torch.einsum("hij,jhc->ihc", torch.softmax(s, dim=-1), vv)
    o.backward(torch.tensor(do))
    qr, kr = [0, 5, 36], [0, 17, 36]
    for kvh in range(Hkv):
        rq, rk, rv = attention_bwd_rows(q, k, v, do, 0.3, True, None, 0, kvh, qr, kr)
        np.testing.assert_allclose(rq, tq.grad.numpy()[qr, 2 * kvh:2 * kvh + 2], atol=1e-12)
        np.testing.assert_allclose(rk, tk.grad.numpy()[kr, kvh], atol=1e-12)
        np.testing.assert_allclose(rv, tv.grad.numpy()[kr, kvh], atol=1e-12)


def test_rows_rejects_positions_outside():
    from oracle import attention_bwd_rows
    rng = np.random.default_rng(1)
    q = _rand(rng, 5, 1, 4)
    with pytest.raises(ValueError):
        attention_bwd_rows(q, q, q, q, 1.0, False, None, 0, 0, [5], [0])
