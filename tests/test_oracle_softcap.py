"""Pins for the oracle's soft cap: logits c·tanh(scale·q·k / c) before the softmax.

The FlashAttention-2 page (blog.gitcode.com, section 2.3) adds a soft-cap
step; its printed formula is neither bounded nor continuous, so the oracle takes
the bounded tanh form. Checks fixed independently of the oracle's code: a cap
far above every logit reduces to plain attention (tanh x ≈ x); a cap far below
makes every visible logit ≈ 0, so O is the mean of the visible values;
closed forms for one and two keys; |logit| ≤ c bounds the LSE; a pure-Python
brute force of both passes; central finite differences of the backward (the
1 − tanh² factor); Σ_j dV_j = Σ_i dO_i. Dropping the 1 − tanh² factor, capping
before the scale, or capping with c·tanh(x) instead of c·tanh(x/c) each fails
at least one test.
"""
import math

import numpy as np
import pytest

from oracle import attention_bwd, attention_fwd, bruteforce


def _qkv(seed, T, Hq=2, Hkv=2, d=6, dv=5, amp=1.0):
    rng = np.random.default_rng(seed)
    return (amp * rng.standard_normal((T, Hq, d)), amp * rng.standard_normal((T, Hkv, d)),
            rng.standard_normal((T, Hkv, dv)))


@pytest.mark.parametrize("causal", [False, True])
def test_huge_cap_is_plain_attention(causal):
    q, k, v = _qkv(1, 25)
    o, lse = attention_fwd(q, k, v, 0.4, causal)
    oc, lc = attention_fwd(q, k, v, 0.4, causal, softcap=1e7)
    np.testing.assert_allclose(oc, o, atol=1e-11)
    np.testing.assert_allclose(lc, lse, atol=1e-11)
    do = np.random.default_rng(2).standard_normal(o.shape)
    for a, b in zip(attention_bwd(q, k, v, do, 0.4, causal, softcap=1e7),
                    attention_bwd(q, k, v, do, 0.4, causal)):
        np.testing.assert_allclose(a, b, atol=1e-10)


def test_tiny_cap_averages_the_visible_values():
    q, k, v = _qkv(3, 17, amp=3.0)
    o, lse = attention_fwd(q, k, v, 0.5, True, softcap=1e-9)
    for i in range(17):
        np.testing.assert_allclose(o[i], v[: i + 1].mean(axis=0), atol=1e-8)
        np.testing.assert_allclose(lse[:, i], math.log(i + 1), atol=1e-8)


def test_single_key_closed_form():
    q, k, v = _qkv(4, 1, Hq=3, Hkv=1, amp=4.0)
    cap, scale = 2.5, 0.7
    o, lse = attention_fwd(q, k, v, scale, False, softcap=cap)
    for h in range(3):
        np.testing.assert_allclose(o[0, h], v[0, 0], atol=1e-15)
        x = scale * float(q[0, h] @ k[0, 0])
        assert lse[h, 0] == pytest.approx(cap * math.tanh(x / cap), abs=1e-13)


def test_two_keys_closed_form():
    """Two visible keys: O = σ(Δ)·v_1 + σ(−Δ)·v_0 with Δ the difference of capped logits."""
    q, k, v = _qkv(5, 2, Hq=1, Hkv=1, amp=3.0)
    cap, scale = 1.5, 0.9
    o, _ = attention_fwd(q, k, v, scale, False, softcap=cap)
    for i in range(2):
        z = [cap * math.tanh(scale * float(q[i, 0] @ k[j, 0]) / cap) for j in range(2)]
        sig = 1.0 / (1.0 + math.exp(-(z[1] - z[0])))
        np.testing.assert_allclose(o[i, 0], sig * v[1, 0] + (1 - sig) * v[0, 0], atol=1e-14)


def test_lse_bounded_by_the_cap():
    q, k, v = _qkv(6, 40, amp=10.0)
    cap = 3.0
    _, lse = attention_fwd(q, k, v, 1.0, True, softcap=cap)
    n = np.arange(1, 41)
    assert np.all(lse <= cap + np.log(n) + 1e-12)
    assert np.all(lse >= -cap + np.log(n) - 1e-12)
    assert lse.max() > cap + np.log(n).max() - 1.0     # the cap is actually reached


@pytest.mark.parametrize("causal", [False, True])
def test_bruteforce_agrees(causal):
    rng = np.random.default_rng(7)
    lens = [5, 1, 9, 0, 6]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, Hq, Hkv, d = int(cu[-1]), 4, 2, 5
    q, k = 2 * rng.standard_normal((T, Hq, d)), 2 * rng.standard_normal((T, Hkv, d))
    v, do = rng.standard_normal((T, Hkv, 4)), rng.standard_normal((T, Hq, 4))
    seqs = [(int(cu[i]), int(cu[i + 1])) for i in range(len(lens))]
    o, lse = attention_fwd(q, k, v, 0.45, causal, cu, softcap=1.7)
    ob, lb = bruteforce.forward(q.tolist(), k.tolist(), v.tolist(), 0.45, causal, seqs,
                                softcap=1.7)
    np.testing.assert_allclose(o, np.array(ob), atol=1e-12)
    np.testing.assert_allclose(lse, np.array(lb), atol=1e-12)
    got = attention_bwd(q, k, v, do, 0.45, causal, cu, softcap=1.7)
    ref = bruteforce.backward(q.tolist(), k.tolist(), v.tolist(), do.tolist(), 0.45, causal,
                              seqs, softcap=1.7)
    for a, b in zip(got, ref):
        np.testing.assert_allclose(a, np.array(b), atol=1e-12)


def test_finite_differences():
    """Central differences of Σ O∘dO in float64 (h = 1e-6), logits well into the cap."""
    rng = np.random.default_rng(9)
    lens = [5, 6]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, Hq, Hkv, d = 11, 2, 1, 3
    q, k = 2 * rng.standard_normal((T, Hq, d)), 2 * rng.standard_normal((T, Hkv, d))
    v, do = rng.standard_normal((T, Hkv, d)), rng.standard_normal((T, Hq, d))
    scale, cap = 0.8, 1.2
    dq, dk, dv = attention_bwd(q, k, v, do, scale, True, cu, softcap=cap)

    def loss(q_, k_, v_):
        o, _ = attention_fwd(q_, k_, v_, scale, True, cu, softcap=cap)
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


def test_dv_identity():
    q, k, v = _qkv(10, 21, amp=2.0)
    do = np.random.default_rng(11).standard_normal((21, 2, 5))
    _, _, dv = attention_bwd(q, k, v, do, 0.5, True, softcap=0.8)
    np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=0), atol=1e-12)
