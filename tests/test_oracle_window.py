"""Pins for the oracle's sliding-window (band) mask: query i sees keys
i − wl .. i + wr of its own sequence (a negative bound is unbounded).

The band mask is the "sliding window" mask that the mlqm.cn page (section 四,
mask types) names among the masks of standard attention. Checks fixed
independently of the oracle's code: the bounds that reduce to the full and
causal masks, closed forms for windows of one and two keys, a pure-Python
brute force, torch's CPU float64 SDPA with an explicit boolean band mask
(forward and autograd), central finite differences and invariants. Swapped
bounds, an off-by-one in either bound or a mask applied to the wrong axis
each fails at least one test.
"""
import math

import numpy as np
import pytest

from oracle import attention_bwd, attention_fwd, attention_probs, bruteforce


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _qkv(seed, T, Hq=2, Hkv=2, d=6, dv=5):
    rng = np.random.default_rng(seed)
    return _rand(rng, T, Hq, d), _rand(rng, T, Hkv, d), _rand(rng, T, Hkv, dv)


@pytest.mark.parametrize("causal", [False, True])
def test_unbounded_window_is_the_plain_mask(causal):
    q, k, v = _qkv(1, 23)
    o, lse = attention_fwd(q, k, v, 0.4, causal)
    for w in ((-1, -1), (23, 23), (100, -1), (-1, 40)):
        ow, lw = attention_fwd(q, k, v, 0.4, causal, window=w)
        np.testing.assert_allclose(ow, o, atol=1e-14, err_msg=str(w))
        np.testing.assert_allclose(lw, lse, atol=1e-14, err_msg=str(w))


def test_right_bound_zero_is_causal():
    q, k, v = _qkv(2, 19)
    oc, lc = attention_fwd(q, k, v, 0.4, True)
    ow, lw = attention_fwd(q, k, v, 0.4, False, window=(-1, 0))
    np.testing.assert_allclose(ow, oc, atol=1e-14)
    np.testing.assert_allclose(lw, lc, atol=1e-14)


def test_window_of_one_key():
    """(0, 0): each query sees only its own position: O_i = V_i, LSE_i = scale·q_i·k_i."""
    q, k, v = _qkv(3, 9, Hq=4, Hkv=2)
    o, lse = attention_fwd(q, k, v, 0.7, False, window=(0, 0))
    g = 2
    for h in range(4):
        np.testing.assert_allclose(o[:, h], v[:, h // g], atol=1e-15)
        np.testing.assert_allclose(lse[h], 0.7 * np.einsum("tc,tc->t", q[:, h], k[:, h // g]),
                                   atol=1e-14)


@pytest.mark.parametrize("side", ["left", "right"])
def test_window_of_two_keys(side):
    """(1, 0): keys i−1, i; (0, 1): keys i, i+1 — a two-way softmax, O = σ(Δ)·v_a + σ(−Δ)·v_b."""
    q, k, v = _qkv(4, 8, Hq=1, Hkv=1)
    scale = 0.8
    w = (1, 0) if side == "left" else (0, 1)
    o, lse = attention_fwd(q, k, v, scale, False, window=w)
    L = q.shape[0]
    for i in range(L):
        other = i - 1 if side == "left" else i + 1
        if not 0 <= other < L:            # the band runs off the sequence: one key
            np.testing.assert_allclose(o[i, 0], v[i, 0], atol=1e-15)
            continue
        delta = scale * q[i, 0] @ (k[other, 0] - k[i, 0])
        sig = 1.0 / (1.0 + math.exp(-delta))
        np.testing.assert_allclose(o[i, 0], sig * v[other, 0] + (1 - sig) * v[i, 0], atol=1e-14)
        s_i = scale * q[i, 0] @ k[i, 0]
        np.testing.assert_allclose(lse[0, i], s_i - math.log(1 - sig), atol=1e-13)


@pytest.mark.parametrize("w", [(2, 3), (5, 0), (0, 4)])
def test_probs_live_on_the_band(w):
    q, k, _ = _qkv(5, 17, Hq=1, Hkv=1)
    P = attention_probs(q[:, 0], k[:, 0], 0.5, False, window=w)
    i, j = np.meshgrid(np.arange(17), np.arange(17), indexing="ij")
    band = (j >= i - w[0]) & (j <= i + w[1])
    assert np.all(P[~band] == 0.0)
    assert np.all(P[band] > 0.0)
    np.testing.assert_allclose(P.sum(axis=1), 1.0, atol=1e-14)


def test_constant_values():
    q, k, v = _qkv(6, 13, Hq=2, Hkv=1)
    v[:] = v[:1]
    o, _ = attention_fwd(q, k, v, 0.5, True, window=(3, 0))
    np.testing.assert_allclose(o, np.broadcast_to(v[:1], o.shape), atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("w", [(0, 0), (2, 1), (3, -1), (-1, 2), (4, 0)])
def test_bruteforce_agrees(causal, w):
    """Pure-Python loops vs NumPy on tiny packed batches (varlen, GQA), both passes."""
    rng = np.random.default_rng(7)
    lens = [5, 1, 11, 0, 7]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, Hq, Hkv, d = int(cu[-1]), 4, 2, 5
    q, k, v = _rand(rng, T, Hq, d), _rand(rng, T, Hkv, d), _rand(rng, T, Hkv, 4)
    do = _rand(rng, T, Hq, 4)
    seqs = [(int(cu[i]), int(cu[i + 1])) for i in range(len(lens))]
    o, lse = attention_fwd(q, k, v, 0.45, causal, cu, window=w)
    ob, lb = bruteforce.forward(q.tolist(), k.tolist(), v.tolist(), 0.45, causal, seqs, window=w)
    np.testing.assert_allclose(o, np.array(ob), atol=1e-12)
    np.testing.assert_allclose(lse, np.array(lb), atol=1e-12)
    dq, dk, dv = attention_bwd(q, k, v, do, 0.45, causal, cu, window=w)
    bq, bk, bv = bruteforce.backward(q.tolist(), k.tolist(), v.tolist(), do.tolist(), 0.45,
                                     causal, seqs, window=w)
    np.testing.assert_allclose(dq, np.array(bq), atol=1e-12)
    np.testing.assert_allclose(dk, np.array(bk), atol=1e-12)
    np.testing.assert_allclose(dv, np.array(bv), atol=1e-12)


@pytest.mark.parametrize("w", [(3, 5), (7, 0), (0, 2)])
def test_torch_cpu_sdpa_band_mask(w):
    """Library special case: torch's CPU float64 SDPA with a boolean band mask, and its autograd."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(8)
    T, H, d = 40, 2, 16
    q, k, v, do = (_rand(rng, T, H, d) for _ in range(4))
    o, lse = attention_fwd(q, k, v, d ** -0.5, False, window=w)
    dq, dk, dv = attention_bwd(q, k, v, do, d ** -0.5, False, window=w)
    i, j = torch.meshgrid(torch.arange(T), torch.arange(T), indexing="ij")
    mask = (j >= i - w[0]) & (j <= i + w[1])
    tq, tk, tv = (torch.from_numpy(x).permute(1, 0, 2).unsqueeze(0).requires_grad_()
                  for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask)
    np.testing.assert_allclose(o, out[0].permute(1, 0, 2).detach().numpy(), atol=1e-12)
    out.backward(torch.from_numpy(do).permute(1, 0, 2).unsqueeze(0))
    for mine, t in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(mine, t.grad[0].permute(1, 0, 2).numpy(), atol=1e-11)


def test_finite_differences():
    """Central differences of Σ O∘dO in float64 (h = 1e-6) under a band mask."""
    rng = np.random.default_rng(9)
    lens = [5, 6]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, Hq, Hkv, d = 11, 2, 1, 3
    q, k, v = _rand(rng, T, Hq, d), _rand(rng, T, Hkv, d), _rand(rng, T, Hkv, d)
    do = _rand(rng, T, Hq, d)
    w, scale = (2, 1), 0.6
    dq, dk, dv = attention_bwd(q, k, v, do, scale, False, cu, window=w)

    def loss(q_, k_, v_):
        o, _ = attention_fwd(q_, k_, v_, scale, False, cu, window=w)
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


def test_gradient_identities():
    """Rows of dS sum to zero (Σ_j dK_j = 0); rows of P sum to one (Σ_j dV_j = Σ_i dO_i)."""
    q, k, v = _qkv(10, 21, Hq=2, Hkv=2)
    do = np.random.default_rng(11).standard_normal((21, 2, 5))
    dq, dk, dv = attention_bwd(q, k, v, do, 0.5, True, window=(4, 0))
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=0), atol=1e-12)
