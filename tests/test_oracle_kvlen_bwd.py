"""Pins for the backward of attention with queries and keys of different
lengths (oracle.decode.kvlen_head_bwd / kvlen_bwd).

The queries of a sequence sit at its last Lq key positions (bottom-right
causal alignment, the forward oracle kvcache_head). Checks fixed
independently of the function's code: equality with the pinned full-sequence
backward when Lq = Lk; central finite differences of the pinned forward;
torch's CPU float64 autograd with an explicit bottom-right mask; queries that
see no key (zero dQ, no effect on dK and dV); the identities Σ_j dK_j = 0 and
Σ_j dV_j = Σ_i dO_i over the rows that see a key; empty sides.
"""
import numpy as np
import pytest

from oracle import attention_bwd
from oracle.decode import kvcache_head, kvlen_bwd, kvlen_head_bwd


def _rand(rng, *shape):
    return rng.standard_normal(shape)


@pytest.mark.parametrize("causal", [False, True])
def test_equal_lengths_is_the_full_backward(causal):
    rng = np.random.default_rng(3)
    lens = [7, 12]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, Hq, Hkv, d = int(cu[-1]), 4, 2, 5
    q, k, v, do = _rand(rng, T, Hq, d), _rand(rng, T, Hkv, d), _rand(rng, T, Hkv, d), \
        _rand(rng, T, Hq, d)
    want = attention_bwd(q, k, v, do, 0.4, causal, cu)
    got = kvlen_bwd(q, k, v, do, 0.4, causal, cu, cu)
    for a, b in zip(got, want):
        np.testing.assert_allclose(a, b, atol=1e-13)


def _loss_grad_fd(Q, K, V, dO, scale, causal, h=1e-6):
    """Central differences of L = Σ O∘dO (O from the pinned forward oracle)."""
    def loss(Qx, Kx, Vx):
        O, _ = kvcache_head(Qx, Kx, Vx, scale, causal)
        return float((O * dO).sum())
    grads = []
    for idx, X in enumerate((Q, K, V)):
        G = np.zeros_like(X)
        for pos in np.ndindex(X.shape):
            Xp, Xm = X.copy(), X.copy()
            Xp[pos] += h
            Xm[pos] -= h
            args_p = [Q, K, V]
            args_m = [Q, K, V]
            args_p[idx], args_m[idx] = Xp, Xm
            G[pos] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        grads.append(G)
    return grads


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Lq,Lk", [(3, 7), (6, 4), (5, 5), (1, 6)])
def test_finite_differences(causal, Lq, Lk):
    rng = np.random.default_rng(10 * Lq + Lk)
    d = 3
    Q, K, V, dO = _rand(rng, Lq, d), _rand(rng, Lk, d), _rand(rng, Lk, d), _rand(rng, Lq, d)
    got = kvlen_head_bwd(Q, K, V, dO, 0.7, causal)
    for g, fd, n in zip(got, _loss_grad_fd(Q, K, V, dO, 0.7, causal), "QKV"):
        np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-7, err_msg=f"d{n}")


@pytest.mark.parametrize("causal", [False, True])
def test_torch_autograd(causal):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(17)
    Lq, Lk, Hq, Hkv, d = 9, 21, 4, 2, 6
    q, k, v, do = _rand(rng, Lq, Hq, d), _rand(rng, Lk, Hkv, d), _rand(rng, Lk, Hkv, d), \
        _rand(rng, Lq, Hq, d)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    kk = tk.repeat_interleave(Hq // Hkv, dim=1)
    vv = tv.repeat_interleave(Hq // Hkv, dim=1)
    s = torch.einsum("ihc,jhc->hij", tq, kk) * 0.35
    if causal:   # query i at position Lk - Lq + i sees keys j <= that position
        mask = torch.arange(Lk)[None, :] <= (Lk - Lq + torch.arange(Lq))[:, None]
        s = s.masked_fill(~mask, float("-inf"))
    o = torch.einsum("hij,jhc->ihc", torch.softmax(s, dim=-1), vv)
    o.backward(torch.tensor(do))
    dq, dk, dv = kvlen_bwd(q, k, v, do, 0.35, causal, [0, Lq], [0, Lk])
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)


def test_rows_without_keys():
    """Causal with Lq > Lk: the first Lq - Lk queries see nothing. Their dQ is
    exactly 0 and dropping them leaves dK and dV unchanged."""
    rng = np.random.default_rng(5)
    Lq, Lk, d = 8, 3, 4
    Q, K, V, dO = _rand(rng, Lq, d), _rand(rng, Lk, d), _rand(rng, Lk, d), _rand(rng, Lq, d)
    dQ, dK, dV = kvlen_head_bwd(Q, K, V, dO, 0.6, True)
    assert (dQ[:Lq - Lk] == 0).all()
    dQ2, dK2, dV2 = kvlen_head_bwd(Q[Lq - Lk:], K, V, dO[Lq - Lk:], 0.6, True)
    np.testing.assert_allclose(dQ[Lq - Lk:], dQ2, atol=1e-14)
    np.testing.assert_allclose(dK, dK2, atol=1e-14)
    np.testing.assert_allclose(dV, dV2, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_identities(causal):
    rng = np.random.default_rng(8)
    Lq, Lk, d = 11, 29, 5
    Q, K, V, dO = _rand(rng, Lq, d), _rand(rng, Lk, d), _rand(rng, Lk, d), _rand(rng, Lq, d)
    dQ, dK, dV = kvlen_head_bwd(Q, K, V, dO, 0.5, causal)
    np.testing.assert_allclose(dK.sum(axis=0), 0.0, atol=1e-12)
    np.testing.assert_allclose(dV.sum(axis=0), dO.sum(axis=0), atol=1e-12)


def test_empty_sides():
    rng = np.random.default_rng(2)
    d = 3
    for Lq, Lk in ((0, 4), (4, 0), (0, 0)):
        Q, K, V, dO = _rand(rng, Lq, d), _rand(rng, Lk, d), _rand(rng, Lk, d), _rand(rng, Lq, d)
        for g in kvlen_head_bwd(Q, K, V, dO, 0.5, True):
            assert (g == 0).all()
    with pytest.raises(ValueError):
        kvlen_bwd(np.zeros((2, 3, 4)), np.zeros((2, 2, 4)), np.zeros((2, 2, 4)),
                  np.zeros((2, 3, 4)), 1.0, True, [0, 2], [0, 2])
