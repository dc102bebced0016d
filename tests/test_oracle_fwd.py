"""Pins for the oracle's forward: O and LSE.

Each check is something the definition (FlashAttention guide, cxbdf.cn, part 1)
or plain mathematics fixes independently of the oracle's code: hand-worked
values, closed forms, invariants, a pure-Python brute force and torch's CPU
float64 SDPA. A dropped scale, a wrong sign, a transposed operand, an
off-by-one causal mask or a wrong GQA head map each fails at least one test.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import attention_fwd, attention_probs, attention_fwd_rows, bruteforce

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")))


def _rand(rng, *shape):
    return rng.standard_normal(shape)


@pytest.mark.parametrize("case", ["full", "causal"])
def test_worked_example(case):
    c = GOLD["cases"][case]
    q = np.array([0.0, 1.0]).reshape(2, 1, 1)
    k = np.array([0.0, math.log(3.0)]).reshape(2, 1, 1)
    v = np.array([4.0, 8.0]).reshape(2, 1, 1)
    o, lse = attention_fwd(q, k, v, 1.0, c["causal"])
    np.testing.assert_allclose(o[:, 0, 0], c["o"]["values"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[0], c["lse"]["values"], rtol=0, atol=1e-14)


def test_single_token():
    rng = np.random.default_rng(0)
    q, k, v = _rand(rng, 1, 3, 5), _rand(rng, 1, 3, 5), _rand(rng, 1, 3, 7)
    for causal in (False, True):
        o, lse = attention_fwd(q, k, v, 0.3, causal)
        np.testing.assert_allclose(o, v, atol=1e-15)
        np.testing.assert_allclose(lse[:, 0], 0.3 * np.einsum("hc,hc->h", q[0], k[0]), atol=1e-14)


def test_two_tokens_logistic():
    """N=2: O_i = σ(Δ_i)·v0 + σ(−Δ_i)·v1 with Δ_i = scale·q_i·(k0 − k1)."""
    rng = np.random.default_rng(1)
    q, k, v = _rand(rng, 2, 1, 4), _rand(rng, 2, 1, 4), _rand(rng, 2, 1, 6)
    scale = 0.7
    o, lse = attention_fwd(q, k, v, scale, False)
    for i in range(2):
        delta = scale * q[i, 0] @ (k[0, 0] - k[1, 0])
        sig = 1.0 / (1.0 + math.exp(-delta))
        np.testing.assert_allclose(o[i, 0], sig * v[0, 0] + (1 - sig) * v[1, 0], atol=1e-14)
        # ln(e^{s0} + e^{s1}) = s1 − ln σ(−Δ)
        s1 = scale * q[i, 0] @ k[1, 0]
        np.testing.assert_allclose(lse[0, i], s1 - math.log(1 - sig), atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_constant_values(causal):
    rng = np.random.default_rng(2)
    T, H, d = 37, 3, 8
    q, k = _rand(rng, T, H, d), _rand(rng, T, H, d)
    row = _rand(rng, H, d)
    v = np.broadcast_to(row, (T, H, d)).copy()
    o, _ = attention_fwd(q, k, v, 0.5, causal)
    np.testing.assert_allclose(o, np.broadcast_to(row, (T, H, d)), atol=1e-13)


def test_one_dominant_key():
    """All keys zero except j*, with scale·q·k_j* = a: O = (eᵃ·V_j* + Σ_{j≠j*} V_j)/(eᵃ + n − 1)."""
    rng = np.random.default_rng(3)
    n, d, jstar, scale = 9, 4, 5, 0.25
    q = np.zeros((n, 1, d)); q[:, 0, 0] = 1.0
    k = np.zeros((n, 1, d))
    v = _rand(rng, n, 1, 3)
    for a in (0.0, 3.0, 40.0):
        k[:] = 0.0
        k[jstar, 0, 0] = a / scale
        o, lse = attention_fwd(q, k, v, scale, False)
        rest = v[:, 0].sum(axis=0) - v[jstar, 0]
        want = (math.exp(a) * v[jstar, 0] + rest) / (math.exp(a) + n - 1)
        np.testing.assert_allclose(o[:, 0], np.broadcast_to(want, (n, 3)), rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(lse[0], a + math.log1p((n - 1) * math.exp(-a)), atol=1e-13)
    # a → large: the output tends to the dominant key's value row (one-hot P)
    np.testing.assert_allclose(o[0, 0], v[jstar, 0], atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_equal_keys_lse(causal):
    """All keys equal to k: LSE_i = scale·q_i·k + ln|vis(i)|."""
    rng = np.random.default_rng(4)
    T, d, scale = 23, 6, 0.4
    q = _rand(rng, T, 1, d)
    kr = _rand(rng, d)
    k = np.broadcast_to(kr, (T, 1, d)).copy()
    v = _rand(rng, T, 1, d)
    o, lse = attention_fwd(q, k, v, scale, causal)
    count = np.arange(1, T + 1) if causal else np.full(T, T)
    np.testing.assert_allclose(lse[0], scale * q[:, 0] @ kr + np.log(count), atol=1e-13)
    # and O is the plain mean of the visible values
    cum = np.cumsum(v[:, 0], axis=0) / count[:, None] if causal else np.broadcast_to(
        v[:, 0].mean(axis=0), (T, d))
    np.testing.assert_allclose(o[:, 0], cum, atol=1e-13)


def test_causal_row_zero():
    rng = np.random.default_rng(5)
    q, k, v = _rand(rng, 19, 2, 8), _rand(rng, 19, 2, 8), _rand(rng, 19, 2, 8)
    o, lse = attention_fwd(q, k, v, 0.35, True)
    np.testing.assert_allclose(o[0], v[0], atol=1e-15)
    np.testing.assert_allclose(lse[:, 0], 0.35 * np.einsum("hc,hc->h", q[0], k[0]), atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_rows_sum_to_one(causal):
    rng = np.random.default_rng(6)
    P = attention_probs(_rand(rng, 50, 16), _rand(rng, 50, 16), 0.25, causal)
    np.testing.assert_allclose(P.sum(axis=1), 1.0, atol=1e-12)
    assert (P >= 0).all()
    if causal:
        assert np.all(np.triu(P, 1) == 0.0)


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift(causal):
    """K' = K + 1·uᵀ: O unchanged, LSE'_i = LSE_i + scale·q_i·u (large u hits the max path)."""
    rng = np.random.default_rng(7)
    T, d, scale = 41, 8, 0.3
    q, k, v = _rand(rng, T, 1, d), _rand(rng, T, 1, d), _rand(rng, T, 1, d)
    u = 300.0 * _rand(rng, d)
    o1, l1 = attention_fwd(q, k, v, scale, causal)
    o2, l2 = attention_fwd(q, k + u, v, scale, causal)
    np.testing.assert_allclose(o2, o1, atol=1e-10)
    np.testing.assert_allclose(l2[0], l1[0] + scale * q[:, 0] @ u, atol=1e-9)


def test_key_permutation_invariance():
    rng = np.random.default_rng(8)
    T = 33
    q, k, v = _rand(rng, T, 2, 8), _rand(rng, T, 2, 8), _rand(rng, T, 2, 8)
    perm = rng.permutation(T)
    o1, l1 = attention_fwd(q, k, v, 0.3, False)
    o2, l2 = attention_fwd(q, k[perm], v[perm], 0.3, False)
    np.testing.assert_allclose(o2, o1, atol=1e-13)
    np.testing.assert_allclose(l2, l1, atol=1e-13)


def test_linear_in_v():
    rng = np.random.default_rng(9)
    T = 29
    q, k = _rand(rng, T, 2, 8), _rand(rng, T, 2, 8)
    v1, v2 = _rand(rng, T, 2, 8), _rand(rng, T, 2, 8)
    for causal in (False, True):
        oa, _ = attention_fwd(q, k, 2.0 * v1 - 3.0 * v2, 0.3, causal)
        o1, _ = attention_fwd(q, k, v1, 0.3, causal)
        o2, _ = attention_fwd(q, k, v2, 0.3, causal)
        np.testing.assert_allclose(oa, 2.0 * o1 - 3.0 * o2, atol=1e-12)


def _nested(a):
    return a.tolist()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Hq,Hkv", [(1, 1), (4, 2), (3, 1)])
def test_bruteforce_agrees(causal, Hq, Hkv):
    """Pure-Python loops vs NumPy on tiny packed batches (varlen, GQA)."""
    rng = np.random.default_rng(10 + Hq)
    lens = [5, 1, 11, 0, 7]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, d = int(cu[-1]), 6
    q, k, v = _rand(rng, T, Hq, d), _rand(rng, T, Hkv, d), _rand(rng, T, Hkv, 5)
    scale = 0.45
    o, lse = attention_fwd(q, k, v, scale, causal, cu)
    seqs = [(int(cu[i]), int(cu[i + 1])) for i in range(len(lens))]
    ob, lb = bruteforce.forward(_nested(q), _nested(k), _nested(v), scale, causal, seqs)
    np.testing.assert_allclose(o, np.array(ob), atol=1e-12)
    np.testing.assert_allclose(lse, np.array(lb), atol=1e-12)


def test_varlen_is_concatenation():
    rng = np.random.default_rng(11)
    lens = [13, 4, 20]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    q, k, v = _rand(rng, T, 2, 8), _rand(rng, T, 2, 8), _rand(rng, T, 2, 8)
    o, lse = attention_fwd(q, k, v, 0.3, True, cu)
    for a, b in zip(cu[:-1], cu[1:]):
        oi, li = attention_fwd(q[a:b], k[a:b], v[a:b], 0.3, True)
        np.testing.assert_allclose(o[a:b], oi, atol=1e-14)
        np.testing.assert_allclose(lse[:, a:b], li, atol=1e-14)


def test_gqa_equals_repeated_mha():
    """Query head h uses KV head ⌊h / (Hq/Hkv)⌋: same as MHA on repeat-interleaved K/V."""
    rng = np.random.default_rng(12)
    T, Hq, Hkv = 17, 6, 2
    q, k, v = _rand(rng, T, Hq, 8), _rand(rng, T, Hkv, 8), _rand(rng, T, Hkv, 8)
    o, lse = attention_fwd(q, k, v, 0.3, True)
    kr, vr = np.repeat(k, Hq // Hkv, axis=1), np.repeat(v, Hq // Hkv, axis=1)
    o2, lse2 = attention_fwd(q, kr, vr, 0.3, True)
    np.testing.assert_allclose(o, o2, atol=1e-14)
    np.testing.assert_allclose(lse, lse2, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_torch_cpu_sdpa(causal):
    """Library special case: torch's CPU float64 scaled_dot_product_attention."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(13)
    T, H, d = 70, 3, 16
    q, k, v = _rand(rng, T, H, d), _rand(rng, T, H, d), _rand(rng, T, H, d)
    o, _ = attention_fwd(q, k, v, d ** -0.5, causal)
    tq, tk, tv = (torch.from_numpy(x).permute(1, 0, 2).unsqueeze(0) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal)
    np.testing.assert_allclose(o, ref[0].permute(1, 0, 2).numpy(), atol=1e-12)


def test_rows_helper_matches_whole():
    rng = np.random.default_rng(14)
    lens = [30, 45]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v = _rand(rng, 75, 4, 8), _rand(rng, 75, 2, 8), _rand(rng, 75, 2, 8)
    o, lse = attention_fwd(q, k, v, 0.3, True, cu)
    rows = [0, 7, 44]
    orow, lrow = attention_fwd_rows(q, k, v, 0.3, True, cu, 1, 3, rows)
    np.testing.assert_allclose(orow, o[30 + np.array(rows), 3], atol=1e-14)
    np.testing.assert_allclose(lrow, lse[3, 30 + np.array(rows)], atol=1e-14)


def test_row_blocks_are_whole_rows(monkeypatch):
    """Splitting into row blocks must not change anything (blocks hold whole rows)."""
    import oracle.attention as A
    rng = np.random.default_rng(15)
    q, k, v = _rand(rng, 64, 1, 8), _rand(rng, 64, 1, 8), _rand(rng, 64, 1, 8)
    o1, l1 = attention_fwd(q, k, v, 0.3, True)
    monkeypatch.setattr(A, "_BLOCK_ELEMS", 64 * 3)
    o2, l2 = attention_fwd(q, k, v, 0.3, True)
    np.testing.assert_allclose(o2, o1, atol=1e-15)
    np.testing.assert_allclose(l2, l1, atol=1e-15)
