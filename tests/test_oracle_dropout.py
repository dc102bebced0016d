"""Pins for the dropout oracle: the Philox4x32-10 generator, the keep decisions
built on it, and attention with dropout on the softmax weights.

The generator is pinned by the published known-answer vectors of Philox4x32-10
(tests/golden/philox4x32_10_kat.json, cited there), in both the NumPy version
and the pure-Python one written separately. The keep decisions by their
frequency (t/256 within binomial bounds) and by their counter layout (4 x 4
blocks per call; heads and sequences see different bits). Attention by:
p = 0 reduces to plain attention; the average over many seeds tends to plain
attention (the 256/t scaling is unbiased); the brute force of both passes;
central finite differences at a fixed seed; D_i = dO_i · O_i.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import (attention_bwd, attention_bwd_dropout, attention_fwd, attention_fwd_dropout,
                    bruteforce, keep_mask, keep_threshold, philox4x32_10)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.json")


def _kat():
    return json.load(open(GOLDEN))["vectors"]


@pytest.mark.parametrize("vec", _kat())
def test_philox_known_answers_numpy(vec):
    ctr = [int(x, 16) for x in vec["ctr"]]
    key = [int(x, 16) for x in vec["key"]]
    out = [int(x) for x in philox4x32_10(ctr, key)]
    assert out == [int(x, 16) for x in vec["out"]]


@pytest.mark.parametrize("vec", _kat())
def test_philox_known_answers_pure_python(vec):
    ctr = [int(x, 16) for x in vec["ctr"]]
    key = [int(x, 16) for x in vec["key"]]
    assert list(bruteforce.philox4x32_10(*ctr, *key)) == [int(x, 16) for x in vec["out"]]


def test_philox_vectorised_matches_scalar():
    rng = np.random.default_rng(1)
    c = rng.integers(0, 2 ** 32, size=(4, 50), dtype=np.uint64)
    k = (0x12345678, 0x9ABCDEF0)
    vec = philox4x32_10(list(c), k)
    for n in range(50):
        ref = bruteforce.philox4x32_10(*(int(c[r, n]) for r in range(4)), *k)
        assert tuple(int(w[n]) for w in vec) == ref


@pytest.mark.parametrize("p,t", [(0.0, 256), (0.1, 230), (0.5, 128), (0.25, 192), (0.998, 1),
                                 (1.5 / 256, 255), (2.5 / 256, 254)])   # halves round up
def test_keep_threshold(p, t):
    assert keep_threshold(p) == t


@pytest.mark.parametrize("p", [-0.1, 1.0, 0.999, float("nan")])
def test_keep_threshold_rejects(p):
    with pytest.raises(ValueError):
        keep_threshold(p)


@pytest.mark.parametrize("t", [26, 128, 230])
def test_keep_frequency(t):
    m = keep_mask(77, 3, 5, np.arange(512), np.arange(512), t)
    n = m.size
    mean, sd = n * t / 256, math.sqrt(n * (t / 256) * (1 - t / 256))
    assert abs(m.sum() - mean) < 5 * sd


def test_mask_layout():
    """One generator call per 4 x 4 block: recomputing any sub-block from its own
    rows/columns gives the same bits, and heads/sequences/seeds differ."""
    full = keep_mask(5, 1, 2, np.arange(64), np.arange(64), 128)
    sub = keep_mask(5, 1, 2, np.arange(12, 20), np.arange(33, 47), 128)
    np.testing.assert_array_equal(sub, full[12:20, 33:47])
    for other in (keep_mask(5, 1, 3, np.arange(64), np.arange(64), 128),
                  keep_mask(5, 2, 2, np.arange(64), np.arange(64), 128),
                  keep_mask(6, 1, 2, np.arange(64), np.arange(64), 128)):
        assert 0.3 < np.mean(other != full) < 0.7
    # the element's byte: word i mod 4, byte j mod 4 of the call for (j/4, i/4, head, seq)
    i, j = 13, 42
    w = bruteforce.philox4x32_10(j // 4, i // 4, 2, 1, 5, 0)
    assert full[i, j] == (((w[i % 4] >> (8 * (j % 4))) & 0xFF) < 128)


def _data(seed, T, Hq=2, Hkv=1, d=6):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((T, Hq, d)), rng.standard_normal((T, Hkv, d)),
            rng.standard_normal((T, Hkv, d)), rng.standard_normal((T, Hq, d)))


def test_zero_dropout_is_plain_attention():
    q, k, v, do = _data(2, 30)
    o, lse = attention_fwd(q, k, v, 0.4, True)
    od, ld = attention_fwd_dropout(q, k, v, 0.4, True, None, 0.0, 123)
    np.testing.assert_allclose(od, o, atol=1e-14)
    np.testing.assert_allclose(ld, lse, atol=1e-14)
    for a, b in zip(attention_bwd_dropout(q, k, v, do, 0.4, True, None, 0.0, 123),
                    attention_bwd(q, k, v, do, 0.4, True)):
        np.testing.assert_allclose(a, b, atol=1e-13)


def test_unbiased_over_seeds():
    """E_seed[O_dropout] = O: the mean over 800 seeds is within 5 standard errors."""
    q, k, v, _ = _data(3, 12, Hq=1, d=4)
    o, lse = attention_fwd(q, k, v, 0.7, False)
    outs = np.stack([attention_fwd_dropout(q, k, v, 0.7, False, None, 0.5, s)[0]
                     for s in range(800)])
    mean, se = outs.mean(axis=0), outs.std(axis=0) / math.sqrt(800)
    assert np.all(np.abs(mean - o) < 5 * se + 1e-12)
    np.testing.assert_allclose(attention_fwd_dropout(q, k, v, 0.7, False, None, 0.5, 9)[1], lse)


@pytest.mark.parametrize("causal", [False, True])
def test_bruteforce_agrees(causal):
    rng = np.random.default_rng(7)
    lens = [5, 1, 9, 0, 6]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, Hq, Hkv, d = int(cu[-1]), 4, 2, 5
    q, k = rng.standard_normal((T, Hq, d)), rng.standard_normal((T, Hkv, d))
    v, do = rng.standard_normal((T, Hkv, 4)), rng.standard_normal((T, Hq, 4))
    seqs = [(int(cu[i]), int(cu[i + 1])) for i in range(len(lens))]
    seed = 0xDEADBEEF12345
    o, lse = attention_fwd_dropout(q, k, v, 0.45, causal, cu, 0.3, seed)
    ob, lb = bruteforce.forward_dropout(q.tolist(), k.tolist(), v.tolist(), 0.45, causal, seqs,
                                        keep_threshold(0.3), seed)
    np.testing.assert_allclose(o, np.array(ob), atol=1e-12)
    np.testing.assert_allclose(lse, np.array(lb), atol=1e-12)
    got = attention_bwd_dropout(q, k, v, do, 0.45, causal, cu, 0.3, seed)
    ref = bruteforce.backward_dropout(q.tolist(), k.tolist(), v.tolist(), do.tolist(), 0.45,
                                      causal, seqs, keep_threshold(0.3), seed)
    for a, b in zip(got, ref):
        np.testing.assert_allclose(a, np.array(b), atol=1e-12)


def test_finite_differences():
    """Central differences of Σ O∘dO at a fixed seed (the mask does not depend on q, k, v)."""
    q, k, v, do = _data(9, 11, Hq=2, Hkv=1, d=3)
    cu = np.array([0, 5, 11])
    scale, p, seed = 0.6, 0.4, 31337
    dq, dk, dv = attention_bwd_dropout(q, k, v, do, scale, True, cu, p, seed)

    def loss(q_, k_, v_):
        o, _ = attention_fwd_dropout(q_, k_, v_, scale, True, cu, p, seed)
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


def test_delta_is_do_dot_o():
    """The backward's D_i = Σ_j P Z dP equals dO_i · O_i of the dropout output."""
    q, k, v, do = _data(10, 20, Hq=1, d=5)
    o, _ = attention_fwd_dropout(q, k, v, 0.5, False, None, 0.2, 77)
    from oracle.attention import _lse, _scores
    from oracle.dropout import keep_mask as km
    S = _scores(q[:, 0], np.arange(20), k[:, 0], 0.5, False)
    P = np.exp(S - _lse(S)[:, None])
    Z = km(77, 0, 0, np.arange(20), np.arange(20), keep_threshold(0.2)) * (256 / keep_threshold(0.2))
    D = (P * Z * (do[:, 0] @ v[:, 0].T)).sum(axis=1)
    np.testing.assert_allclose(D, (do[:, 0] * o[:, 0]).sum(axis=1), atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_rows_match_whole(monkeypatch, causal):
    """head_fwd_dropout(rows=...) equals those rows of attention_fwd_dropout
    (pinned above), across row blocks of a few rows, in the second sequence of a
    packed batch and for the second head of a GQA group (so the generator's
    sequence, head and row counters all differ from 0)."""
    import oracle.attention as A
    from oracle import head_fwd_dropout
    monkeypatch.setattr(A, "_BLOCK_ELEMS", 50)
    rng = np.random.default_rng(8)
    lens = [13, 29]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, Hq, Hkv, d = int(cu[-1]), 4, 2, 5
    q, k, v = (rng.standard_normal((T, H, d)) for H in (Hq, Hkv, Hkv))
    o, lse = attention_fwd_dropout(q, k, v, 0.6, causal, cu, 0.3, 2 ** 40 + 77)
    rows = [28, 0, 5, 17, 4]
    a = int(cu[1])
    O, L = head_fwd_dropout(q[a:, 3], k[a:, 1], v[a:, 1], 0.6, causal, 1, 3, 0.3, 2 ** 40 + 77,
                            rows=rows)
    np.testing.assert_allclose(O, o[a + np.array(rows), 3], atol=1e-14)
    np.testing.assert_allclose(L, lse[3, a + np.array(rows)], atol=1e-14)
