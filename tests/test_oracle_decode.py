"""Pins for the decode (key/value cache) oracle.

Checks fixed independently of oracle.decode's code: the hand-worked example of
tests/golden (the decode of the last token of that two-token sequence), the
pure-Python brute force on tiny caches, the already-pinned full-sequence
oracle when the queries are the whole sequence, closed forms (constant V,
a single visible key, empty rows) and the exact merge of two key ranges by
their log-sum-exp. A wrong query position, an off-by-one causal limit, a
wrong GQA head map or a missing scale each fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import attention_fwd, bruteforce, kvcache_fwd

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")))


def _cache(rng, B, Nq, Nk, Hq, Hkv, d):
    q = rng.standard_normal((B, Nq, Hq, d))
    k = rng.standard_normal((B, Nk, Hkv, d))
    v = rng.standard_normal((B, Nk, Hkv, d))
    return q, k, v


@pytest.mark.parametrize("causal", [False, True])
def test_worked_example_last_token(causal):
    """Decoding token 1 of the worked example over a 2-entry cache gives that row's O, LSE."""
    q = np.array([1.0]).reshape(1, 1, 1, 1)
    k = np.array([0.0, math.log(3.0)]).reshape(1, 2, 1, 1)
    v = np.array([4.0, 8.0]).reshape(1, 2, 1, 1)
    o, lse = kvcache_fwd(q, k, v, [2], 1.0, causal)
    c = GOLD["cases"]["causal" if causal else "full"]
    assert o[0, 0, 0, 0] == pytest.approx(c["o"]["values"][1], abs=1e-14)
    assert lse[0, 0] == pytest.approx(c["lse"]["values"][1], abs=1e-14)


def test_worked_example_two_queries_causal():
    q = np.array([0.0, 1.0]).reshape(1, 2, 1, 1)
    k = np.array([0.0, math.log(3.0), 5.0]).reshape(1, 3, 1, 1)   # third slot past the valid length
    v = np.array([4.0, 8.0, -1.0]).reshape(1, 3, 1, 1)
    o, lse = kvcache_fwd(q, k, v, [2], 1.0, True)
    c = GOLD["cases"]["causal"]
    np.testing.assert_allclose(o[0, :, 0, 0], c["o"]["values"], atol=1e-14)
    np.testing.assert_allclose(lse[0], c["lse"]["values"], atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(2, 1, 5, 4, 2, 3), (3, 3, 6, 2, 1, 4), (2, 4, 4, 4, 4, 2)])
def test_bruteforce(causal, shape):
    B, Nq, Nk, Hq, Hkv, d = shape
    rng = np.random.default_rng(sum(shape) + causal)
    q, k, v = _cache(rng, B, Nq, Nk, Hq, Hkv, d)
    lens = [int(x) for x in rng.integers(0, Nk, size=B, endpoint=True)]
    lens[0] = Nk
    lens[-1] = min(1, Nk)          # a one-entry cache: causal rows before it see nothing
    scale = 0.37
    o, lse = kvcache_fwd(q, k, v, lens, scale, causal)
    ob, lb = bruteforce.forward_kvcache(q.tolist(), k.tolist(), v.tolist(), lens, scale, causal)
    for b in range(B):
        for i in range(Nq):
            for h in range(Hq):
                np.testing.assert_allclose(o[b, i, h], ob[b][i][h], atol=1e-12)
                want = lb[b][i][h]
                got = lse[h, b * Nq + i]
                if math.isinf(want):
                    assert math.isinf(got) and got < 0
                else:
                    assert got == pytest.approx(want, abs=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_queries_are_the_whole_sequence(causal):
    """Nq = L: the decode result is the full-sequence attention (pinned separately)."""
    rng = np.random.default_rng(7)
    B, L, Hq, Hkv, d = 2, 9, 4, 2, 8
    q, k, v = _cache(rng, B, L, L, Hq, Hkv, d)
    o, lse = kvcache_fwd(q, k, v, [L] * B, 0.5, causal)
    cu = np.arange(B + 1) * L
    of, lf = attention_fwd(q.reshape(B * L, Hq, d), k.reshape(B * L, Hkv, d),
                           v.reshape(B * L, Hkv, d), 0.5, causal, cu)
    np.testing.assert_allclose(o.reshape(B * L, Hq, d), of, atol=1e-12)
    np.testing.assert_allclose(lse, lf, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("wl,cap", [(3, None), (None, 2.0), (2, 1.5), (0, 4.0)])
def test_window_and_cap_queries_are_the_whole_sequence(causal, wl, cap):
    """Nq = L with a left window and/or a soft cap: the full-sequence oracle with
    window (wl, unbounded right) and the same cap, both pinned separately."""
    rng = np.random.default_rng(11)
    B, L, Hq, Hkv, d = 2, 9, 4, 2, 8
    q, k, v = _cache(rng, B, L, L, Hq, Hkv, d)
    o, lse = kvcache_fwd(q, k, v, [L] * B, 0.5, causal, window_left=wl, softcap=cap)
    cu = np.arange(B + 1) * L
    win = None if wl is None else (wl, -1)
    of, lf = attention_fwd(q.reshape(B * L, Hq, d), k.reshape(B * L, Hkv, d),
                           v.reshape(B * L, Hkv, d), 0.5, causal, cu, window=win, softcap=cap)
    np.testing.assert_allclose(o.reshape(B * L, Hq, d), of, atol=1e-12)
    np.testing.assert_allclose(lse, lf, atol=1e-12)


def test_zero_window_sees_only_itself():
    """window_left = 0, causal: each query sees only the key at its own position, so
    O is that key's V row and the LSE is its (capped) logit, c·tanh(s / c)."""
    rng = np.random.default_rng(12)
    B, Nq, L, H, d, c = 1, 3, 7, 2, 4, 1.5
    q, k, v = _cache(rng, B, Nq, L, H, H, d)
    o, lse = kvcache_fwd(q, k, v, [L], 0.7, True, window_left=0, softcap=c)
    for h in range(H):
        for i in range(Nq):
            p = L - Nq + i
            np.testing.assert_allclose(o[0, i, h], v[0, p, h], atol=1e-12)
            s = 0.7 * float(q[0, i, h] @ k[0, p, h])
            assert abs(lse[h, i] - c * math.tanh(s / c)) < 1e-12


def test_single_query_causal_equals_full():
    """With one new query every valid key is at or before it."""
    rng = np.random.default_rng(8)
    q, k, v = _cache(rng, 3, 1, 12, 4, 1, 5)
    lens = [12, 5, 1]
    o0, l0 = kvcache_fwd(q, k, v, lens, 0.3, False)
    o1, l1 = kvcache_fwd(q, k, v, lens, 0.3, True)
    np.testing.assert_array_equal(o0, o1)
    np.testing.assert_array_equal(l0, l1)


def test_constant_values_and_first_position():
    rng = np.random.default_rng(9)
    B, Nq, Nk, H, d = 1, 3, 3, 2, 4
    q, k, _ = _cache(rng, B, Nq, Nk, H, H, d)
    row = rng.standard_normal(d)
    v = np.broadcast_to(row, (B, Nk, H, d)).copy()
    o, _ = kvcache_fwd(q, k, v, [Nk], 0.8, False)
    np.testing.assert_allclose(o, np.broadcast_to(row, o.shape), atol=1e-14)
    # causal, Nq = L: query 0 sees only key 0
    v = rng.standard_normal((B, Nk, H, d))
    o, lse = kvcache_fwd(q, k, v, [Nk], 0.8, True)
    np.testing.assert_allclose(o[0, 0], v[0, 0], atol=1e-14)
    np.testing.assert_allclose(lse[:, 0], 0.8 * np.einsum("hc,hc->h", q[0, 0], k[0, 0]), atol=1e-14)


def test_empty_rows():
    rng = np.random.default_rng(10)
    q, k, v = _cache(rng, 2, 3, 4, 2, 2, 3)
    o, lse = kvcache_fwd(q, k, v, [0, 2], 1.0, True)
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[:, 0:3]))
    # entry 1: positions of the queries are -1, 0, 1: the first sees nothing
    assert np.all(o[1, 0] == 0) and np.all(np.isneginf(lse[:, 3]))
    np.testing.assert_allclose(o[1, 1], v[1, 0], atol=1e-14)
    assert np.all(np.isfinite(lse[:, 4:]))


def test_dominant_key_is_one_hot():
    rng = np.random.default_rng(11)
    B, Nq, Nk, H, d = 1, 1, 6, 1, 4
    q, k, v = _cache(rng, B, Nq, Nk, H, H, d)
    k[0, 3, 0] = 60.0 * q[0, 0, 0] / np.linalg.norm(q[0, 0, 0]) ** 2   # S_3 = 60·scale
    o, _ = kvcache_fwd(q, k, v, [Nk], 1.0, False)
    np.testing.assert_allclose(o[0, 0, 0], v[0, 3, 0], atol=1e-12)


def test_split_merge_by_lse():
    """Attention over keys [0, L) = merge of the two key ranges [0, s) and [s, L) by LSE."""
    rng = np.random.default_rng(12)
    B, Nq, L, Hq, Hkv, d, s = 1, 2, 10, 4, 2, 6, 4
    q, k, v = _cache(rng, B, Nq, L, Hq, Hkv, d)
    o, lse = kvcache_fwd(q, k, v, [L], 0.6, False)
    o1, l1 = kvcache_fwd(q, k[:, :s], v[:, :s], [s], 0.6, False)
    o2, l2 = kvcache_fwd(q, k[:, s:], v[:, s:], [L - s], 0.6, False)
    lm = np.logaddexp(l1, l2)                        # [Hq, Nq]
    w1 = np.exp(l1 - lm).T[None, :, :, None]
    w2 = np.exp(l2 - lm).T[None, :, :, None]
    np.testing.assert_allclose(lse, lm, atol=1e-13)
    np.testing.assert_allclose(o, w1 * o1 + w2 * o2, atol=1e-13)


def test_gqa_head_map():
    """Query heads 2g and 2g+1 read KV head g: swapping KV heads permutes the outputs."""
    rng = np.random.default_rng(13)
    q, k, v = _cache(rng, 1, 2, 5, 4, 2, 3)
    o, _ = kvcache_fwd(q, k, v, [5], 1.0, False)
    o_sw, _ = kvcache_fwd(q[:, :, [2, 3, 0, 1]], k[:, :, [1, 0]], v[:, :, [1, 0]], [5], 1.0, False)
    np.testing.assert_allclose(o_sw, o[:, :, [2, 3, 0, 1]], atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("opts", [{}, {"window_left": 3}, {"softcap": 2.0},
                                  {"window_left": 0, "softcap": 1.0}])
def test_units_match_whole(causal, opts):
    """kvcache_fwd_units on selected (entry, head) units equals those units of the
    whole-tensor kvcache_fwd (pinned above): ragged, empty and one-key caches,
    GQA, several queries, with and without a window and a cap."""
    from oracle import kvcache_fwd_units
    rng = np.random.default_rng(31)
    B, Nq, Nk, Hq, Hkv, d = 5, 3, 12, 4, 2, 8
    q, k, v = _cache(rng, B, Nq, Nk, Hq, Hkv, d)
    lens = np.array([12, 0, 1, 7, 2], dtype=np.int32)   # full, empty, one key, ragged, < Nq
    o, lse = kvcache_fwd(q, k, v, lens, 0.35, causal, **opts)
    units = [(b, h) for b in range(B) for h in range(Hq)]
    res = kvcache_fwd_units(q, k, v, lens, 0.35, causal, units, **opts)
    assert sorted(res) == units
    for (b, h), (O, L) in res.items():
        np.testing.assert_allclose(O, o[b, :, h], atol=1e-14)
        np.testing.assert_array_equal(np.isneginf(L), np.isneginf(lse[h, b * Nq:(b + 1) * Nq]))
        fin = np.isfinite(L)
        np.testing.assert_allclose(L[fin], lse[h, b * Nq:(b + 1) * Nq][fin], atol=1e-14)
    # a one-key cache (closed form): a query that sees the key returns its value
    # row; causal queries placed before position 0 see nothing (O = 0, LSE = −inf)
    O2, L2 = res[(2, 3)]
    sees = np.array([not causal, not causal, True])
    np.testing.assert_allclose(O2[sees], np.broadcast_to(v[2, 0, 1], O2[sees].shape), atol=1e-14)
    assert (O2[~sees] == 0).all() and np.isneginf(L2[~sees]).all()


def test_units_rejects_bad_group():
    from oracle import kvcache_fwd_units
    q = np.zeros((1, 1, 3, 4))
    k = np.zeros((1, 2, 2, 4))
    with pytest.raises(ValueError):
        kvcache_fwd_units(q, k, k, np.array([2]), 1.0, False, [(0, 0)])
