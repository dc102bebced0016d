"""Attention with dropout on the softmax weights: float64 forward and backward.

Test infrastructure only (see the package docstring).

The pages show ``flash_attn_func(q, k, v, dropout_p=0.0, ...)`` (the
FlashAttention-2 page, blog.gitcode.com, API example) and say nothing about the
random numbers behind it. Reading taken (every choice below is this module's,
stated once here):

* Dropout acts on the softmax weights: O = (P ∘ Z) V with Z_ij = M_ij · 256/t,
  M_ij ∈ {0, 1} the keep decision and t/256 the keep probability; LSE stays
  the log-sum-exp of the undropped logits.
* t = ⌊256 · (1 − p) + 1/2⌋ for the caller's dropout_p = p as a 32-bit float
  (the type the library receives; the arithmetic in double), 1 ≤ t ≤ 256, so
  the keep probability is t/256 and 256/t keeps O unbiased.
* Random bits: Philox4x32-10, the counter-based generator of Salmon, Moraes,
  Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC '11),
  written here from its published definition: per round
  (hi0, lo0) = M0·c0, (hi1, lo1) = M1·c2 (32 x 32 → 64-bit products),
  c ← (hi1 ⊕ c1 ⊕ k0, lo1, hi0 ⊕ c3 ⊕ k1, lo0); the key grows by the Weyl
  constants (W0, W1) between rounds; ten rounds.
* One generator call covers a 4 x 4 block of (query i, key j) of one query
  head h of one sequence b (positions local to the sequence): counter
  (⌊j/4⌋, ⌊i/4⌋, h, b), key (seed mod 2^32, ⌊seed / 2^32⌋). Output word i mod 4,
  byte j mod 4 (bits 8·(j mod 4) … +7) is the element's byte; it is kept iff
  byte < t.
* Backward (chain rule through O = (P ∘ Z) V): dV = (P ∘ Z)ᵀ dO,
  dP = dO Vᵀ, D_i = Σ_j P_ij Z_ij dP_ij (= dO_i · O_i), dS = P ∘ (Z ∘ dP − D),
  dQ = scale · dS K, dK = scale · dSᵀ Q.
"""
from __future__ import annotations

import numpy as np

from .attention import _f64, _group, _lse, _row_blocks, _scores, _segments

PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(ctr, key):
    """Philox4x32-10 on arrays: ctr = (c0, c1, c2, c3) and key = (k0, k1), each an
    integer or an array (broadcast together), uint32 values. Returns four uint32
    arrays."""
    c = [np.asarray(x, dtype=np.uint64) & _MASK32 for x in ctr]
    k0 = np.asarray(key[0], dtype=np.uint64) & _MASK32
    k1 = np.asarray(key[1], dtype=np.uint64) & _MASK32
    for r in range(10):
        if r:
            k0 = (k0 + np.uint64(PHILOX_W0)) & _MASK32
            k1 = (k1 + np.uint64(PHILOX_W1)) & _MASK32
        p0 = np.uint64(PHILOX_M0) * c[0]
        p1 = np.uint64(PHILOX_M1) * c[2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]
    return [x.astype(np.uint32) for x in c]


def keep_threshold(dropout_p: float) -> int:
    """t = ⌊256·(1 − p) + 1/2⌋ with p rounded to float32 first; keep probability
    t/256. Needs 0 ≤ p < 1 and t ≥ 1."""
    p = float(np.float32(dropout_p))
    if not (0.0 <= p < 1.0):
        raise ValueError(f"dropout_p={dropout_p} must lie in [0, 1)")
    t = int(np.floor(256.0 * (1.0 - p) + 0.5))
    if t < 1:
        raise ValueError(f"dropout_p={dropout_p} gives no kept weights")
    return min(t, 256)


def keep_mask(seed: int, seq: int, head: int, rows, cols, t: int) -> np.ndarray:
    """M[r, c] for query positions rows[r] and key positions cols[c] of one
    (sequence, query head): True where the weight is kept. The generator runs
    once per 4 x 4 block touched (the block's four words serve its 16 elements)."""
    i = np.asarray(rows, dtype=np.int64)
    j = np.asarray(cols, dtype=np.int64)
    ub_i, inv_i = np.unique(i >> 2, return_inverse=True)
    ub_j, inv_j = np.unique(j >> 2, return_inverse=True)
    words = np.stack(philox4x32_10((ub_j[None, :], ub_i[:, None], head, seq),
                                   (seed & 0xFFFFFFFF, seed >> 32)))   # [4, blocks_i, blocks_j]
    w = words[(i & 3)[:, None], inv_i[:, None], inv_j[None, :]]
    byte = (w >> (8 * (j & 3)).astype(np.uint32)[None, :]) & np.uint32(0xFF)
    return byte < t


def head_fwd_dropout(Qs, Ks, Vs, scale: float, causal: bool, seq: int, head: int,
                     dropout_p: float, seed: int, rows=None):
    """One (sequence, query head): O [R, d] and LSE [R] for ``rows`` (default all)."""
    Qs, Ks, Vs = _f64(Qs), _f64(Ks), _f64(Vs)
    t = keep_threshold(dropout_p)
    L = Ks.shape[0]
    rows = np.arange(Qs.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    O = np.empty((len(rows), Vs.shape[1]))
    lse = np.empty(len(rows))
    pos = 0
    for blk in _row_blocks(rows, L):
        S = _scores(Qs[blk], blk, Ks, scale, causal)
        l = _lse(S)
        Z = keep_mask(seed, seq, head, blk, np.arange(L), t) * (256.0 / t)
        O[pos:pos + len(blk)] = (np.exp(S - l[:, None]) * Z) @ Vs
        lse[pos:pos + len(blk)] = l
        pos += len(blk)
    return O, lse


def head_bwd_dropout(Qs, Ks, Vs, dOs, scale: float, causal: bool, seq: int, head: int,
                     dropout_p: float, seed: int):
    """One (sequence, query head): dQ, dK, dV [L, d] of the dropout forward."""
    Qs, Ks, Vs, dOs = _f64(Qs), _f64(Ks), _f64(Vs), _f64(dOs)
    t = keep_threshold(dropout_p)
    L = Qs.shape[0]
    dQ = np.empty_like(Qs)
    dK = np.zeros_like(Ks)
    dV = np.zeros_like(Vs)
    for blk in _row_blocks(np.arange(L), L):
        S = _scores(Qs[blk], blk, Ks, scale, causal)
        P = np.exp(S - _lse(S)[:, None])
        Z = keep_mask(seed, seq, head, blk, np.arange(L), t) * (256.0 / t)
        dO = dOs[blk]
        dV += (P * Z).T @ dO
        dP = dO @ Vs.T
        D = (P * Z * dP).sum(axis=1)
        dS = P * (Z * dP - D[:, None])
        dQ[blk] = scale * (dS @ Ks)
        dK += scale * (dS.T @ Qs[blk])
    return dQ, dK, dV


def attention_fwd_dropout(q, k, v, scale: float, causal: bool, cu_seqlens, dropout_p: float,
                          seed: int):
    """O [T, Hq, d] and LSE [Hq, T] (float64) with dropout on the softmax weights."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    T, Hq, d = q.shape
    g = _group(Hq, k.shape[1])
    o = np.zeros((T, Hq, v.shape[2]))
    lse = np.zeros((Hq, T))
    for s, (a, b) in enumerate(_segments(T, cu_seqlens)):
        if b <= a:
            continue
        for h in range(Hq):
            O, l = head_fwd_dropout(q[a:b, h], k[a:b, h // g], v[a:b, h // g], scale, causal, s,
                                    h, dropout_p, seed)
            o[a:b, h] = O
            lse[h, a:b] = l
    return o, lse


def attention_bwd_dropout(q, k, v, do, scale: float, causal: bool, cu_seqlens, dropout_p: float,
                          seed: int):
    """dq [T, Hq, d], dk/dv [T, Hkv, d] (float64) of the dropout forward above."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    T, Hq, d = q.shape
    g = _group(Hq, k.shape[1])
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for s, (a, b) in enumerate(_segments(T, cu_seqlens)):
        if b <= a:
            continue
        for h in range(Hq):
            dQ, dK, dV = head_bwd_dropout(q[a:b, h], k[a:b, h // g], v[a:b, h // g], do[a:b, h],
                                          scale, causal, s, h, dropout_p, seed)
            dq[a:b, h] = dQ
            dk[a:b, h // g] += dK
            dv[a:b, h // g] += dV
    return dq, dk, dv
