"""NumPy float64 oracle: attention of a few new queries over a key/value cache.

Test infrastructure only (see the package docstring).

Per batch entry b the cache holds L_b = cache_seqlens[b] valid positions
(0 .. L_b−1) of keys and values; the Nq queries of entry b are the newest Nq
positions of that sequence, so query i sits at position p_i = L_b − Nq + i
(the decode reading: the new tokens were appended to the cache before
attention runs; the pages speak of long-context inference and of inference
tools that turn the method on, Flash Attention 是什麼, adersaytech.com,
sections 原理拆解 and 各推論工具怎麼開, and leave the alignment open).

For query head h and its KV head g = ⌊h / (Hq/Hkv)⌋ the scores, softmax and
output are those of plain attention (FlashAttention guide, cxbdf.cn, part 1):

    S_ij  = scale · Σ_c Q[i,c]·K[j,c]           for j visible from i
    LSE_i = ln Σ_j exp(S_ij),  O_i = Σ_j exp(S_ij − LSE_i)·V_j

Visibility: every valid key j < L_b, or keys j ≤ p_i when causal. A query
that sees no key (L_b = 0, or causal with p_i < 0) has the empty sum: O_i = 0
and LSE_i = −∞.

Options, as in the full-sequence oracle (oracle.attention): a sliding window
of `window_left` keys behind the query (keys j ≥ p_i − window_left stay
visible; the sliding-window mask that the mlqm.cn evaluation page, section
四, names among the masks standard attention supports) and a soft cap c (S_ij → c·tanh(S_ij / c),
the same page's section 2.3 in the bounded reading).

Layouts: q [B, Nq, Hq, d], k/v [B, Nk, Hkv, d] with Nk ≥ max L_b;
returns o [B, Nq, Hq, d] and lse [Hq, B·Nq] (query (b, i) at column b·Nq + i).

The same placement serves queries and keys of different lengths in a
training step (a chunk of new tokens over a longer context): kvlen_head_bwd
is the backward of kvcache_head by the chain rule (the pages only say the
backward recomputes the scores rather than storing them: FlashAttention
guide, cxbdf.cn, part 2, item 3), with P_ij = exp(S_ij − LSE_i) over the
visible keys:

    dV_j = Σ_i P_ij dO_i,  dP_ij = dO_i·V_j,  D_i = Σ_j P_ij dP_ij,
    dS_ij = P_ij (dP_ij − D_i),  dQ_i = scale Σ_j dS_ij K_j,  dK_j = scale Σ_i dS_ij Q_i.

A query that sees no key has no weights: its dQ is 0 and it adds nothing to
dK and dV. kvlen_bwd applies it to packed [T, H, d] tensors.
"""
from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):          # a torch tensor: exact upcast of fp16/bf16
        x = x.detach().cpu().double().numpy()
    return np.asarray(x, dtype=np.float64)


def kvcache_head(Qs, Ks, Vs, scale: float, causal: bool, window_left=None, softcap=None):
    """One (batch entry, query head): Qs [Nq, d], Ks/Vs [L, d] (valid keys only).

    Returns O [Nq, dv] and LSE [Nq].
    """
    Qs, Ks, Vs = _f64(Qs), _f64(Ks), _f64(Vs)
    Nq, L = Qs.shape[0], Ks.shape[0]
    O = np.zeros((Nq, Vs.shape[1]))
    lse = np.full(Nq, -np.inf)
    if L == 0:
        return O, lse
    S = scale * (Qs @ Ks.T)                                  # [Nq, L]
    if softcap:
        S = softcap * np.tanh(S / softcap)
    pos = L - Nq + np.arange(Nq)                              # query positions
    if causal:
        S = np.where(np.arange(L)[None, :] <= pos[:, None], S, -np.inf)
    if window_left is not None and window_left >= 0:
        S = np.where(np.arange(L)[None, :] >= pos[:, None] - window_left, S, -np.inf)
    seen = np.isfinite(S).any(axis=1)
    if not seen.any():
        return O, lse
    Sv = S[seen]
    m = Sv.max(axis=1)
    l = m + np.log(np.exp(Sv - m[:, None]).sum(axis=1))
    O[seen] = np.exp(Sv - l[:, None]) @ Vs
    lse[seen] = l
    return O, lse


def kvcache_fwd(q, k_cache, v_cache, cache_seqlens, scale: float, causal: bool = False,
                window_left=None, softcap=None):
    """Whole-tensor decode attention; see the module docstring for layouts."""
    q, k, v = _f64(q), _f64(k_cache), _f64(v_cache)
    lens = [int(x) for x in np.asarray(_f64(cache_seqlens))]
    B, Nq, Hq, d = q.shape
    Hkv = k.shape[2]
    if Hkv <= 0 or Hq % Hkv:
        raise ValueError(f"Hq={Hq} must be a positive multiple of Hkv={Hkv}")
    g = Hq // Hkv
    o = np.zeros((B, Nq, Hq, v.shape[3]))
    lse = np.full((Hq, B * Nq), -np.inf)
    for b in range(B):
        L = lens[b]
        for h in range(Hq):
            O, l = kvcache_head(q[b, :, h], k[b, :L, h // g], v[b, :L, h // g], scale, causal,
                                window_left, softcap)
            o[b, :, h] = O
            lse[h, b * Nq:(b + 1) * Nq] = l
    return o, lse


def kvcache_fwd_units(q, k_cache, v_cache, cache_seqlens, scale: float, causal: bool, units,
                      window_left=None, softcap=None):
    """O and LSE of selected (batch entry, query head) units: {(b, h): (O [Nq, d], LSE [Nq])}.

    The same per-unit computation as kvcache_fwd (window and cap included);
    inputs may be torch tensors, and only the selected slices are upcast.
    """
    lens = [int(x) for x in np.asarray(_f64(cache_seqlens))]
    Hq, Hkv = q.shape[2], k_cache.shape[2]
    if Hkv <= 0 or Hq % Hkv:
        raise ValueError(f"Hq={Hq} must be a positive multiple of Hkv={Hkv}")
    g = Hq // Hkv
    res = {}
    for b, h in units:
        L = lens[b]
        res[(b, h)] = kvcache_head(q[b, :, h], k_cache[b, :L, h // g], v_cache[b, :L, h // g],
                                   scale, causal, window_left, softcap)
    return res


def kvlen_head_bwd(Qs, Ks, Vs, dOs, scale: float, causal: bool):
    """One (sequence, query head): Qs, dOs [Lq, d], Ks, Vs [Lk, d], the queries
    at the last Lq key positions. Returns dQ [Lq, d], dK [Lk, d], dV [Lk, dv]."""
    Qs, Ks, Vs, dOs = _f64(Qs), _f64(Ks), _f64(Vs), _f64(dOs)
    Lq, Lk = Qs.shape[0], Ks.shape[0]
    dQ = np.zeros_like(Qs)
    dK = np.zeros_like(Ks)
    dV = np.zeros_like(Vs)
    if Lq == 0 or Lk == 0:
        return dQ, dK, dV
    S = scale * (Qs @ Ks.T)                                  # [Lq, Lk]
    if causal:
        pos = Lk - Lq + np.arange(Lq)
        S = np.where(np.arange(Lk)[None, :] <= pos[:, None], S, -np.inf)
    seen = np.isfinite(S).any(axis=1)
    if not seen.any():
        return dQ, dK, dV
    Sv = S[seen]
    m = Sv.max(axis=1)
    lse = m + np.log(np.exp(Sv - m[:, None]).sum(axis=1))
    P = np.exp(Sv - lse[:, None])                            # rows that see a key
    dO = dOs[seen]
    dV = P.T @ dO
    dP = dO @ Vs.T
    D = (P * dP).sum(axis=1)
    dS = P * (dP - D[:, None])
    dQ[seen] = scale * (dS @ Ks)
    dK = scale * (dS.T @ Qs[seen])
    return dQ, dK, dV


def kvlen_bwd(q, k, v, do, scale: float, causal: bool, cu_q, cu_k):
    """Packed backward: q, do [Tq, Hq, d] split by cu_q, k, v [Tk, Hkv, d] by cu_k
    (B+1 prefix sums each). dK, dV of a KV head are summed over its query heads.
    Returns dq [Tq, Hq, d], dk, dv [Tk, Hkv, d] in float64."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    cq = [int(x) for x in np.asarray(cu_q)]
    ck = [int(x) for x in np.asarray(cu_k)]
    if len(cq) != len(ck):
        raise ValueError("cu_q and cu_k need the same number of entries")
    Hq, Hkv = q.shape[1], k.shape[1]
    if Hkv <= 0 or Hq % Hkv:
        raise ValueError(f"Hq={Hq} must be a positive multiple of Hkv={Hkv}")
    g = Hq // Hkv
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(len(cq) - 1):
        qa, qb, ka, kb = cq[b], cq[b + 1], ck[b], ck[b + 1]
        for h in range(Hq):
            dQ, dK, dV = kvlen_head_bwd(q[qa:qb, h], k[ka:kb, h // g], v[ka:kb, h // g],
                                        do[qa:qb, h], scale, causal)
            dq[qa:qb, h] = dQ
            dk[ka:kb, h // g] += dK
            dv[ka:kb, h // g] += dV
    return dq, dk, dv
