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
