"""NumPy float64 oracle: attention by its definition, with S materialised.

Test infrastructure only (see the package docstring).

Forward, per sequence s, query head h and its KV head g = ⌊h / (Hq/Hkv)⌋,
positions local to the sequence (FlashAttention guide, cxbdf.cn, part 1,
"計算注意力分數" / "應用 Softmax" / "與 V 聚合"):

    S_ij  = scale · Σ_c Q[i,c]·K[j,c]           for j visible from i
    LSE_i = ln Σ_j exp(S_ij)                     (computed as m_i + ln Σ exp(S_ij − m_i))
    P_ij  = exp(S_ij − LSE_i)                    (softmax along the row)
    O_i   = Σ_j P_ij · V_j

Visibility: every key of the same sequence, or keys j ≤ i when causal (the
causal flag of ``flash_attn_func``, Llama-Factory page, first code sample).
Optionally a sliding window (wl, wr) keeps only keys i − wl ≤ j ≤ i + wr
(a negative bound is unbounded): the band mask that the mlqm.cn page,
section 四 (mask types), names among the masks standard attention allows;
with causal the two conditions both apply.
Optionally a soft cap c > 0 bounds the logits smoothly before the softmax:
S_ij = c · tanh(scale · Q_i·K_j / c). The FlashAttention-2 page (blog.gitcode.com,
section 2.3, adaptive soft cap) introduces a softcap step; the formula printed
there neither bounds the score nor is continuous at the cap, so the bounded
tanh form is the reading taken (the backward then carries the factor
1 − tanh² of the chain rule).
Sequences never see each other (padding-free packing; the mlqm.cn page,
section 四, lists padding masks among what the method supports).
The row logsumexp is the ``softmax_lse`` the forward kernel writes out
(FlashAttention-2 全解析, blog.gitcode.com, core tiling sketch), in natural
log of the scaled logits.

Backward, given dO (chain rule; the pages only say the backward recomputes
S from Q, K, V blocks instead of storing it: cxbdf.cn guide, part 2, item 3):

    dV_j  = Σ_i P_ij · dO_i
    dP_ij = dO_i · V_j
    D_i   = Σ_j P_ij · dP_ij
    dS_ij = P_ij · (dP_ij − D_i)
    dQ_i  = scale · Σ_j dS_ij · K_j
    dK_j  = scale · Σ_i dS_ij · Q_i

dK and dV of a KV head are summed over the query heads that share it.

Large sequences are processed in blocks of whole rows, so a block holds
complete rows of S and nothing is reordered within a row.
"""
from __future__ import annotations

from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np

_BLOCK_ELEMS = 1 << 25   # at most 32 Mi score entries (256 MiB) per row block


def _segments(T: int, cu_seqlens) -> List[Tuple[int, int]]:
    if cu_seqlens is None:
        return [(0, T)]
    cu = [int(x) for x in np.asarray(cu_seqlens)]
    return [(cu[i], cu[i + 1]) for i in range(len(cu) - 1)]


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):          # a torch tensor: exact upcast of fp16/bf16
        x = x.detach().cpu().double().numpy()
    return np.asarray(x, dtype=np.float64)


def _group(Hq: int, Hkv: int) -> int:
    if Hkv <= 0 or Hq % Hkv:
        raise ValueError(f"Hq={Hq} must be a positive multiple of Hkv={Hkv}")
    return Hq // Hkv


def _scores(Qr: np.ndarray, rows: np.ndarray, Ks: np.ndarray, scale: float,
            causal: bool, window=None, softcap=None) -> np.ndarray:
    """S for the query rows ``rows`` (positions in the sequence) against all keys;
    invisible keys get −inf."""
    S = scale * (Qr @ Ks.T)
    if softcap:
        S = softcap * np.tanh(S / softcap)
    keys = np.arange(Ks.shape[0])[None, :]
    if causal:
        S = np.where(keys <= rows[:, None], S, -np.inf)
    if window is not None:
        wl, wr = window
        if wl >= 0:
            S = np.where(keys >= rows[:, None] - wl, S, -np.inf)
        if wr >= 0:
            S = np.where(keys <= rows[:, None] + wr, S, -np.inf)
    return S


def _lse(S: np.ndarray) -> np.ndarray:
    m = S.max(axis=1)
    return m + np.log(np.exp(S - m[:, None]).sum(axis=1))


def _row_blocks(rows: np.ndarray, L: int):
    step = max(1, _BLOCK_ELEMS // max(L, 1))
    for a in range(0, len(rows), step):
        yield rows[a:a + step]


def head_fwd(Qs, Ks, Vs, scale: float, causal: bool, rows=None, window=None, softcap=None):
    """One (sequence, query head): O [R, d] and LSE [R] for ``rows`` (default all)."""
    Qs, Ks, Vs = _f64(Qs), _f64(Ks), _f64(Vs)
    L = Ks.shape[0]
    rows = np.arange(Qs.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    O = np.empty((len(rows), Vs.shape[1]))
    lse = np.empty(len(rows))
    pos = 0
    for blk in _row_blocks(rows, L):
        S = _scores(Qs[blk], blk, Ks, scale, causal, window, softcap)
        l = _lse(S)
        P = np.exp(S - l[:, None])
        O[pos:pos + len(blk)] = P @ Vs
        lse[pos:pos + len(blk)] = l
        pos += len(blk)
    return O, lse


def head_bwd(Qs, Ks, Vs, dOs, scale: float, causal: bool, window=None, softcap=None):
    """One (sequence, query head): dQ, dK, dV [L, d] by the chain rule above."""
    Qs, Ks, Vs, dOs = _f64(Qs), _f64(Ks), _f64(Vs), _f64(dOs)
    L = Qs.shape[0]
    dQ = np.empty_like(Qs)
    dK = np.zeros_like(Ks)
    dV = np.zeros_like(Vs)
    for blk in _row_blocks(np.arange(L), L):
        S = _scores(Qs[blk], blk, Ks, scale, causal, window, softcap)
        P = np.exp(S - _lse(S)[:, None])
        dO = dOs[blk]
        dV += P.T @ dO
        dP = dO @ Vs.T
        D = (P * dP).sum(axis=1)
        dS = P * (dP - D[:, None])
        if softcap:   # d/dx [c·tanh(x/c)] = 1 − tanh²(x/c)
            dS = dS * (1.0 - np.tanh(scale * (Qs[blk] @ Ks.T) / softcap) ** 2)
        dQ[blk] = scale * (dS @ Ks)
        dK += scale * (dS.T @ Qs[blk])
    return dQ, dK, dV


def attention_probs(Qs, Ks, scale: float, causal: bool, window=None,
                    softcap=None) -> np.ndarray:
    """The full softmax matrix P [L, L] of one (sequence, head)."""
    Qs, Ks = _f64(Qs), _f64(Ks)
    S = _scores(Qs, np.arange(Qs.shape[0]), Ks, scale, causal, window, softcap)
    return np.exp(S - _lse(S)[:, None])


def attention_fwd(q, k, v, scale: float, causal: bool = False, cu_seqlens=None, window=None,
                  softcap=None):
    """Whole-tensor forward.

    q [T, Hq, d], k/v [T, Hkv, d] (any float type; upcast exactly to float64);
    cu_seqlens: B+1 prefix sums of sequence lengths, or None for one sequence.
    Returns o [T, Hq, d] and lse [Hq, T], float64.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    T, Hq, d = q.shape
    g = _group(Hq, k.shape[1])
    o = np.zeros((T, Hq, v.shape[2]))
    lse = np.zeros((Hq, T))
    for a, b in _segments(T, cu_seqlens):
        if b <= a:
            continue
        for h in range(Hq):
            O, l = head_fwd(q[a:b, h], k[a:b, h // g], v[a:b, h // g], scale, causal,
                            window=window, softcap=softcap)
            o[a:b, h] = O
            lse[h, a:b] = l
    return o, lse


def attention_fwd_rows(q, k, v, scale: float, causal: bool, cu_seqlens, seq: int,
                       head: int, rows: Sequence[int], window=None, softcap=None):
    """O and LSE of selected query rows (positions inside sequence ``seq``) of one head."""
    q, k, v = _seq_head_views(q, k, v, cu_seqlens, seq, head)
    return head_fwd(q, k, v, scale, causal, rows=np.asarray(rows), window=window,
                    softcap=softcap)


def _seq_head_views(q, k, v, cu_seqlens, seq, head):
    T, Hq = q.shape[0], q.shape[1]
    g = _group(Hq, k.shape[1])
    a, b = _segments(T, cu_seqlens)[seq]
    return q[a:b, head], k[a:b, head // g], v[a:b, head // g]


def attention_bwd(q, k, v, do, scale: float, causal: bool = False, cu_seqlens=None,
                  window=None, softcap=None):
    """Whole-tensor backward: dq [T, Hq, d], dk/dv [T, Hkv, d] in float64."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    T, Hq, d = q.shape
    g = _group(Hq, k.shape[1])
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for a, b in _segments(T, cu_seqlens):
        if b <= a:
            continue
        for h in range(Hq):
            dQ, dK, dV = head_bwd(q[a:b, h], k[a:b, h // g], v[a:b, h // g], do[a:b, h],
                                  scale, causal, window, softcap)
            dq[a:b, h] = dQ
            dk[a:b, h // g] += dK
            dv[a:b, h // g] += dV
    return dq, dk, dv


def attention_bwd_sampled(q, k, v, do, scale: float, causal: bool, cu_seqlens,
                          units: Iterable[Tuple[int, int]],
                          window=None, softcap=None) -> Dict[Tuple[int, int], tuple]:
    """Backward of selected (sequence, KV head) units only.

    Returns {(seq, kv_head): (dq [L, g, d], dk [L, d], dv [L, d])}, where the
    g query heads are those sharing the KV head. Inputs may be torch tensors;
    only the selected slices are upcast.
    """
    T, Hq = q.shape[0], q.shape[1]
    g = _group(Hq, k.shape[1])
    segs = _segments(T, cu_seqlens)
    res = {}
    for s, kvh in units:
        a, b = segs[s]
        Ks, Vs = _f64(k[a:b, kvh]), _f64(v[a:b, kvh])
        dq = np.zeros((b - a, g, Ks.shape[1]))
        dk = np.zeros_like(Ks)
        dv = np.zeros_like(Vs)
        for r in range(g):
            h = kvh * g + r
            dQ, dK, dV = head_bwd(q[a:b, h], Ks, Vs, do[a:b, h], scale, causal, window,
                                  softcap)
            dq[:, r] = dQ
            dk += dK
            dv += dV
        res[(s, kvh)] = (dq, dk, dv)
    return res


def attention_bwd_rows(q, k, v, do, scale: float, causal: bool, cu_seqlens, seq: int,
                       kv_head: int, q_rows: Sequence[int], k_rows: Sequence[int],
                       window=None, softcap=None):
    """Backward of one (sequence, KV head) at selected positions only.

    Returns (dq [len(q_rows), g, d], dk [len(k_rows), d], dv [len(k_rows), d]):
    dQ at query positions ``q_rows`` for each of the g query heads sharing the
    KV head, and dK, dV at key positions ``k_rows``, summed over those heads.

    The same chain rule as head_bwd. A selected key's dK/dV column sums over
    every query row, and each row's P needs its whole LSE and its D, so S, P,
    dP and D are formed for every row (in blocks of whole rows); only the
    selected rows of dQ and the selected columns of dK/dV are then contracted.
    With causal and no window, a block of rows sees no key past its last row,
    so the keys after it are left out of the block's products (their weights
    are exactly zero). Inputs may be torch tensors; only the slices of this
    (sequence, KV head) are upcast.
    """
    T, Hq = q.shape[0], q.shape[1]
    g = _group(Hq, k.shape[1])
    a, b = _segments(T, cu_seqlens)[seq]
    L = b - a
    Ks, Vs = _f64(k[a:b, kv_head]), _f64(v[a:b, kv_head])
    qr = np.asarray(q_rows, dtype=np.int64)
    kr = np.asarray(k_rows, dtype=np.int64)
    if L and ((qr < 0).any() or (qr >= L).any() or (kr < 0).any() or (kr >= L).any()):
        raise ValueError("selected positions must lie inside the sequence")
    dq = np.zeros((len(qr), g, Ks.shape[1]))
    dk = np.zeros((len(kr), Ks.shape[1]))
    dv = np.zeros((len(kr), Vs.shape[1]))
    prefix = causal and window is None
    for r in range(g):
        h = kv_head * g + r
        Qs, dOs = _f64(q[a:b, h]), _f64(do[a:b, h])
        for blk in _row_blocks(np.arange(L), L):
            hi = int(blk[-1]) + 1 if prefix else L       # keys any row of the block can see
            Kb, Vb = Ks[:hi], Vs[:hi]
            S = _scores(Qs[blk], blk, Kb, scale, causal, window, softcap)
            P = np.exp(S - _lse(S)[:, None])
            dO = dOs[blk]
            dP = dO @ Vb.T
            D = (P * dP).sum(axis=1)
            dS = P * (dP - D[:, None])
            if softcap:   # d/dx [c·tanh(x/c)] = 1 − tanh²(x/c)
                dS = dS * (1.0 - np.tanh(scale * (Qs[blk] @ Kb.T) / softcap) ** 2)
            sel = kr < hi                                  # selected keys inside this block's range
            if sel.any():
                dv[sel] += P[:, kr[sel]].T @ dO
                dk[sel] += scale * (dS[:, kr[sel]].T @ Qs[blk])
            mine = np.nonzero((qr >= blk[0]) & (qr <= blk[-1]))[0]
            if len(mine):
                dq[mine, r] = scale * (dS[qr[mine] - blk[0]] @ Kb)
    return dq, dk, dv
