"""Pure-Python attention for tiny shapes: explicit loops, math.exp, math.fsum.

Test infrastructure only. Written independently of the NumPy oracle (no
NumPy, no shared helpers) so that the two can pin each other on tiny cases.
Inputs are nested lists q[t][h][c], k[t][g][c], v[t][g][c] (t = packed token,
h/g = head, c = feature); ``seqs`` lists (start, end) token ranges.

Definition followed: the attention formula of the FlashAttention guide
(cxbdf.cn, part 1), softmax along each query row, with the causal and
padding-free visibility rules; the backward is the chain rule of that formula.
``window`` = (left, right) additionally restricts query i to the keys i − left
.. i + right (a negative bound is unbounded): the band ("sliding window") mask
of the mlqm.cn page, section 四. ``softcap`` = c > 0 replaces each logit x by
c·tanh(x / c) (the bounded reading of the FlashAttention-2 page's soft cap,
blog.gitcode.com section 2.3); its derivative 1 − tanh² enters the backward.
"""
from __future__ import annotations

import math


def _dot(a, b):
    return math.fsum(x * y for x, y in zip(a, b))


def _visible(i, L, causal, window=None):
    lo, hi = 0, L - 1
    if causal:
        hi = min(hi, i)
    if window is not None:
        if window[0] >= 0:
            lo = max(lo, i - window[0])
        if window[1] >= 0:
            hi = min(hi, i + window[1])
    return range(lo, hi + 1)


def _logit(x, softcap):
    return softcap * math.tanh(x / softcap) if softcap else x


def forward(q, k, v, scale, causal, seqs, window=None, softcap=None):
    Hq, Hkv = len(q[0]), len(k[0])
    grp = Hq // Hkv
    o = [[None] * Hq for _ in q]
    lse = [[None] * len(q) for _ in range(Hq)]
    for (a, b) in seqs:
        L = b - a
        for h in range(Hq):
            g = h // grp
            for i in range(L):
                js = list(_visible(i, L, causal, window))
                s = [_logit(scale * _dot(q[a + i][h], k[a + j][g]), softcap) for j in js]
                m = max(s)
                lsum = math.log(math.fsum(math.exp(x - m) for x in s)) + m
                p = [math.exp(x - lsum) for x in s]
                dv = len(v[0][0])
                o[a + i][h] = [math.fsum(p[n] * v[a + j][g][c] for n, j in enumerate(js))
                               for c in range(dv)]
                lse[h][a + i] = lsum
    return o, lse


def backward(q, k, v, do, scale, causal, seqs, window=None, softcap=None):
    Hq, Hkv = len(q[0]), len(k[0])
    grp = Hq // Hkv
    d = len(q[0][0])
    dv_ = len(v[0][0])
    dq = [[[0.0] * d for _ in range(Hq)] for _ in q]
    dk = [[[0.0] * d for _ in range(Hkv)] for _ in k]
    dvv = [[[0.0] * dv_ for _ in range(Hkv)] for _ in v]
    for (a, b) in seqs:
        L = b - a
        for h in range(Hq):
            g = h // grp
            # P and dP for the whole (sequence, head), then the sums term by term
            P = [[0.0] * L for _ in range(L)]
            dP = [[0.0] * L for _ in range(L)]
            G = [[1.0] * L for _ in range(L)]   # derivative of the soft cap
            for i in range(L):
                js = list(_visible(i, L, causal, window))
                raw = [scale * _dot(q[a + i][h], k[a + j][g]) for j in js]
                s = [_logit(x, softcap) for x in raw]
                m = max(s)
                lsum = math.log(math.fsum(math.exp(x - m) for x in s)) + m
                for n, j in enumerate(js):
                    P[i][j] = math.exp(s[n] - lsum)
                    dP[i][j] = _dot(do[a + i][h], v[a + j][g])
                    if softcap:
                        G[i][j] = 1.0 - math.tanh(raw[n] / softcap) ** 2
            D = [math.fsum(P[i][j] * dP[i][j] for j in range(L)) for i in range(L)]
            dS = [[P[i][j] * (dP[i][j] - D[i]) * G[i][j] for j in range(L)] for i in range(L)]
            for i in range(L):
                for c in range(d):
                    dq[a + i][h][c] = scale * math.fsum(dS[i][j] * k[a + j][g][c]
                                                        for j in range(L))
            for j in range(L):
                for c in range(d):
                    dk[a + j][g][c] += scale * math.fsum(dS[i][j] * q[a + i][h][c]
                                                         for i in range(L))
                for c in range(dv_):
                    dvv[a + j][g][c] += math.fsum(P[i][j] * do[a + i][h][c]
                                                  for i in range(L))
    return dq, dk, dvv


def forward_kvcache(q, k, v, lens, scale, causal):
    """Decode attention over a cache, loop by loop.

    q[b][i][h][c] (Nq new queries per entry), k[b][j][g][c], v[b][j][g][c]
    (cache positions), lens[b] valid positions. Query i of entry b sits at
    position lens[b] − Nq + i; causal keys are those at or before it.
    Returns o[b][i][h] (list of floats) and lse[b][i][h] (−inf for no key).
    """
    o, lse = [], []
    for b in range(len(q)):
        Nq, Hq, Hkv = len(q[b]), len(q[b][0]), len(k[b][0])
        grp = Hq // Hkv
        L = lens[b]
        dv = len(v[b][0][0])
        ob, lb = [], []
        for i in range(Nq):
            p = L - Nq + i
            oi, li = [], []
            for h in range(Hq):
                g = h // grp
                js = [j for j in range(L) if (not causal or j <= p)]
                if not js:
                    oi.append([0.0] * dv)
                    li.append(-math.inf)
                    continue
                s = [scale * _dot(q[b][i][h], k[b][j][g]) for j in js]
                m = max(s)
                lsum = math.log(math.fsum(math.exp(x - m) for x in s)) + m
                w = [math.exp(x - lsum) for x in s]
                oi.append([math.fsum(w[n] * v[b][j][g][c] for n, j in enumerate(js))
                           for c in range(dv)])
                li.append(lsum)
            ob.append(oi)
            lb.append(li)
        o.append(ob)
        lse.append(lb)
    return o, lse


# ---- dropout (the reading of oracle/dropout.py), written separately ------------
_M32 = 0xFFFFFFFF


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Philox4x32-10 on Python ints (Salmon et al., SC '11): ten rounds of two
    32 x 32 -> 64-bit products, key bumped by the Weyl constants in between."""
    for r in range(10):
        if r:
            k0 = (k0 + 0x9E3779B9) & _M32
            k1 = (k1 + 0xBB67AE85) & _M32
        p0 = 0xD2511F53 * c0
        p1 = 0xCD9E8D57 * c2
        c0, c1, c2, c3 = ((p1 >> 32) ^ c1 ^ k0, p1 & _M32, (p0 >> 32) ^ c3 ^ k1, p0 & _M32)
    return c0, c1, c2, c3


def _kept(seed, seq, head, i, j, t):
    words = philox4x32_10(j // 4, i // 4, head, seq, seed & _M32, seed >> 32)
    return ((words[i % 4] >> (8 * (j % 4))) & 0xFF) < t


def forward_dropout(q, k, v, scale, causal, seqs, t, seed):
    """O and LSE with dropout on the softmax weights (keep iff byte < t, kept
    weights scaled by 256/t)."""
    Hq, Hkv = len(q[0]), len(k[0])
    grp = Hq // Hkv
    dv = len(v[0][0])
    o = [[None] * Hq for _ in q]
    lse = [[None] * len(q) for _ in range(Hq)]
    for sidx, (a, b) in enumerate(seqs):
        L = b - a
        for h in range(Hq):
            g = h // grp
            for i in range(L):
                js = list(_visible(i, L, causal))
                s = [scale * _dot(q[a + i][h], k[a + j][g]) for j in js]
                m = max(s)
                lsum = math.log(math.fsum(math.exp(x - m) for x in s)) + m
                z = [256.0 / t if _kept(seed, sidx, h, i, j, t) else 0.0 for j in js]
                p = [math.exp(x - lsum) * zz for x, zz in zip(s, z)]
                o[a + i][h] = [math.fsum(p[n] * v[a + j][g][c] for n, j in enumerate(js))
                               for c in range(dv)]
                lse[h][a + i] = lsum
    return o, lse


def backward_dropout(q, k, v, do, scale, causal, seqs, t, seed):
    Hq, Hkv = len(q[0]), len(k[0])
    grp = Hq // Hkv
    d = len(q[0][0])
    dv_ = len(v[0][0])
    dq = [[[0.0] * d for _ in range(Hq)] for _ in q]
    dk = [[[0.0] * d for _ in range(Hkv)] for _ in k]
    dvv = [[[0.0] * dv_ for _ in range(Hkv)] for _ in v]
    for sidx, (a, b) in enumerate(seqs):
        L = b - a
        for h in range(Hq):
            g = h // grp
            P = [[0.0] * L for _ in range(L)]
            Z = [[0.0] * L for _ in range(L)]
            dP = [[0.0] * L for _ in range(L)]
            for i in range(L):
                js = list(_visible(i, L, causal))
                s = [scale * _dot(q[a + i][h], k[a + j][g]) for j in js]
                m = max(s)
                lsum = math.log(math.fsum(math.exp(x - m) for x in s)) + m
                for n, j in enumerate(js):
                    P[i][j] = math.exp(s[n] - lsum)
                    Z[i][j] = 256.0 / t if _kept(seed, sidx, h, i, j, t) else 0.0
                    dP[i][j] = _dot(do[a + i][h], v[a + j][g])
            D = [math.fsum(P[i][j] * Z[i][j] * dP[i][j] for j in range(L)) for i in range(L)]
            dS = [[P[i][j] * (Z[i][j] * dP[i][j] - D[i]) for j in range(L)] for i in range(L)]
            for i in range(L):
                for c in range(d):
                    dq[a + i][h][c] = scale * math.fsum(dS[i][j] * k[a + j][g][c]
                                                        for j in range(L))
            for j in range(L):
                for c in range(d):
                    dk[a + j][g][c] += scale * math.fsum(dS[i][j] * q[a + i][h][c]
                                                         for i in range(L))
                for c in range(dv_):
                    dvv[a + j][g][c] += math.fsum(P[i][j] * Z[i][j] * do[a + i][h][c]
                                                  for i in range(L))
    return dq, dk, dvv
