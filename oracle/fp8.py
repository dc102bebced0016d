"""FP8 (e4m3) attention forward: the float64 reference and its error bound.

Test infrastructure only (see the package docstring).

The pages name e4m3 (``torch.float8_e4m3fn``) as the 8-bit format for keys
and values (FlashAttention-2 全解析, blog.gitcode.com, section 4.3, the
KV-cache quantisation pitfall) and credit FlashAttention-3's FP8 forward with
a lower error than plain FP8 attention (Flash Attention 是什麼,
adersaytech.com, FA-1 to FA-4 table and the note after it). They give no
scaling recipe. The reading taken here: Q, K and V arrive as e4m3fn codes,
each tensor with one positive float "descale" that maps a code's value back
to the real number (x = decode(code) · descale). The exact result of the FP8
forward is then plain attention (the definition in ``attention``) on those
real numbers, and that is what this module returns.

A kernel that feeds the softmax weights P to an FP8 matrix product must round
them to e4m3 as well; that rounding is the one step whose error is not at
fp32 level. ``o_bound`` gives an element-wise bound for it (derivation in
its docstring), which the parity tests use as their tolerance for O. The
LSE does not depend on the rounded P and keeps the ordinary tolerance.

e4m3fn (the OCP 8-bit float "E4M3", finite-only variant): bit 7 sign,
bits 6..3 exponent with bias 7, bits 2..0 mantissa. Exponent 0 encodes
subnormals m·2^-9; exponent 15 with mantissa 7 encodes NaN (there is no
infinity); every other code is (1 + m/8)·2^(e−7). The largest finite value
is 448 = 0x7E, the smallest subnormal 2^-9.
"""
from __future__ import annotations

import math

import numpy as np

from .attention import _f64, _group, _scores, _segments, attention_fwd

E4M3_MAX = 448.0
U_E4M3 = 2.0 ** -4           # unit roundoff of a 3-bit mantissa (half an ulp, relative)
SUBNORMAL_HALF_GAP = 2.0 ** -10   # half the spacing 2^-9 of the subnormal codes


def e4m3fn_decode(codes) -> np.ndarray:
    """Value of each e4m3fn code (uint8 array) as float64, from the bit layout."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


def dequantize(codes, descale: float) -> np.ndarray:
    return e4m3fn_decode(codes) * float(descale)


def attention_fwd_fp8(q8, k8, v8, scale: float, descale_q: float, descale_k: float,
                      descale_v: float, causal: bool = False, cu_seqlens=None):
    """O [T, Hq, d] and LSE [Hq, T] (float64) of attention on the decoded inputs."""
    return attention_fwd(dequantize(q8, descale_q), dequantize(k8, descale_k),
                         dequantize(v8, descale_v), scale, causal, cu_seqlens)


# values of the non-negative finite codes 0x00 .. 0x7E, increasing with the code
_E4M3_POS = None


def e4m3fn_round(x) -> np.ndarray:
    """x rounded to the nearest e4m3fn value (float64 in, float64 out).

    Ties go to the code with an even last mantissa bit; magnitudes above 448
    saturate to ±448 (the reading taken for a value past the largest code);
    the sign is kept, zero stays zero. Written from the format: the finite
    non-negative values are the codes 0x00 .. 0x7E, increasing with the code,
    so the nearest one is found between two neighbours of a sorted table.
    """
    global _E4M3_POS
    if _E4M3_POS is None:
        _E4M3_POS = e4m3fn_decode(np.arange(0x7F, dtype=np.uint8))
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    i = np.clip(np.searchsorted(_E4M3_POS, a), 1, 0x7E)   # _E4M3_POS[i-1] < a <= _E4M3_POS[i]
    lo, hi = _E4M3_POS[i - 1], _E4M3_POS[i]
    up = (hi - a < a - lo) | ((hi - a == a - lo) & (i % 2 == 0))
    return np.copysign(np.where(up, hi, lo), x)


def attention_fwd_fp8_plain(q8, k8, v8, scale: float, descale_q: float, descale_k: float,
                            descale_v: float, causal: bool = False, cu_seqlens=None):
    """O [T, Hq, d] (float64) of plain FP8 attention: the baseline that the
    pages compare FlashAttention-3's FP8 forward with (Flash Attention 是什麼,
    adersaytech.com, the note after the FA-1 to FA-4 table), which they do not
    define. The plainest reading: the same per-tensor e4m3 inputs; per row the
    softmax weights P_j = exp(S_j − max S) in [0, 1], each rounded to e4m3 for
    the FP8 product with V; O = Σ_j round(P_j)·V_j / Σ_j P_j, normalised by
    the sum of the unrounded weights. Everything else is exact (float64), so
    the only roundings are those of the inputs and of P.
    """
    q, k, v = dequantize(q8, descale_q), dequantize(k8, descale_k), dequantize(v8, descale_v)
    T, Hq, d = q.shape
    g = _group(Hq, k.shape[1])
    o = np.zeros((T, Hq, d))
    for a, b in _segments(T, cu_seqlens):
        if b <= a:
            continue
        for h in range(Hq):
            S = _scores(q[a:b, h], np.arange(b - a), k[a:b, h // g], scale, causal)
            P = np.exp(S - S.max(axis=1, keepdims=True))
            o[a:b, h] = (e4m3fn_round(P) @ v[a:b, h // g]) / P.sum(axis=1, keepdims=True)
    return o


def o_bound(q, k, v, o, scale: float, causal: bool = False, cu_seqlens=None,
            out_dtype: str = "bf16") -> np.ndarray:
    """Element-wise bound on |O_kernel − O| for a forward that rounds P to e4m3.

    q, k, v are the decoded (real) inputs, o the exact output from
    ``attention_fwd_fp8``. Model of the kernel: per row, weights
    p̃_j = 2^(S_j·log2 e − m̃) for some reference m̃ not above the row's true
    maximum, each rounded to e4m3 (p̃'_j = p̃_j + ε_j), and
    O' = Σ_j p̃'_j V_j / Σ_j p̃'_j, both sums over the same rounded weights.
    (A kernel may round key j's weight at an earlier, lower reference m̃_j ≤ m̃
    and carry it to m̃ exactly; in units of m̃ that rounding moves it by at
    most U_E4M3 relative, or 2^-10·2^(m̃_j − m̃) ≤ 2^-10 absolute, so the
    terms below hold for it too.)
    Writing P_j = p̃_j / Σ p̃ (the exact softmax) and e_j ≥ |ε_j| / Σ p̃,

        O' − O = Σ_j ε_j (V_j − O) / Σ_j p̃'_j
        |O' − O| ≤ Σ_j e_j |V_j − O| / (1 − Σ_j e_j).

    Rounding a normal e4m3 value moves it by at most U_E4M3 relative; below
    2^-6 the codes are evenly spaced 2^-9 apart, so the move is at most 2^-10
    absolute, and never by more than the weight itself (a weight under 2^-10
    rounds to zero). The largest weight has p̃ ≥ 1 (m̃ is not above the
    maximum), so Σ p̃ ≥ 1 and 2^-10 / Σ p̃ ≤ 2^-10 · max_j P_j. Hence

        e_j = max((U_E4M3 + a_j)·P_j·(1 + a_j), min(P_j, 2^-10 · max_j P_j))

    where a_j covers fp32 work before the rounding: the score as a sum of d
    products (≤ (d + 8)·2^-24·scale·Σ_c |q_c k_c| in natural-log units), the
    exponent's fma and the hardware exp2 (≤ 2^-21 relative). Added to the
    bound: the fp32 sums of O and of the weights (≤ (n + 64)·2^-24 of
    Σ_j P_j |V_j| + |O| over the n visible keys) and the final rounding of
    O to the output type (half an ulp, at most 2^-8 relative for bf16 with
    its 8 significant bits and 2^-11 for fp16 with 11, plus 2^-25 absolute
    for fp16's subnormals).
    """
    q, k, v, o = _f64(q), _f64(k), _f64(v), _f64(o)
    T, Hq, d = q.shape
    g = _group(Hq, k.shape[1])
    bound = np.zeros_like(o)
    for a, b in _segments(T, cu_seqlens):
        if b <= a:
            continue
        for h in range(Hq):
            bound[a:b, h] = head_o_bound(q[a:b, h], k[a:b, h // g], v[a:b, h // g], o[a:b, h],
                                         scale, causal, out_dtype=out_dtype)
    return bound


def head_o_bound(Qs, Ks, Vs, O, scale: float, causal: bool, rows=None,
                 out_dtype: str = "bf16") -> np.ndarray:
    """``o_bound`` for one (sequence, query head): the query rows ``rows``
    (positions in the sequence, default all) with their exact outputs O."""
    Qs, Ks, Vs, O = _f64(Qs), _f64(Ks), _f64(Vs), _f64(O)
    d = Qs.shape[1]
    rows = np.arange(Qs.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    out_half_ulp = {"bf16": 2.0 ** -8, "fp16": 2.0 ** -11}[out_dtype]
    out_abs = {"bf16": 0.0, "fp16": 2.0 ** -25}[out_dtype]
    L = Ks.shape[0]
    S = _scores(Qs[rows], rows, Ks, scale, causal)
    m = S.max(axis=1)
    P = np.exp(S - m[:, None])
    P /= P.sum(axis=1, keepdims=True)
    A = scale * (np.abs(Qs[rows]) @ np.abs(Ks).T)
    Sl = np.where(np.isfinite(S), np.abs(S), 0.0)
    a_j = (math.log(2.0) * (d + 8) * 2.0 ** -24 * A * math.log2(math.e)
           + 2.0 ** -21 + 2.0 ** -23 * (Sl + np.abs(m)[:, None]) * math.log2(math.e))
    e = np.maximum((U_E4M3 + a_j) * P * (1.0 + a_j),
                   np.minimum(P, SUBNORMAL_HALF_GAP * P.max(axis=1, keepdims=True)))
    e = np.where(P > 0, e, 0.0)
    esum = e.sum(axis=1)
    num = np.empty_like(O)
    step = max(1, (1 << 22) // max(1, L * d))      # rows per block of |V − O|
    for r0 in range(0, len(rows), step):
        dev = np.abs(Vs[None, :, :] - O[r0:r0 + step, None, :])   # [rows, keys, d]
        num[r0:r0 + step] = np.einsum("ij,ijc->ic", e[r0:r0 + step], dev)
    denom = np.where(esum < 1.0, 1.0 - esum, np.nan)
    nvis = (P > 0).sum(axis=1)
    acc = (nvis + 64)[:, None] * 2.0 ** -24 * (P @ np.abs(Vs) + np.abs(O))
    return num / denom[:, None] + acc + out_half_ulp * (np.abs(O) + num) + out_abs
