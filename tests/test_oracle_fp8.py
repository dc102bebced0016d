"""Pins for the FP8 (e4m3) forward oracle and for its error bound on O.

The e4m3fn decoder is checked against torch's float8_e4m3fn (a library
routine) on all 256 codes and against values fixed by the format (largest
finite 448, smallest subnormal 2^-9, smallest normal 2^-6, NaN codes). The
forward on decoded inputs is checked against closed forms (one key; a
descale only scales its own tensor) and torch's CPU float64 SDPA. The bound
is checked against its own model: weights rounded to e4m3 by torch's cast,
each at a reference 8 (log2 units) below the running max of its tile's
time, never exceed it; an adversarial rounding direction reaches most of it; and a forward that
loses one key block falls outside it.
"""
import math

import numpy as np
import pytest

from oracle import attention_fwd, attention_fwd_fp8, dequantize, e4m3fn_decode, o_bound
import workloads as W


def test_decoder_matches_torch_on_every_code():
    torch = pytest.importorskip("torch")
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(e4m3fn_decode(codes), ref)


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x38, 1.0), (0xB8, -1.0), (0x7E, 448.0), (0xFE, -448.0),
    (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6), (0x3C, 1.5),
    (0x40, 2.0), (0x30, 0.5), (0x77, 240.0), (0x78, 256.0)])
def test_decoder_format_values(code, value):
    assert e4m3fn_decode(np.array([code], np.uint8))[0] == value


def test_decoder_nan_and_signed_zero():
    v = e4m3fn_decode(np.array([0x7F, 0xFF, 0x80], np.uint8))
    assert math.isnan(v[0]) and math.isnan(v[1])
    assert v[2] == 0.0 and math.copysign(1.0, v[2]) == -1.0


def _codes(seed, shape):
    rng = np.random.default_rng(seed)
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    return np.where((c & 0x7F) == 0x7F, np.uint8(0x38), c)   # no NaN codes


def test_single_key_closed_form():
    q8, k8, v8 = _codes(1, (1, 3, 16)), _codes(2, (1, 1, 16)), _codes(3, (1, 1, 16))
    dq, dk, dv = 0.01, 0.02, 0.5
    o, lse = attention_fwd_fp8(q8, k8, v8, 0.3, dq, dk, dv)
    qd, kd, vd = e4m3fn_decode(q8), e4m3fn_decode(k8), e4m3fn_decode(v8)
    for h in range(3):
        np.testing.assert_allclose(o[0, h], dv * vd[0, 0], rtol=1e-15)
        assert lse[h, 0] == pytest.approx(0.3 * dq * dk * float(qd[0, h] @ kd[0, 0]), rel=1e-12)


def test_descales_act_on_their_own_tensor():
    q8, k8, v8 = _codes(4, (20, 2, 8)), _codes(5, (20, 1, 8)), _codes(6, (20, 1, 8))
    o1, l1 = attention_fwd_fp8(q8, k8, v8, 0.2, 0.01, 0.03, 0.7, causal=True)
    o2, l2 = attention_fwd_fp8(q8, k8, v8, 0.2, 0.03, 0.01, 1.4, causal=True)
    np.testing.assert_allclose(l2, l1, rtol=1e-13)           # only the product dq·dk enters S
    np.testing.assert_allclose(o2, 2 * o1, rtol=1e-13)       # O is linear in V's descale


def test_torch_sdpa_on_decoded_inputs():
    torch = pytest.importorskip("torch")
    q8, k8, v8 = _codes(7, (33, 4, 16)), _codes(8, (33, 2, 16)), _codes(9, (33, 2, 16))
    ds = (0.004, 0.006, 0.3)
    o, lse = attention_fwd_fp8(q8, k8, v8, 0.25, *ds, causal=True)
    tq, tk, tv = (torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64) * s
                  for c, s in zip((q8, k8, v8), ds))
    tk = tk.repeat_interleave(2, dim=1)
    tv = tv.repeat_interleave(2, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq.permute(1, 0, 2), tk.permute(1, 0, 2), tv.permute(1, 0, 2), is_causal=True, scale=0.25)
    np.testing.assert_allclose(o, ref.permute(1, 0, 2).numpy(), atol=1e-12)


def test_quantized_inputs_round_trip():
    """The input recipe: codes·descale stay within half an e4m3 step of the float input."""
    w = W.custom(B=1, Hq=2, Hkv=1, N=50, d=32, seed=11)
    a = W.generate(w, with_grad=False)
    f8 = W.quantize_e4m3(a)
    for n in ("q", "k", "v"):
        x = a[n].astype(np.float64)
        xd = dequantize(f8[n], f8["descale_" + n])
        assert np.abs(xd).max() == pytest.approx(np.abs(x).max(), rel=1e-6)
        err = np.abs(xd - x)
        assert np.all(err <= np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * f8["descale_" + n]) * 1.0001)


# ---- the bound on O -------------------------------------------------------------
RMS_FRACTION = 0.3   # rms error / rms bound that the model stays under (also used on the GPU)

def _round_e4m3(x):
    import torch
    return torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()


def _model_forward(q, k, v, scale, causal, rng, lift=8.0):
    """The bound's model, one head, in log2 units: key j's weight is rounded to
    e4m3 (torch's cast) at the reference its tile had, r_j = M_j − lift with
    M_j anywhere between its own score s_j and the row's max M (the running
    max when the tile was processed), so 2^(s_j − r_j) ≤ 2^lift; it is then
    carried to the final reference M − lift exactly, and O is normalised by
    the sum of the rounded weights."""
    S = scale * (q @ k.T) * math.log2(math.e)
    L = S.shape[0]
    if causal:
        S = np.where(np.arange(L)[None, :] <= np.arange(L)[:, None], S, -np.inf)
    M = S.max(axis=1, keepdims=True)
    Sf = np.where(np.isfinite(S), S, M)
    Mj = Sf + rng.uniform(0, 1, size=S.shape) * (M - Sf)
    Mj = np.where(rng.random(S.shape) < 0.5, M, Mj)   # half the keys: the final reference
    r = Mj - lift
    pr = _round_e4m3(np.exp2(S - r)) * np.exp2(r - (M - lift))
    return (pr @ v) / pr.sum(axis=1, keepdims=True)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("sharp", [0.1, 1.0, 6.0])
def test_bound_holds_for_rounded_weights(causal, sharp):
    torch = pytest.importorskip("torch")
    del torch
    rng = np.random.default_rng(12)
    L, d = 200, 32
    w = W.custom(B=1, Hq=1, Hkv=1, N=L, d=d, seed=13)
    f8 = W.quantize_e4m3(W.generate(w, with_grad=False), v_shift=0.5)
    q, k, v = (dequantize(f8[n], f8["descale_" + n]) for n in ("q", "k", "v"))
    scale = sharp / math.sqrt(d)
    o, _ = attention_fwd(q, k, v, scale, causal)
    bnd = o_bound(q, k, v, o, scale, causal)
    assert np.all(np.isfinite(bnd))
    for _ in range(5):
        om = _model_forward(q[:, 0], k[:, 0], v[:, 0], scale, causal, rng)
        err = np.abs(om - o[:, 0])
        assert np.all(err <= bnd[:, 0])
        # independent roundings mostly cancel: the GPU tests' second criterion
        assert np.sqrt((err ** 2).mean()) <= RMS_FRACTION * np.sqrt((bnd[:, 0] ** 2).mean())


def test_bound_is_nearly_reached_by_adversarial_rounding():
    """Weights pushed up by U where V_jc > O_ic and down elsewhere (all normal)."""
    rng = np.random.default_rng(14)
    L, d = 64, 16
    q, k, v = rng.standard_normal((L, 1, d)), rng.standard_normal((L, 1, d)), rng.standard_normal((L, 1, d))
    scale = 0.05
    o, _ = attention_fwd(q, k, v, scale, False)
    bnd = o_bound(q, k, v, o, scale, False)
    S = scale * (q[:, 0] @ k[:, 0].T)
    P = np.exp(S - S.max(axis=1, keepdims=True))
    c = 3
    sgn = np.sign(v[:, 0, c][None, :] - o[:, 0, c][:, None])
    Pp = P * (1 + 2.0 ** -4 * sgn)
    oa = (Pp @ v[:, 0, c]) / Pp.sum(axis=1)
    ratio = np.abs(oa - o[:, 0, c]) / bnd[:, 0, c]
    assert ratio.max() <= 1.0
    assert ratio.min() > 0.85


def test_bound_rejects_a_lost_key_block():
    """A forward that drops keys 64..127 is outside the bound on most rows."""
    w = W.custom(B=1, Hq=1, Hkv=1, N=300, d=64, seed=15)
    f8 = W.quantize_e4m3(W.generate(w, with_grad=False), v_shift=0.5)
    q, k, v = (dequantize(f8[n], f8["descale_" + n]) for n in ("q", "k", "v"))
    scale = 1 / 8
    o, _ = attention_fwd(q, k, v, scale, False)
    bnd = o_bound(q, k, v, o, scale, False)
    keep = np.r_[0:64, 128:300]
    o_bad, _ = attention_fwd(q, k[keep], v[keep], scale, False) if False else (None, None)
    S = scale * (q[:, 0] @ k[keep, 0].T)
    P = np.exp(S - S.max(axis=1, keepdims=True))
    o_bad = (P @ v[keep, 0]) / P.sum(axis=1, keepdims=True)
    outside = np.any(np.abs(o_bad - o[:, 0]) > bnd[:, 0], axis=1)
    assert outside.mean() > 0.9


def test_bound_rejects_a_wrong_value_descale():
    w = W.custom(B=1, Hq=2, Hkv=1, N=150, d=64, seed=16)
    f8 = W.quantize_e4m3(W.generate(w, with_grad=False), v_shift=0.5)
    ds = [f8["descale_" + n] for n in ("q", "k", "v")]
    o, _ = attention_fwd_fp8(f8["q"], f8["k"], f8["v"], 1 / 8, *ds)
    q, k, v = (dequantize(f8[n], s) for n, s in zip(("q", "k", "v"), ds))
    bnd = o_bound(q, k, v, o, 1 / 8, False)
    assert np.mean(np.abs(1.25 * o - o) > bnd) > 0.9


def test_row_subset_bound_matches_the_whole_head():
    from oracle import head_o_bound
    rng = np.random.default_rng(17)
    q, k, v = (rng.standard_normal((90, 1, 16)) for _ in range(3))
    o, _ = attention_fwd(q, k, v, 0.3, True)
    full = o_bound(q, k, v, o, 0.3, True)
    rows = np.array([0, 5, 44, 89])
    sub = head_o_bound(q[:, 0], k[:, 0], v[:, 0], o[rows, 0], 0.3, True, rows=rows)
    np.testing.assert_allclose(sub, full[rows, 0], rtol=1e-12)


@pytest.mark.parametrize("out", ["bf16", "fp16"])
def test_bound_covers_the_output_rounding(out):
    """One key: O = V exactly, so a correct kernel returns V rounded to the
    output type; the bound must admit that rounding for every value."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(18)
    v = np.concatenate([rng.standard_normal((1, 1, 64)) * 10.0 ** rng.integers(-6, 3),
                        np.exp2(np.arange(-20, 4))[None, None, :64] * (1 + 2.0 ** -9)], axis=2)
    q, k = rng.standard_normal((1, 1, v.shape[2])), rng.standard_normal((1, 1, v.shape[2]))
    o, _ = attention_fwd(q, k, v, 0.1, False)
    td = {"bf16": torch.bfloat16, "fp16": torch.float16}[out]
    rounded = torch.from_numpy(o).to(td).double().numpy()
    assert np.all(np.abs(rounded - o) <= o_bound(q, k, v, o, 0.1, False, out_dtype=out))


# ---- e4m3fn rounding and the plain FP8 baseline --------------------------------

def test_e4m3_round_keeps_every_code():
    from oracle import e4m3fn_round
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = e4m3fn_decode(codes)
    assert np.array_equal(e4m3fn_round(vals), vals)


def test_e4m3_round_ties_to_even_and_nearest():
    """Midpoints between neighbouring codes go to the code whose last mantissa
    bit is 0; a hair either side goes to the nearer code."""
    from oracle import e4m3fn_round
    pos = e4m3fn_decode(np.arange(0x7F, dtype=np.uint8))
    for c in range(0x7E):
        lo, hi = pos[c], pos[c + 1]
        mid = 0.5 * (lo + hi)
        even = lo if c % 2 == 0 else hi
        assert e4m3fn_round(mid) == even, (c, mid)
        assert e4m3fn_round(-mid) == -even
        eps = (hi - lo) * 1e-6
        assert e4m3fn_round(mid - eps) == lo and e4m3fn_round(mid + eps) == hi
    assert e4m3fn_round(1e6) == 448.0 and e4m3fn_round(-449.0) == -448.0


def test_e4m3_round_matches_torch_cast():
    """Against torch's float8_e4m3fn conversion (round to nearest even) on
    magnitudes from below the subnormals to the largest code."""
    import torch
    rng = np.random.default_rng(3)
    x = np.exp2(rng.uniform(-12, np.log2(448.0), 200_000)) * rng.choice([-1.0, 1.0], 200_000)
    x = x.astype(np.float32).astype(np.float64)        # torch converts from float32
    from oracle import e4m3fn_round
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(e4m3fn_round(x), ref)


def test_plain_fp8_baseline_exact_cases():
    """Where every weight is an e4m3 value the baseline is exact attention on
    the decoded inputs: equal scores (all weights 1) and the first causal row
    (a single key). Elsewhere it differs from the exact result by no more than
    the weights' rounding allows."""
    from oracle import attention_fwd_fp8_plain
    rng = np.random.default_rng(9)
    T, H, d = 40, 2, 16
    f8 = {"q": np.zeros((T, H, d), np.float32), "k": rng.standard_normal((T, H, d)).astype(np.float32),
          "v": rng.standard_normal((T, H, d)).astype(np.float32)}
    import workloads as W
    c = W.quantize_e4m3(f8)
    ds = (1.0, c["descale_k"], c["descale_v"])
    exact, _ = attention_fwd_fp8(c["q"], c["k"], c["v"], 0.3, *ds)
    plain = attention_fwd_fp8_plain(c["q"], c["k"], c["v"], 0.3, *ds)
    assert np.allclose(plain, exact, rtol=0, atol=1e-13)          # Q = 0: every P_j = 1
    f8["q"] = rng.standard_normal((T, H, d)).astype(np.float32)
    c = W.quantize_e4m3(f8)
    ds = (c["descale_q"], c["descale_k"], c["descale_v"])
    exact, _ = attention_fwd_fp8(c["q"], c["k"], c["v"], 0.3, *ds, causal=True)
    plain = attention_fwd_fp8_plain(c["q"], c["k"], c["v"], 0.3, *ds, causal=True)
    assert np.allclose(plain[0], exact[0], rtol=0, atol=1e-13)    # one visible key
    q, k, v = (dequantize(c[n], ds[i]) for i, n in enumerate("qkv"))
    err = np.abs(plain - exact)
    assert err.max() > 1e-6                                       # the rounding shows
    # each weight moves by at most max(2^-4·P, min(P, 2^-10)) (half an ulp of a
    # normal code, or of the 2^-9 subnormal spacing, never past zero), so
    # |O_plain − O| ≤ Σ_j max(2^-4·P_j, min(P_j, 2^-10))·|V_j| / Σ_j P_j
    for h in range(H):
        S = 0.3 * q[:, h] @ k[:, h].T
        S = np.where(np.tril(np.ones((T, T), bool)), S, -np.inf)
        P = np.exp(S - S.max(axis=1, keepdims=True))
        e = np.maximum(2.0 ** -4 * P, np.minimum(P, 2.0 ** -10))
        bound = (e @ np.abs(v[:, h])) / P.sum(axis=1, keepdims=True)
        assert np.all(err[:, h] <= bound * (1 + 1e-9) + 1e-15), h


def test_plain_fp8_baseline_worked_two_keys():
    """One query, two keys, worked by hand: q = 1, k0 = 0, k1 = ln 0.53 (code
    −1.0 with descale −ln 0.53), v0 = 0, v1 = 1, scale 1. Then S = (0, ln 0.53),
    P = (1, 0.53); 0.53 lies between the codes 0.5 and 0.5625 and rounds to
    0.5. Plain FP8 attention gives 0.5 / (1 + 0.53) (rounded weight over the
    unrounded sum), exact attention 0.53 / 1.53; normalising by the rounded
    sum instead would give 0.5 / 1.5."""
    from oracle import attention_fwd_fp8_plain
    q8 = np.full((1, 1, 1), 0x38, np.uint8)                 # 1.0
    k8 = np.array([0x00, 0xB8], np.uint8).reshape(2, 1, 1)  # 0, −1.0
    v8 = np.array([0x00, 0x38], np.uint8).reshape(2, 1, 1)  # 0, 1.0
    q8 = np.concatenate([q8, q8])                           # two queries, same row
    ds = (1.0, -np.log(0.53), 1.0)
    plain = attention_fwd_fp8_plain(q8, k8, v8, 1.0, *ds)
    exact, _ = attention_fwd_fp8(q8, k8, v8, 1.0, *ds)
    assert abs(plain[0, 0, 0] - 0.5 / 1.53) < 1e-12
    assert abs(exact[0, 0, 0] - 0.53 / 1.53) < 1e-12
