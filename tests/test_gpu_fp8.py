"""GPU parity of the FP8 (e4m3) forward (fa_fwd_fp8) against the oracle.

Inputs: the usual normal draws quantised per tensor to e4m3fn (descale =
max|x| / 448); V optionally shifted so that O is far from zero. The oracle is
plain attention on the decoded inputs in float64. Criteria:
  O    every element within the oracle's bound for a forward that rounds P to
       e4m3 (oracle.o_bound), and the rms error below RMS_FRACTION of the rms
       bound (the level the bound's own model stays under, pinned on the CPU)
       plus the rms of the output type's own rounding;
  LSE  max |LSE_gpu − LSE_ref| ≤ 1e-3 (the 16-bit forward's rule: the LSE does
       not use the rounded weights);
plus exact invariants of the descales: doubling V's descale doubles O bit for
bit, and exchanging power-of-two Q and K descales changes no bit.
"""
import numpy as np
import pytest

import workloads as W
from oracle import attention_fwd, attention_fwd_fp8, dequantize, head_o_bound, o_bound
from parity_util import TOL_LSE, bits_equal, say
from test_oracle_fp8 import RMS_FRACTION

pytestmark = pytest.mark.gpu


def _fa():
    import exact_io_aware_12_amd as fa   # raises if libfa.so is missing: no fallback
    return fa


def _inputs(w, v_shift=0.0):
    import torch
    f8 = W.quantize_e4m3(W.generate(w, with_grad=False), v_shift=v_shift)
    dev = {n: torch.from_numpy(f8[n]).cuda().view(torch.float8_e4m3fn) for n in ("q", "k", "v")}
    dev["cu_seqlens"] = torch.from_numpy(f8["cu_seqlens"]).cuda()
    return f8, dev


def run_fp8(w, f8, dev, scale=None, out="bf16", ds=None):
    import torch
    fa = _fa()
    scale = w.scale if scale is None else scale
    ds = ds or (f8["descale_q"], f8["descale_k"], f8["descale_v"])
    od = {"bf16": torch.bfloat16, "fp16": torch.float16}[out]
    if w.varlen:
        q, k, v = dev["q"], dev["k"], dev["v"]
        kw = dict(cu_seqlens=dev["cu_seqlens"], max_seqlen=w.N)
    else:
        shp = (w.B, w.N)
        q = dev["q"].view(*shp, w.Hq, w.d)
        k, v = (dev[n].view(*shp, w.Hkv, w.d) for n in ("k", "v"))
        kw = {}
    o, lse = fa.flash_attn_func_fp8(q, k, v, *ds, causal=w.causal, softmax_scale=scale,
                                    out_dtype=od, **kw)
    torch.cuda.synchronize()
    return o.reshape(w.T, w.Hq, w.d), lse


def compare(w, v_shift=0.0, scale=None, out="bf16"):
    say(f"[fa_fwd_fp8] B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} d={w.d} causal={w.causal} "
        f"varlen={w.varlen} v_shift={v_shift} scale={scale} out={out}")
    f8, dev = _inputs(w, v_shift)
    scale = w.scale if scale is None else scale
    o, lse = run_fp8(w, f8, dev, scale, out)
    cu = f8["cu_seqlens"]
    q, k, v = (dequantize(f8[n], f8["descale_" + n]) for n in ("q", "k", "v"))
    o_ref, lse_ref = attention_fwd(q, k, v, scale, w.causal, cu)
    bnd = o_bound(q, k, v, o_ref, scale, w.causal, cu, out_dtype=out)
    og = o.double().cpu().numpy()
    err = np.abs(og - o_ref)
    assert np.isfinite(og).all()
    bad = err > bnd
    if bad.any():
        idx = np.unravel_index(np.argmax(err - bnd), err.shape)
        raise AssertionError(f"O: {bad.sum()} elements outside the bound; worst at {idx}: gpu "
                             f"{og[idx]!r} ref {o_ref[idx]!r} err {err[idx]:.3e} bound {bnd[idx]:.3e}")
    if err.size:
        # the rms rule covers the weights' rounding; the output's own rounding
        # (half an ulp: 2^-8 relative for bf16, 2^-11 for fp16) comes on top
        u_out = {"bf16": 2.0 ** -8, "fp16": 2.0 ** -11}[out]
        rms = lambda x: float(np.sqrt((x ** 2).mean()))
        lim = RMS_FRACTION * rms(bnd) + rms(u_out * o_ref)
        assert rms(err) <= lim, f"O: rms err {rms(err):.3e} > {lim:.3e}"
    el = np.abs(lse.double().cpu().numpy() - lse_ref)
    assert np.isfinite(lse.cpu().numpy()).all()
    assert el.max(initial=0.0) <= TOL_LSE, f"LSE: max err {el.max():.3e}"
    say(f"   max|dO| {err.max(initial=0):.2e} (max err/bound {(err / bnd).max(initial=0):.2f}) "
        f"max|dLSE| {el.max(initial=0):.2e}")


@pytest.mark.parametrize("out", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 64, 65, 333, 700])
def test_fp8_forward(N, causal, out):
    compare(W.custom(B=2, Hq=2, Hkv=1, N=N, d=128, causal=causal, seed=800 + N), v_shift=0.5,
            out=out)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 65, 700])
@pytest.mark.parametrize("d", [64, 256])
def test_fp8_forward_head_dims(d, N, causal):
    """d = 64 and 256: rows of 64 and 256 bytes, each with its own LDS swizzle;
    d = 256 runs one workgroup per CU."""
    compare(W.custom(B=2, Hq=2, Hkv=1, N=N, d=d, causal=causal, seed=820 + N + d), v_shift=0.5)


@pytest.mark.parametrize("d", [64, 256])
def test_fp8_forward_head_dims_varlen_gqa_fp16(d):
    w = W.custom(B=0, Hq=8, Hkv=2, N=0, d=d, causal=True, seed=821 + d,
                 lens=[300, 0, 1, 129, 64, 513])
    compare(w, v_shift=-0.3, out="fp16")


@pytest.mark.parametrize("scale", [0.02, 0.5])
def test_fp8_forward_sharp_and_flat(scale):
    """A large scale makes rows peaked (the rounded-sum normalisation matters);
    a small one spreads weight over every key."""
    compare(W.custom(B=1, Hq=4, Hkv=2, N=500, d=128, causal=True, seed=810), scale=scale)


def test_fp8_forward_varlen_gqa():
    w = W.custom(B=0, Hq=8, Hkv=2, N=0, d=128, causal=True, seed=811,
                 lens=[300, 0, 1, 129, 64, 513])
    compare(w, v_shift=-0.3)


def test_fp8_forward_long():
    compare(W.custom(B=1, Hq=2, Hkv=1, N=2100, d=128, causal=False, seed=812), v_shift=0.5)


def test_fp8_descale_invariants():
    import torch
    w = W.custom(B=1, Hq=4, Hkv=2, N=300, d=128, causal=True, seed=813)
    f8, dev = _inputs(w, 0.5)
    o1, l1 = run_fp8(w, f8, dev, ds=(2.0 ** -5, 2.0 ** -7, 0.01))
    o2, l2 = run_fp8(w, f8, dev, ds=(2.0 ** -7, 2.0 ** -5, 0.02))
    o3, l3 = run_fp8(w, f8, dev, ds=(2.0 ** -5, 2.0 ** -7, 0.01))
    assert bits_equal(l1, l2) and bits_equal(l1, l3)
    assert bits_equal(o1, o3)                               # run to run deterministic
    assert bits_equal((o1.float() * 2).to(torch.bfloat16), o2)


def test_fp8_full_size_sampled_rows():
    """The benchmark's shape and launch (2 x 16 heads x 16384 tokens, causal):
    sampled rows of two (sequence, head) pairs against the oracle row by row."""
    import torch
    w = W.custom(B=2, Hq=16, Hkv=16, N=16384, d=128, causal=True, seed=814)
    f8, dev = _inputs(w)
    o, lse = run_fp8(w, f8, dev)
    o = o.double().cpu().numpy()
    lse = lse.double().cpu().numpy()
    rng = np.random.default_rng(5)
    for b, h in ((0, 3), (1, 15)):
        rows = np.unique(np.r_[0, 1, 127, 128, 16383, rng.integers(0, 16384, 40)])
        sl = slice(b * w.N, (b + 1) * w.N)
        q, k, v = (dequantize(f8[n][sl, h], f8["descale_" + n]) for n in ("q", "k", "v"))
        from oracle import attention_fwd_rows
        o_ref, lse_ref = attention_fwd_rows(q[:, None], k[:, None], v[:, None], w.scale, True,
                                            None, 0, 0, rows)
        bnd = head_o_bound(q, k, v, o_ref, w.scale, True, rows=rows)
        err = np.abs(o[b * w.N + rows, h] - o_ref)
        assert np.all(err <= bnd), f"(b={b}, h={h}) max err/bound {(err / bnd).max():.2f}"
        assert np.abs(lse[h, b * w.N + rows] - lse_ref).max() <= TOL_LSE
    del torch


def test_fp8_empty_and_zero_length():
    import torch
    fa = _fa()
    q = torch.zeros((0, 4, 128), dtype=torch.uint8, device="cuda")
    cu = torch.zeros(3, dtype=torch.int32, device="cuda")
    o, lse = fa.flash_attn_func_fp8(q, q[:, :2], q[:, :2], cu_seqlens=cu, max_seqlen=0)
    torch.cuda.synchronize()
    assert o.shape == (0, 4, 128) and lse.shape == (4, 0)


@pytest.mark.parametrize("v_shift", [0.0, 2.0])
@pytest.mark.parametrize("mix", ["normal", "outliers"])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_fp8_accuracy_against_plain_baseline(d, mix, v_shift):
    """Error of the FP8 forward next to plain FP8 attention (the baseline the
    pages compare FlashAttention-3's FP8 forward with; oracle
    attention_fwd_fp8_plain) and the bf16 forward, all against exact float64
    attention on the unquantised inputs. Inputs (B1 H4 N1024, not causal):
    standard normal Q, K, V, or the same with 0.1 % of the Q and K entries ten
    times larger (outliers that set the per-tensor descale and sharpen some
    rows); V as drawn or shifted by 2 (values with a common offset). Both
    FP8 results are written as fp16 (the finer of the two output types; the
    baseline's float64 O is rounded the same way), the bf16 forward as bf16.
    The FP8 forward's weights are rounded 8 (log2 units) above the running
    max's reference, so the largest is exactly 256 and few fall into e4m3's
    coarse subnormal range, and O is normalised by the sum of the rounded
    weights it was built from. It must be at least as accurate as the
    baseline in every case (emulated on the CPU first: 0.99x the baseline's
    rms error for zero-mean V, down to 0.36x with shifted V and outliers)."""
    import torch
    from oracle import attention_fwd_fp8_plain
    w = W.custom(B=1, Hq=4, Hkv=4, N=1024, d=d, causal=False, seed=830 + d)
    a = W.generate(w, with_grad=False)
    if mix == "outliers":
        rng = np.random.default_rng(831 + d)
        for n in ("q", "k"):
            m = rng.random(a[n].shape) < 1e-3
            a[n] = np.where(m, a[n] * 10.0, a[n]).astype(np.float32)
    a["v"] = (a["v"] + np.float32(v_shift)).astype(np.float32)
    exact, _ = attention_fwd(a["q"], a["k"], a["v"], w.scale, False)
    f8 = W.quantize_e4m3(a)
    dev = {n: torch.from_numpy(f8[n]).cuda().view(torch.float8_e4m3fn) for n in ("q", "k", "v")}
    o8, _ = run_fp8(w, f8, dev, out="fp16")
    plain = attention_fwd_fp8_plain(f8["q"], f8["k"], f8["v"], w.scale, f8["descale_q"],
                                    f8["descale_k"], f8["descale_v"])
    # both written as fp16 (nearest even): the output's own rounding on both sides
    plain = torch.from_numpy(plain).to(torch.float16).double().numpy()
    fa = _fa()
    t = {n: torch.from_numpy(a[n]).to(torch.bfloat16).cuda().view(1, w.N, w.Hq, d)
         for n in ("q", "k", "v")}
    o16, _ = fa.flash_attn_func(t["q"], t["k"], t["v"], causal=False)
    torch.cuda.synchronize()
    rms = lambda x: float(np.sqrt((x ** 2).mean()))
    e8 = rms(o8.double().cpu().numpy() - exact)
    ep = rms(plain - exact)
    e16 = rms(o16.view(w.T, w.Hq, d).double().cpu().numpy() - exact)
    say(f"[fp8 accuracy] d={d} {mix} v_shift={v_shift}: rms error bf16 {e16:.3e}  "
        f"fa_fwd_fp8 {e8:.3e}  plain FP8 {ep:.3e}  (fa_fwd_fp8 / plain = {e8 / ep:.2f})")
    assert e8 <= ep, (e8, ep)
