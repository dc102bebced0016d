"""GPU parity of fa_fwd_kvcache_local (decode with a sliding window behind
each query and/or a soft cap) against the float64 decode oracle with the same
options, through the C ABI.

Windows narrower than a key tile, spanning several tiles and wider than the
cache, caps from 1.5 to 50, causal or not, several new queries, ragged, short
and empty cache lengths, explicit key-range splits, head dims 64/128/256 and
both dtypes; window -1 with cap 0 must equal fa_fwd_kvcache bit for bit.
"""
import numpy as np
import pytest

import workloads as W
from oracle import kvcache_fwd
from parity_util import bits_equal, check_lse, check_o, host64, say, torch_dtype

pytestmark = pytest.mark.gpu


def _fa():
    import exact_io_aware_12_amd as fa   # raises if libfa.so is missing: no fallback
    return fa


def _inputs(w):
    import torch
    a = W.generate_decode(w)
    td = torch_dtype(w.dtype)
    return {n: (torch.from_numpy(x).cuda() if n == "cache_seqlens"
                else torch.from_numpy(x).to(td).cuda()) for n, x in a.items()}


def compare(w, window_left, softcap, splits=0, t=None):
    import torch
    fa = _fa()
    t = _inputs(w) if t is None else t
    say(f"[fa_fwd_kvcache_local] B={w.B} Hq={w.Hq} Hkv={w.Hkv} Nq={w.Nq} Nk={w.Nk} d={w.d} "
        f"{w.dtype} causal={w.causal} lens={w.cache_lens()} wl={window_left} cap={softcap} "
        f"splits={splits}")
    o, lse = fa.flash_attn_with_kvcache(t["q"], t["k"], t["v"], t["cache_seqlens"],
                                        causal=w.causal, softmax_scale=w.scale,
                                        num_splits=splits, window_left=window_left,
                                        softcap=softcap)
    torch.cuda.synchronize()
    o_ref, lse_ref = kvcache_fwd(host64(t["q"]), host64(t["k"]), host64(t["v"]),
                                 t["cache_seqlens"].cpu().numpy(), w.scale, w.causal,
                                 window_left=None if window_left < 0 else window_left,
                                 softcap=softcap or None)
    o_g, lse_g = host64(o), host64(lse)
    seen = np.isfinite(lse_ref)
    if (~seen).any():
        assert np.all(np.isneginf(lse_g[~seen]))
        assert np.all(o_g.transpose(2, 0, 1, 3).reshape(w.Hq, w.B * w.Nq, w.d)[~seen] == 0.0)
    e, _, _ = check_o(o_g, o_ref, w.dtype)
    el = check_lse(lse_g[seen], lse_ref[seen]) if seen.any() else 0.0
    say(f"   max|dO|={e:.2e} max|dLSE|={el:.2e}")
    return o, lse, t


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("wl,cap", [(0, 0.0), (5, 0.0), (100, 0.0), (-1, 1.5), (40, 50.0),
                                    (5000, 5.0)])
def test_local_decode(dtype, d, causal, wl, cap):
    lens = [300, 77, 1, 2, 0]
    compare(W.decode_custom(B=5, Hq=8, Hkv=2, Nq=3, Nk=300, d=d, dtype=dtype, causal=causal,
                            seed=600 + d, lens=lens), wl, cap)


@pytest.mark.parametrize("splits", [1, 3, 7])
def test_local_explicit_splits(splits):
    compare(W.decode_custom(B=3, Hq=4, Hkv=1, Nq=2, Nk=900, d=128, dtype="bf16", causal=True,
                            seed=61, lens=[900, 450, 31]), 200, 30.0, splits=splits)


def test_local_long_cache_window():
    """Gemma-2-like local layer: 4096-key window over 9000-token caches, cap 50."""
    compare(W.decode_custom(B=2, Hq=16, Hkv=8, Nq=1, Nk=9000, d=256, dtype="bf16", causal=True,
                            seed=62, lens=[9000, 5000]), 4096, 50.0)


def test_no_window_no_cap_equals_plain_decode():
    import torch
    fa = _fa()
    w = W.decode_custom(B=3, Hq=8, Hkv=2, Nq=2, Nk=700, d=128, dtype="bf16", causal=True,
                        seed=63, lens=[700, 512, 33])
    t = _inputs(w)
    o1, l1 = fa.flash_attn_with_kvcache(t["q"], t["k"], t["v"], t["cache_seqlens"], causal=True)
    # window_left = Nk is no restriction; the split count must match the plain call's
    n = fa.fa_kvcache_num_splits(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d)
    o2, l2 = fa.flash_attn_with_kvcache(t["q"], t["k"], t["v"], t["cache_seqlens"], causal=True,
                                        num_splits=n, window_left=w.Nk)
    o3, l3 = fa.flash_attn_with_kvcache(t["q"], t["k"], t["v"], t["cache_seqlens"], causal=True,
                                        num_splits=n)
    torch.cuda.synchronize()
    assert bits_equal(o1, o3) and bits_equal(l1, l3)
    assert bits_equal(o2, o3) and bits_equal(l2, l3)
