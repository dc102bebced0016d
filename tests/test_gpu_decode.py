"""GPU parity of fa_fwd_kvcache (decode over a key/value cache) against the
float64 oracle, through the C ABI.

Small caches compare every element, across head dims, dtypes, causal or not,
GQA groups, several new queries per entry, ragged, short and empty cache
lengths, and explicit key-range splits (including ranges that hold no valid
key). The benchmark's decode workload is checked on sampled (entry, head)
units in the launch configuration the benchmark times.
Rows that see no key must come out as exactly O = 0 and LSE = −inf.
"""
import numpy as np
import pytest

import workloads as W
from oracle import kvcache_fwd, kvcache_fwd_units
from parity_util import bits_equal, check_lse, check_o, host64, say, torch_dtype

pytestmark = pytest.mark.gpu


def _fa():
    import exact_io_aware_12_amd as fa   # raises if libfa.so is missing: no fallback
    return fa


def to_dev(arrays, dtype):
    import torch
    out = {}
    for n, a in arrays.items():
        if n == "cache_seqlens":
            out[n] = torch.from_numpy(a).to("cuda")
        else:
            out[n] = torch.from_numpy(a).to(torch_dtype(dtype)).to("cuda")
    return out


def run_decode(w: W.DecodeWorkload, splits=0, t=None):
    import torch
    fa = _fa()
    if t is None:
        t = to_dev(W.generate_decode(w), w.dtype)
    say(f"[fa_fwd_kvcache] {w.name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} Nq={w.Nq} Nk={w.Nk} d={w.d} "
        f"{w.dtype} causal={w.causal} lens={w.cache_lens()[:8]} splits={splits}")
    o, lse = fa.flash_attn_with_kvcache(t["q"], t["k"], t["v"], t["cache_seqlens"],
                                        causal=w.causal, softmax_scale=w.scale,
                                        num_splits=splits)
    torch.cuda.synchronize()
    return o, lse, t


def split_rows(lse_ref):
    """Boolean mask of (head, column) entries that see at least one key."""
    return np.isfinite(lse_ref)


def compare_whole(w, splits=0):
    o, lse, t = run_decode(w, splits)
    o_ref, lse_ref = kvcache_fwd(host64(t["q"]), host64(t["k"]), host64(t["v"]),
                                 t["cache_seqlens"].cpu().numpy(), w.scale, w.causal)
    o_g, lse_g = host64(o), host64(lse)
    seen = split_rows(lse_ref)                       # [Hq, B·Nq]
    # rows with no visible key: exactly zero output and −inf LSE
    empty = ~seen
    if empty.any():
        assert np.all(np.isneginf(lse_g[empty])), "empty rows must have LSE = -inf"
        o_rows = o_g.transpose(2, 0, 1, 3).reshape(w.Hq, w.B * w.Nq, w.d)
        assert np.all(o_rows[empty] == 0.0), "empty rows must have O = 0"
    e, floor, exc = check_o(o_g, o_ref, w.dtype)
    el = check_lse(lse_g[seen], lse_ref[seen]) if seen.any() else 0.0
    say(f"   max|dO|={e:.2e} floor={floor:.2e} exceptions={exc} max|dLSE|={el:.2e} "
        f"empty rows={int(empty.sum())}")
    return o, lse, t


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Nq", [1, 3])
def test_small_caches(dtype, d, causal, Nq):
    # lengths: full, ragged (not a multiple of the 32-key tile), 1, shorter than Nq, 0
    lens = [200, 77, 1, 2, 0]
    compare_whole(W.decode_custom(B=5, Hq=8, Hkv=2, Nq=Nq, Nk=200, d=d, dtype=dtype,
                                  causal=causal, seed=300 + d + Nq, lens=lens))


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_head_dim_256(dtype, causal):
    compare_whole(W.decode_custom(B=3, Hq=8, Hkv=2, Nq=2, Nk=400, d=256, dtype=dtype,
                                  causal=causal, seed=47, lens=[400, 93, 0]))


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 13])
def test_explicit_splits(splits):
    """Ranges that end inside a tile, and ranges past every valid key (13 x 32 > 300)."""
    compare_whole(W.decode_custom(B=3, Hq=4, Hkv=1, Nq=2, Nk=300, d=128, dtype="bf16",
                                  causal=True, seed=41, lens=[300, 150, 31]), splits=splits)


def test_rows_beyond_one_block():
    """(Hq/Hkv)·Nq = 40 rows per KV head: two 32-row blocks."""
    compare_whole(W.decode_custom(B=2, Hq=8, Hkv=1, Nq=5, Nk=96, d=64, dtype="fp16",
                                  causal=True, seed=42, lens=[96, 61]))


@pytest.mark.parametrize("causal", [False, True])
def test_mha_and_long_cache(causal):
    compare_whole(W.decode_custom(B=2, Hq=4, Hkv=4, Nq=1, Nk=3000, d=128, dtype="bf16",
                                  causal=causal, seed=43, lens=[3000, 2049]))


def test_stress_peaked_queries():
    """Large logits (queries ×8): the reference max is raised inside the cache range."""
    w = W.decode_custom(B=2, Hq=8, Hkv=2, Nq=2, Nk=500, d=128, dtype="bf16", causal=True,
                        seed=44, lens=[500, 333])
    a = W.generate_decode(w)
    a["q"] = a["q"] * 8.0
    t = to_dev(a, w.dtype)
    o, lse, _ = run_decode(w, t=t)
    o_ref, lse_ref = kvcache_fwd(host64(t["q"]), host64(t["k"]), host64(t["v"]),
                                 t["cache_seqlens"].cpu().numpy(), w.scale, w.causal)
    check_o(host64(o), o_ref, w.dtype)
    check_lse(host64(lse), lse_ref)


def test_deterministic():
    w = W.decode_custom(B=2, Hq=8, Hkv=2, Nq=3, Nk=700, d=128, dtype="bf16", causal=True,
                        seed=45, lens=[700, 512])
    o1, l1, t = run_decode(w)
    o2, l2, _ = run_decode(w, t=t)
    assert bits_equal(o1, o2) and bits_equal(l1, l2)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_matches_full_attention_when_queries_are_the_sequence(dtype):
    """Nq = L = Nk, causal: the decode result equals fa_fwd on the same sequences.

    bf16 LSEs come from fp32 sums of the unrounded P on both paths and agree
    to 1e-4. fp16 LSEs come from the sums of P rounded to fp16 (at most 2^-11
    relative each), taken against different reference maxima on the two
    paths, so they agree to twice that bound, ~1e-3."""
    import torch
    fa = _fa()
    w = W.decode_custom(B=2, Hq=4, Hkv=2, Nq=96, Nk=96, d=128, dtype=dtype, causal=True, seed=46)
    o, lse, t = run_decode(w)
    o_f, lse_f = fa.flash_attn_func(t["q"], t["k"], t["v"], causal=True, softmax_scale=w.scale)
    torch.cuda.synchronize()
    # the two paths may round an output to neighbouring values: one ulp apart
    ulp = 2.0 ** -10 if dtype == "fp16" else 2.0 ** -7
    np.testing.assert_allclose(host64(o), host64(o_f), rtol=ulp, atol=2e-3)
    np.testing.assert_allclose(host64(lse), host64(lse_f), atol=1e-3 if dtype == "fp16" else 1e-4)


@pytest.mark.parametrize("name", ["decode_llama", "decode_multi"])
def test_benchmark_workload_every_unit(name):
    """The benchmark's workloads at full size, automatic splits: every
    (entry, query head) unit against the oracle."""
    w = W.DECODE_WORKLOADS[name]
    o, lse, t = run_decode(w)
    units = [(b, h) for b in range(w.B) for h in range(w.Hq)]
    ref = kvcache_fwd_units(t["q"], t["k"], t["v"], t["cache_seqlens"].cpu(), w.scale, w.causal,
                            units)
    lse_h, o_h = host64(lse), host64(o)
    for (b, h), (O, L) in ref.items():
        check_o(o_h[b, :, h], O, w.dtype, what=f"O[{b},:,{h}]")
        check_lse(lse_h[h, b * w.Nq:(b + 1) * w.Nq], L, what=f"LSE[{h},{b}]")
    say(f"   {len(units)} units ok")
