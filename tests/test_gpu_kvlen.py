"""GPU parity of fa_fwd_kvlen (queries and keys of different lengths) against
the float64 oracle, through the C ABI.

The oracle is the decode oracle's per-(sequence, head) function, which places
the Lq queries of a sequence at its last Lq key positions (bottom-right causal
alignment) and gives a query with no visible key O = 0 and LSE = −inf. Cases:
fixed length with Nq < Nk (chunked prefill), Nq = Nk (equal to fa_fwd bit for
bit), Nq > Nk (causal rows before every key), Nk = 0; head dims 64/128/256,
fp16/bf16, causal or not, GQA; varlen with ragged query and key lengths
including empty sequences on either side; and the chunked-prefill workload at
full size on sampled units.
"""
import numpy as np
import pytest

from oracle.decode import kvcache_fwd, kvcache_head
from parity_util import bits_equal, check_lse, check_o, host64, say, torch_dtype

pytestmark = pytest.mark.gpu


def _fa():
    import exact_io_aware_12_amd as fa   # raises if libfa.so is missing: no fallback
    return fa


def _randn(rng, shape, dtype):
    import torch
    return torch.from_numpy(rng.standard_normal(shape, dtype=np.float32)).to(
        torch_dtype(dtype)).cuda()


def check_rows(o_g, lse_g, o_ref, lse_ref, dtype):
    """Rows with no visible key exactly O = 0, LSE = −inf; the rest to tolerance.
    o_* [rows, Hq, d], lse_* [Hq, rows]."""
    seen = np.isfinite(lse_ref)
    empty = ~seen
    if empty.any():
        assert np.all(np.isneginf(lse_g[empty])), "rows with no key must have LSE = -inf"
        assert np.all(o_g.transpose(1, 0, 2)[empty] == 0.0), "rows with no key must have O = 0"
    e, floor, exc = check_o(o_g, o_ref, dtype)
    el = check_lse(lse_g[seen], lse_ref[seen]) if seen.any() else 0.0
    say(f"   max|dO|={e:.2e} floor={floor:.2e} exceptions={exc} max|dLSE|={el:.2e} "
        f"empty rows={int(empty.sum())}")


def run_fixed(B, Hq, Hkv, Nq, Nk, d, dtype, causal, seed):
    import torch
    fa = _fa()
    rng = np.random.default_rng(seed)
    q = _randn(rng, (B, Nq, Hq, d), dtype)
    k = _randn(rng, (B, Nk, Hkv, d), dtype)
    v = _randn(rng, (B, Nk, Hkv, d), dtype)
    say(f"[fa_fwd_kvlen] B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} {dtype} causal={causal}")
    o, lse = fa.flash_attn_kvlen_func(q, k, v, causal=causal)
    torch.cuda.synchronize()
    return q, k, v, o, lse


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Nq,Nk", [(200, 700), (130, 130), (300, 77), (64, 0), (1, 513)])
def test_fixed_length(dtype, d, causal, Nq, Nk):
    B, Hq, Hkv = 2, 4, 2
    q, k, v, o, lse = run_fixed(B, Hq, Hkv, Nq, Nk, d, dtype, causal, 700 + d + Nq + Nk)
    o_ref, lse_ref = kvcache_fwd(host64(q), host64(k), host64(v), [Nk] * B,
                                 1.0 / np.sqrt(d), causal)
    check_rows(host64(o).reshape(B * Nq, Hq, d), host64(lse),
               o_ref.reshape(B * Nq, Hq, d), lse_ref, dtype)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_equal_lengths_match_fa_fwd_bitwise(dtype, causal):
    """With Lq = Lk the kernel runs fa_fwd's arithmetic: identical bits."""
    import torch
    fa = _fa()
    q, k, v, o, lse = run_fixed(2, 8, 2, 333, 333, 128, dtype, causal, 71)
    o2, lse2 = fa.flash_attn_func(q, k, v, causal=causal)
    torch.cuda.synchronize()
    assert bits_equal(o, o2) and bits_equal(lse, lse2)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_ragged(dtype, d, causal):
    """Per-sequence query and key lengths: more keys than queries, equal, fewer
    (causal rows before every key), no keys, no queries, lengths off the tiles."""
    import torch
    fa = _fa()
    lq = [100, 257, 64, 40, 0, 1, 129]
    lk = [900, 257, 10, 0, 50, 1, 1000]
    Hq, Hkv = 6, 2
    cq = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    rng = np.random.default_rng(72 + d)
    q = _randn(rng, (int(cq[-1]), Hq, d), dtype)
    k = _randn(rng, (int(ck[-1]), Hkv, d), dtype)
    v = _randn(rng, (int(ck[-1]), Hkv, d), dtype)
    say(f"[fa_fwd_kvlen varlen] lq={lq} lk={lk} d={d} {dtype} causal={causal}")
    o, lse = fa.flash_attn_kvlen_func(q, k, v, causal=causal,
                                      cu_seqlens_q=torch.from_numpy(cq).cuda(),
                                      cu_seqlens_k=torch.from_numpy(ck).cuda(),
                                      max_seqlen_q=max(lq), max_seqlen_k=max(lk))
    torch.cuda.synchronize()
    q64, k64, v64 = host64(q), host64(k), host64(v)
    o_ref = np.zeros_like(q64)
    lse_ref = np.full((Hq, int(cq[-1])), -np.inf)
    g = Hq // Hkv
    for s in range(len(lq)):
        a, b, ka, kb = cq[s], cq[s + 1], ck[s], ck[s + 1]
        if b <= a:
            continue
        for h in range(Hq):
            O, L = kvcache_head(q64[a:b, h], k64[ka:kb, h // g], v64[ka:kb, h // g],
                                1.0 / np.sqrt(d), causal)
            o_ref[a:b, h] = O
            lse_ref[h, a:b] = L
    check_rows(host64(o), host64(lse), o_ref, lse_ref, dtype)


def test_deterministic():
    import torch
    fa = _fa()
    q, k, v, o, lse = run_fixed(2, 8, 2, 300, 1000, 128, "bf16", True, 73)
    o2, lse2 = fa.flash_attn_kvlen_func(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert bits_equal(o, o2) and bits_equal(lse, lse2)


def test_chunked_prefill_workload_sampled():
    """The benchmark's chunked-prefill shape (B=4, Hq=32, Hkv=8, 2048 new tokens
    over 8192 keys, d=128, bf16, causal) at full size; sampled (entry, head) units."""
    import workloads as W
    fa = _fa()
    import torch
    w = W.KVLEN_WORKLOADS["prefill_chunk"]
    t = W.generate_kvlen(w)
    td = torch_dtype(w.dtype)
    q, k, v = (torch.from_numpy(t[n]).to(td).cuda() for n in ("q", "k", "v"))
    say(f"[fa_fwd_kvlen] {w.name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} Nq={w.Nq} Nk={w.Nk} d={w.d}")
    o, lse = fa.flash_attn_kvlen_func(q, k, v, causal=w.causal)
    torch.cuda.synchronize()
    g = w.Hq // w.Hkv
    lse_h = host64(lse)
    for b, h in [(0, 0), (w.B - 1, w.Hq - 1), (1, 17)]:
        O, L = kvcache_head(host64(q[b, :, h]), host64(k[b, :, h // g]), host64(v[b, :, h // g]),
                            w.scale, w.causal)
        check_o(host64(o[b, :, h]), O, w.dtype, what=f"O[{b},:,{h}]")
        check_lse(lse_h[h, b * w.Nq:(b + 1) * w.Nq], L, what=f"LSE[{h},{b}]")
