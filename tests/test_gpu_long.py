"""Very long sequences: 131,072 tokens, eight times the benchmark's length, so
tile counts, token offsets and LSE indices run well past the sizes the other
tests reach. The forward is checked on sampled query rows (each computed by
the oracle against all keys), decode over 128k-token caches on every
(entry, query head) unit.
"""
import numpy as np
import pytest

import workloads as W
from oracle import attention_fwd_rows, kvcache_fwd_units
from parity_util import check_lse, check_o, host64, say, to_device, torch_dtype

pytestmark = pytest.mark.gpu

N_LONG = 131072


@pytest.mark.parametrize("causal", [False, True])
def test_forward_128k(causal):
    import torch
    import exact_io_aware_12_amd as fa
    w = W.custom(B=1, Hq=2, Hkv=1, N=N_LONG, d=128, dtype="bf16", causal=causal, seed=990)
    t = to_device(W.generate(w, with_grad=False), w.dtype)
    say(f"[long] fa_fwd N={w.N} Hq={w.Hq} Hkv={w.Hkv} d={w.d} causal={causal}")
    o, lse = fa.flash_attn_func(t["q"].view(1, w.N, w.Hq, w.d), t["k"].view(1, w.N, w.Hkv, w.d),
                                t["v"].view(1, w.N, w.Hkv, w.d), causal=causal)
    torch.cuda.synchronize()
    rng = np.random.default_rng(991)
    rows = sorted({0, 1, 127, 128, N_LONG // 2, N_LONG - 129, N_LONG - 1}
                  | {int(x) for x in rng.integers(0, N_LONG, 6)})
    o2 = o.view(w.N, w.Hq, w.d)
    for h in range(w.Hq):
        o_ref, l_ref = attention_fwd_rows(t["q"], t["k"], t["v"], w.scale, causal,
                                          w.cu_seqlens(), 0, h, rows)
        gi = torch.as_tensor(rows, device=o.device)
        check_o(host64(o2[gi, h]), o_ref, w.dtype, f"O head {h}")
        check_lse(host64(lse[h, gi]), l_ref, f"LSE head {h}")
    say(f"   {len(rows)} rows x {w.Hq} heads ok")


def test_decode_128k_cache():
    import torch
    import exact_io_aware_12_amd as fa
    w = W.decode_custom(B=2, Hq=8, Hkv=2, Nq=1, Nk=N_LONG, d=128, dtype="bf16", causal=True,
                        seed=992, lens=[N_LONG, 100003])
    a = W.generate_decode(w)
    td = torch_dtype(w.dtype)
    q, k, v = (torch.from_numpy(a[n]).to(td).cuda() for n in ("q", "k", "v"))
    lens = torch.from_numpy(a["cache_seqlens"]).cuda()
    say(f"[long] fa_fwd_kvcache Nk={w.Nk} lens={w.cache_lens()}")
    o, lse = fa.flash_attn_with_kvcache(q, k, v, lens, causal=True)
    torch.cuda.synchronize()
    units = [(b, h) for b in range(w.B) for h in range(w.Hq)]
    ref = kvcache_fwd_units(q, k, v, lens.cpu(), w.scale, True, units)
    lse_h = host64(lse)
    for (b, h), (O, L) in ref.items():
        check_o(host64(o[b, :, h]), O, w.dtype, what=f"O[{b},:,{h}]")
        check_lse(lse_h[h, b:b + 1], L, what=f"LSE[{h},{b}]")
    say(f"   {len(units)} units ok")
