"""The entry points inside a HIP graph: fa_fwd + fa_bwd (training step),
fa_fwd_kvcache and fa_fwd_kvcache_fp8 (decode) are captured once with
torch.cuda.graph and replayed several times, with the program's own eager
work and synchronisations between the replays; every replay must reproduce
the eager results bit for bit (the kernels are deterministic and write every
workspace byte they later read, so no replay depends on leftover memory).
"""
import numpy as np
import pytest

import workloads as W
from parity_util import bits_equal, say, torch_dtype

pytestmark = pytest.mark.gpu


def _fa():
    import exact_io_aware_12_amd as fa   # raises if libfa.so is missing: no fallback
    return fa


def _replay_and_check(graph, outs, refs, scribble, what):
    import torch
    for r in range(4):
        for t in outs:           # eager work between replays: clobber the outputs
            t.fill_(float("nan")) if t.dtype.is_floating_point else t.zero_()
        scribble()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (o, ref) in enumerate(zip(outs, refs)):
            assert bits_equal(o, ref), f"{what}: replay {r}, output {i} differs from eager"
    say(f"   {what}: 4 replays bit-identical to eager")


@pytest.mark.parametrize("causal", [False, True])
def test_training_step_graph(causal):
    import torch
    fa = _fa()
    rng = np.random.default_rng(81)
    B, N, Hq, Hkv, d = 2, 700, 8, 2, 128
    mk = lambda *s: torch.from_numpy(rng.standard_normal(s, dtype=np.float32)).to(
        torch.bfloat16).cuda()
    q, k, v, do = mk(B, N, Hq, d), mk(B, N, Hkv, d), mk(B, N, Hkv, d), mk(B, N, Hq, d)
    ws = torch.empty(fa.fa_bwd_workspace_size(B, Hq, Hkv, N, d), dtype=torch.uint8, device="cuda")
    say(f"[graph fa_fwd+fa_bwd] B={B} N={N} Hq={Hq} Hkv={Hkv} d={d} causal={causal}")
    o_ref, lse_ref = fa.flash_attn_func(q, k, v, causal=causal)
    dq_ref, dk_ref, dv_ref = fa.flash_attn_backward(do, q, k, v, o_ref, lse_ref, causal=causal,
                                                    workspace=ws)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):   # warm the binding's allocations outside the capture
        fa.flash_attn_func(q, k, v, causal=causal)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        o, lse = fa.flash_attn_func(q, k, v, causal=causal)
        dq, dk, dv = fa.flash_attn_backward(do, q, k, v, o, lse, causal=causal, workspace=ws)
    scratch = torch.empty(1 << 24, dtype=torch.float32, device="cuda")
    _replay_and_check(g, [o, lse, dq, dk, dv], [o_ref, lse_ref, dq_ref, dk_ref, dv_ref],
                      lambda: (ws.fill_(255), scratch.normal_()), "fwd+bwd")


@pytest.mark.parametrize("fp8", [False, True])
def test_decode_graph(fp8):
    import torch
    fa = _fa()
    w = W.decode_custom(B=4, Hq=16, Hkv=4, Nq=1, Nk=2000, d=128, dtype="bf16", causal=True,
                        seed=82, lens=[2000, 1500, 33, 0], kv_cache="e4m3" if fp8 else "same")
    a = W.decode_fp8_inputs(w) if fp8 else W.generate_decode(w)
    td = torch_dtype(w.dtype)
    q = torch.from_numpy(a["q"]).to(td).cuda()
    if fp8:
        k, v = torch.from_numpy(a["k"]).cuda(), torch.from_numpy(a["v"]).cuda()
        extra = dict(descale_k=a["descale_k"], descale_v=a["descale_v"])
    else:
        k, v = torch.from_numpy(a["k"]).to(td).cuda(), torch.from_numpy(a["v"]).to(td).cuda()
        extra = {}
    lens = torch.from_numpy(a["cache_seqlens"]).cuda()
    ws = torch.empty(fa.fa_fwd_kvcache_workspace_size(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, 0),
                     dtype=torch.uint8, device="cuda")
    say(f"[graph decode] fp8={fp8} lens={w.cache_lens()}")
    o_ref, lse_ref = fa.flash_attn_with_kvcache(q, k, v, lens, causal=True, workspace=ws, **extra)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        o, lse = fa.flash_attn_with_kvcache(q, k, v, lens, causal=True, workspace=ws, **extra)
    _replay_and_check(g, [o, lse], [o_ref, lse_ref], lambda: ws.fill_(255), "decode")
