"""fa_fwd_ex / fa_bwd_ex (one entry point per direction, options in a struct)
against the entry point each set of options names in include/fa.h: same
inputs, and every output must agree bit for bit, since the call runs that
entry point. The routed calls themselves are checked against the oracle by
their own tests."""
import ctypes

import pytest

import workloads as W
from parity_util import bits_equal, say, to_device

pytestmark = pytest.mark.gpu

ROUTES = [
    ("none", dict(), "fwd"),
    ("causal", dict(mask=1), "fwd"),
    ("window", dict(mask=2, window=(40, 7)), "window"),
    ("softcap", dict(mask=1, softcap=5.0), "softcap"),
    ("window_softcap", dict(mask=2, window=(33, 0), softcap=7.5), "window_softcap"),
    ("dropout", dict(mask=1, dropout_p=0.2, dropout_seed=12345), "dropout"),
]


def _run(w, opts, route):
    import torch
    import exact_io_aware_12_amd as fa
    a = W.generate(w, with_grad=True)
    t = to_device(a, w.dtype)
    code = fa.FA_BF16 if w.dtype == "bf16" else fa.FA_FP16
    cu = t["cu_seqlens"].data_ptr() if w.varlen else None
    s = torch.cuda.current_stream().cuda_stream
    o_opts = fa.attn_options(**opts)
    nws = fa.fa_bwd_workspace_size(w.B, w.Hq, w.Hkv, w.N, w.d)
    out = {}
    for via in ("ex", "named"):
        o = torch.empty_like(t["q"])
        lse = torch.empty((w.Hq, w.T), dtype=torch.float32, device="cuda")
        dq, dk, dv = torch.empty_like(t["q"]), torch.empty_like(t["k"]), torch.empty_like(t["v"])
        ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
        head = [t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(), o.data_ptr(),
                lse.data_ptr(), w.B, w.Hq, w.Hkv, w.N, w.d, float(w.scale)]
        bhead = [t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(), o.data_ptr(),
                 t["do"].data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                 w.B, w.Hq, w.Hkv, w.N, w.d, float(w.scale)]
        tail = [cu, code, ws.data_ptr(), nws, s]
        c = int(opts.get("mask", 0) == 1)
        wl, wr = opts.get("window", (-1, -1))
        if via == "ex":
            p = ctypes.addressof(o_opts)
            st_f = fa.fa_fwd_ex(*head, p, cu, code, s)
            st_b = fa.fa_bwd_ex(*bhead, p, *tail)
        elif route == "fwd":
            st_f = fa.fa_fwd(*head, c, cu, code, s)
            st_b = fa.fa_bwd(*bhead, c, *tail)
        elif route == "window":
            st_f = fa.fa_fwd_window(*head, wl, wr, cu, code, s)
            st_b = fa.fa_bwd_window(*bhead, wl, wr, *tail)
        elif route == "softcap":
            st_f = fa.fa_fwd_softcap(*head, c, opts["softcap"], cu, code, s)
            st_b = fa.fa_bwd_softcap(*bhead, c, opts["softcap"], *tail)
        elif route == "window_softcap":
            st_f = fa.fa_fwd_window_softcap(*head, wl, wr, opts["softcap"], cu, code, s)
            st_b = fa.fa_bwd_window_softcap(*bhead, wl, wr, opts["softcap"], *tail)
        else:
            st_f = fa.fa_fwd_dropout(*head, c, opts["dropout_p"], opts["dropout_seed"], cu, code, s)
            st_b = fa.fa_bwd_dropout(*bhead, c, opts["dropout_p"], opts["dropout_seed"], *tail)
        assert st_f == fa.FA_OK and st_b == fa.FA_OK, (via, fa.fa_status_string(st_f),
                                                        fa.fa_status_string(st_b))
        torch.cuda.synchronize()
        out[via] = (o, lse, dq, dk, dv)
    for x, y, n in zip(out["ex"], out["named"], ("O", "LSE", "dQ", "dK", "dV")):
        assert bits_equal(x, y), f"{n} differs between fa_*_ex and the named entry point"


@pytest.mark.parametrize("name,opts,route", ROUTES, ids=[r[0] for r in ROUTES])
@pytest.mark.parametrize("shape", [dict(B=2, Hq=4, Hkv=2, N=200, d=128, dtype="bf16"),
                                   dict(B=0, Hq=2, Hkv=1, N=0, d=64, dtype="fp16",
                                        lens=[70, 0, 129])],
                         ids=["fixed-d128-bf16", "varlen-d64-fp16"])
def test_ex_matches_named_entry_point(name, opts, route, shape):
    w = W.custom(causal=opts.get("mask", 0) == 1, seed=700, backward=True, **shape)
    say(f"[ex] {name} {shape}")
    _run(w, opts, route)
