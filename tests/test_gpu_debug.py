"""The FA_DEBUG build of the library (libfa_debug.so) on the GPU, through the C ABI.

That build copies every cu_seqlens argument to the host and checks it with
fa_check_cu_seqlens before launching, and waits for each launch. Here:
  - with a valid packed batch its forward and backward give results bitwise
    equal to the release library's (the same kernels);
  - a cu_seqlens array that breaks the packing convention (first entry not 0,
    a decreasing entry, a sequence longer than N, or than Nk for the kvlen
    keys) returns FA_ERR_INVALID_ARG from fa_fwd, fa_bwd, fa_fwd_kvlen and
    fa_bwd_kvlen, and the outputs keep their sentinel contents: nothing was
    launched. (The release library is never called with such an array.)
"""
import ctypes
import os

import numpy as np
import pytest

import workloads as W
from parity_util import bits_equal, say, to_device

pytestmark = pytest.mark.gpu


def _libs():
    import exact_io_aware_12_amd as fa
    path = os.path.join(os.path.dirname(fa.lib_path()), "libfa_debug.so")
    assert os.path.exists(path), f"{path} is missing: build it with build.py --all"
    L = ctypes.CDLL(path)
    for name, (res, args) in fa._SIGS.items():
        f = getattr(L, name)
        f.restype, f.argtypes = res, args
    return fa, L


def _stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


LENS = (70, 0, 129, 33)


def _setup():
    import torch
    w = W.custom(B=0, Hq=4, Hkv=2, N=0, d=128, dtype="bf16", causal=True, seed=11, lens=LENS,
                 backward=True)
    t = to_device(W.generate(w, with_grad=True), w.dtype)
    return w, t


def _fwd(lib, fa, w, t, cu):
    import torch
    o = torch.full_like(t["q"], float("nan"))
    lse = torch.full((w.Hq, w.T), float("nan"), dtype=torch.float32, device="cuda")
    st = lib.fa_fwd(t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(), o.data_ptr(),
                    lse.data_ptr(), w.B, w.Hq, w.Hkv, w.N, w.d, float(w.scale), 1, cu,
                    fa.FA_BF16, _stream())
    torch.cuda.synchronize()
    return st, o, lse


def _bwd(lib, fa, w, t, o, lse, cu):
    import torch
    g = {n: torch.full_like(t[s], float("nan")) for n, s in (("dq", "q"), ("dk", "k"), ("dv", "v"))}
    nws = fa.fa_bwd_workspace_size(w.B, w.Hq, w.Hkv, w.N, w.d)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
    st = lib.fa_bwd(t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(), o.data_ptr(),
                    t["do"].data_ptr(), lse.data_ptr(), g["dq"].data_ptr(), g["dk"].data_ptr(),
                    g["dv"].data_ptr(), w.B, w.Hq, w.Hkv, w.N, w.d, float(w.scale), 1, cu,
                    fa.FA_BF16, ws.data_ptr(), nws, _stream())
    torch.cuda.synchronize()
    return st, g


def test_debug_build_matches_release_bitwise():
    fa, dbg = _libs()
    w, t = _setup()
    cu = t["cu_seqlens"].data_ptr()
    say(f"[debug] varlen lens={LENS} Hq4 Hkv2 d128 bf16 causal: release vs FA_DEBUG")
    st_r, o_r, lse_r = _fwd(fa.lib, fa, w, t, cu)
    st_d, o_d, lse_d = _fwd(dbg, fa, w, t, cu)
    assert st_r == fa.FA_OK and st_d == fa.FA_OK, (st_r, st_d)
    assert bits_equal(o_r, o_d) and bits_equal(lse_r, lse_d)
    st_r, g_r = _bwd(fa.lib, fa, w, t, o_r, lse_r, cu)
    st_d, g_d = _bwd(dbg, fa, w, t, o_r, lse_r, cu)
    assert st_r == fa.FA_OK and st_d == fa.FA_OK, (st_r, st_d)
    for n in ("dq", "dk", "dv"):
        assert bits_equal(g_r[n], g_d[n]), n


def _bad_arrays(N):
    T = sum(LENS)
    return {
        "first entry not 0": [3, 73, 73, 202, T],
        "decreasing": [0, 70, 60, 199, T],
        "longer than N": [0, 70, 70, 70 + N + 1, 70 + N + 1],
    }


@pytest.mark.parametrize("case", ["first entry not 0", "decreasing", "longer than N"])
def test_debug_build_rejects_bad_cu_seqlens(case):
    import torch
    fa, dbg = _libs()
    w, t = _setup()
    bad = torch.tensor(_bad_arrays(w.N)[case], dtype=torch.int32, device="cuda")
    good = t["cu_seqlens"].data_ptr()
    say(f"[debug] bad cu_seqlens ({case}): {bad.tolist()}")
    st, o, lse = _fwd(dbg, fa, w, t, bad.data_ptr())
    assert st == fa.FA_ERR_INVALID_ARG, fa.fa_status_string(st)
    assert torch.isnan(o).all() and torch.isnan(lse).all(), "fa_fwd wrote its outputs"
    # a valid forward for the backward's inputs, then the backward with the bad array
    st, o, lse = _fwd(dbg, fa, w, t, good)
    assert st == fa.FA_OK
    st, g = _bwd(dbg, fa, w, t, o, lse, bad.data_ptr())
    assert st == fa.FA_ERR_INVALID_ARG, fa.fa_status_string(st)
    assert all(torch.isnan(x).all() for x in g.values()), "fa_bwd wrote its outputs"
    # kvlen: a bad query array, then a bad key array next to a good query array
    for cq, ck, what in ((bad.data_ptr(), good, "queries"), (good, bad.data_ptr(), "keys")):
        o2 = torch.full_like(t["q"], float("nan"))
        st = dbg.fa_fwd_kvlen(t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(),
                              o2.data_ptr(), lse.data_ptr(), w.B, w.Hq, w.Hkv, w.N, w.N, w.d,
                              float(w.scale), 1, cq, ck, fa.FA_BF16, _stream())
        torch.cuda.synchronize()
        assert st == fa.FA_ERR_INVALID_ARG, (what, fa.fa_status_string(st))
        assert torch.isnan(o2).all(), f"fa_fwd_kvlen ({what}) wrote its output"
        nws = fa.fa_bwd_workspace_size(w.B, w.Hq, w.Hkv, max(w.N, 1), w.d)
        ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
        dq = torch.full_like(t["q"], float("nan"))
        st = dbg.fa_bwd_kvlen(t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(),
                              o.data_ptr(), t["do"].data_ptr(), lse.data_ptr(), dq.data_ptr(),
                              g["dk"].data_ptr(), g["dv"].data_ptr(), w.B, w.Hq, w.Hkv, w.N, w.N,
                              w.d, float(w.scale), 1, cq, ck, fa.FA_BF16, ws.data_ptr(), nws,
                              _stream())
        torch.cuda.synchronize()
        assert st == fa.FA_ERR_INVALID_ARG, (what, fa.fa_status_string(st))
        assert torch.isnan(dq).all(), f"fa_bwd_kvlen ({what}) wrote dQ"
