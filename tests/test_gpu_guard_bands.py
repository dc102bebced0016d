"""Out-of-bounds write detection: every output and workspace of the entry
points sits between two guard bands of a NaN bit pattern, and after each call
(through the C ABI) the bands must be bit-for-bit untouched. Parity tests read
only the outputs themselves, so a write past them would go unseen there.
Ragged small shapes (lengths 1, 33, 129, 300; packed batches with empty
sequences) and one full-size training step (B2 H16 N16384 d128) are covered.
"""
import numpy as np
import pytest

import workloads as W
from parity_util import say, to_device

pytestmark = pytest.mark.gpu

GUARD = 4096   # bytes on each side (a multiple of 256 keeps the outputs aligned)
PATTERN = {2: 0x7FC1, 4: 0x7FC00001}   # quiet NaNs no kernel writes as a result


class Guarded:
    """A device buffer [guard | body | guard] whose body is a tensor of `shape`."""

    def __init__(self, shape, dtype):
        import torch
        self.shape, self.dtype = tuple(shape), dtype
        es = torch.empty((), dtype=dtype).element_size()
        n = int(np.prod(shape)) if len(shape) else 1
        self.g = GUARD // es
        self.buf = torch.empty(n + 2 * self.g, dtype=dtype, device="cuda")
        iv = {2: torch.int16, 4: torch.int32, 1: torch.int8}[es]
        pat = PATTERN.get(es, 0xA5)
        if pat >= 1 << (8 * es - 1):
            pat -= 1 << (8 * es)
        self.bits = self.buf.view(iv)
        self.bits.fill_(pat)                         # the body too: outputs start as NaN
        self.pat = pat
        self.body = self.buf[self.g:self.g + n].view(self.shape)

    def ptr(self):
        return self.body.data_ptr()

    def check(self, what):
        lo, hi = self.bits[:self.g], self.bits[-self.g:]
        bad_lo = int((lo != self.pat).sum())
        bad_hi = int((hi != self.pat).sum())
        assert bad_lo == 0 and bad_hi == 0, \
            f"{what}: {bad_lo} elements written before and {bad_hi} after the buffer"


def _fa():
    import exact_io_aware_12_amd as fa
    return fa


def _stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


def fwd_bwd_guarded(w, entry="plain", extra=None):
    """fa_fwd(+variant) then fa_bwd(+variant) into guarded buffers; checks every band."""
    import torch
    fa = _fa()
    a = W.generate(w, with_grad=True)
    t = to_device(a, w.dtype)
    td = t["q"].dtype
    code = fa.FA_BF16 if w.dtype == "bf16" else fa.FA_FP16
    cu = t["cu_seqlens"].data_ptr() if w.varlen else None
    say(f"[guards] {entry} B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} d={w.d} {w.dtype} "
        f"causal={w.causal} varlen={w.varlen} T={w.T}")
    o = Guarded((w.T, w.Hq, w.d), td)
    lse = Guarded((w.Hq, w.T), torch.float32)
    head = [t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(), o.ptr(), lse.ptr(),
            w.B, w.Hq, w.Hkv, w.N, w.d, float(w.scale)]
    c = int(w.causal)
    if entry == "plain":
        st = fa.fa_fwd(*head, c, cu, code, _stream())
    elif entry == "window":
        st = fa.fa_fwd_window(*head, 40, 7, cu, code, _stream())
    elif entry == "softcap":
        st = fa.fa_fwd_softcap(*head, c, 5.0, cu, code, _stream())
    elif entry == "dropout":
        st = fa.fa_fwd_dropout(*head, c, 0.2, 77, cu, code, _stream())
    assert st == fa.FA_OK, fa.fa_status_string(st)
    torch.cuda.synchronize()
    o.check("O")
    lse.check("LSE")
    assert not torch.isnan(o.body).any() and not torch.isnan(lse.body).any(), \
        "the forward left output elements unwritten"
    dq = Guarded((w.T, w.Hq, w.d), td)
    dk = Guarded((w.T, w.Hkv, w.d), td)
    dv = Guarded((w.T, w.Hkv, w.d), td)
    nws = fa.fa_bwd_workspace_size(w.B, w.Hq, w.Hkv, w.N, w.d)
    ws = Guarded((max(nws, 1),), torch.uint8)
    ptrs = [t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(), o.ptr(), t["do"].data_ptr(),
            lse.ptr(), dq.ptr(), dk.ptr(), dv.ptr(), w.B, w.Hq, w.Hkv, w.N, w.d, float(w.scale)]
    tail = [cu, code, ws.ptr(), nws, _stream()]
    if entry == "plain":
        st = fa.fa_bwd(*ptrs, c, *tail)
    elif entry == "window":
        st = fa.fa_bwd_window(*ptrs, 40, 7, *tail)
    elif entry == "softcap":
        st = fa.fa_bwd_softcap(*ptrs, c, 5.0, *tail)
    elif entry == "dropout":
        st = fa.fa_bwd_dropout(*ptrs, c, 0.2, 77, *tail)
    assert st == fa.FA_OK, fa.fa_status_string(st)
    torch.cuda.synchronize()
    for g, n in ((dq, "dQ"), (dk, "dK"), (dv, "dV"), (ws, "workspace")):
        g.check(n)
    for g, n in ((dq, "dQ"), (dk, "dK"), (dv, "dV")):
        assert not torch.isnan(g.body).any(), f"the backward left {n} elements unwritten"


SMALL = [dict(B=2, Hq=2, Hkv=1, N=n, d=d, dtype=dt, causal=c, seed=600 + n)
         for n in (1, 33, 129, 300) for d in (64, 128) for dt, c in (("fp16", False), ("bf16", True))]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"N{c['N']}-d{c['d']}-{c['dtype']}")
def test_small_ragged(case):
    fwd_bwd_guarded(W.custom(backward=True, **case))


@pytest.mark.parametrize("entry", ["plain", "window", "softcap", "dropout"])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_packed_batch_with_empty_sequences(entry, d):
    w = W.custom(B=0, Hq=4, Hkv=2, N=0, d=d, dtype="bf16", causal=entry != "window",
                 seed=610 + d, lens=[0, 1, 70, 0, 200, 129], backward=True)
    fwd_bwd_guarded(w, entry)


def test_full_size_training_step():
    w = W.WORKLOADS["train_16k"]
    fwd_bwd_guarded(w)


@pytest.mark.parametrize("case", [dict(Nq=1, Nk=700, lens=[700, 0, 1, 513]),
                                  dict(Nq=5, Nk=300, lens=[3, 300, 129, 64])])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_decode(case, d):
    import torch
    fa = _fa()
    w = W.decode_custom(B=4, Hq=8, Hkv=2, d=d, dtype="bf16", causal=True, seed=620 + d, **case)
    a = W.generate_decode(w)
    q, k, v = (torch.from_numpy(a[n]).to(torch.bfloat16).cuda() for n in ("q", "k", "v"))
    lens = torch.from_numpy(a["cache_seqlens"]).cuda()
    say(f"[guards] decode Nq={w.Nq} Nk={w.Nk} d={d} lens={w.cache_lens()}")
    for splits in (0, 3):
        o = Guarded(q.shape, torch.bfloat16)
        lse = Guarded((w.Hq, w.B * w.Nq), torch.float32)
        nws = fa.fa_fwd_kvcache_workspace_size(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, d, splits)
        ws = Guarded((max(nws, 1),), torch.uint8)
        st = fa.fa_fwd_kvcache(q.data_ptr(), k.data_ptr(), v.data_ptr(), lens.data_ptr(), o.ptr(),
                               lse.ptr(), w.B, w.Hq, w.Hkv, w.Nq, w.Nk, d, float(w.scale), 1,
                               splits, fa.FA_BF16, ws.ptr(), nws, _stream())
        assert st == fa.FA_OK, fa.fa_status_string(st)
        torch.cuda.synchronize()
        for g, n in ((o, "O"), (lse, "LSE"), (ws, "workspace")):
            g.check(f"{n} (splits={splits})")
