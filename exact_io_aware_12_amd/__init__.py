"""Python binding of libfa.so: exact fused attention on MI355X (gfx950).

Argument marshalling only. Every step of the computation runs in the HIP
kernels of libfa.so; torch supplies device memory and the current stream.
If the library has not been built, importing the binding raises: there is no
fallback implementation.

Raw entry points: every function include/fa.h declares, under its C name
with its C arguments (pointers as ints, None for NULL), returning the status
(or size); fa_status_string returns a str.
Tensor-level helpers:
    flash_attn_func(q, k, v, causal=False, softmax_scale=None,
                    cu_seqlens=None, max_seqlen=None, dropout_p=0.0,
                    window_size=(-1, -1), softcap=0.0, dropout_seed=None) -> (o, lse)
    flash_attn_backward(dout, q, k, v, o, lse, causal=False, softmax_scale=None,
                        cu_seqlens=None, max_seqlen=None, workspace=None,
                        window_size=(-1, -1), softcap=0.0, dropout_p=0.0,
                        dropout_seed=None) -> (dq, dk, dv)
    flash_attn_func_fp8(q, k, v, descale_q, descale_k, descale_v, ...) -> (o, lse)
    flash_attn_kvlen_func(q, k, v, ...) -> (o, lse)   (queries and keys of different lengths)
    flash_attn_kvlen_backward(dout, q, k, v, o, lse, ...) -> (dq, dk, dv)
    flash_attn_with_kvcache(q, k_cache, v_cache, cache_seqlens, causal=False,
                            softmax_scale=None, num_splits=0) -> (o, lse)
The call shape follows flash_attn_func in the pages' examples (Llama-Factory
page, first code sample: q, k, v as (batch, seq, heads, head_dim), causal flag;
FlashAttention-2 全解析, blog.gitcode.com: dropout_p and softmax_scale).
"""
from __future__ import annotations

import ctypes
import math
import os


FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_HIP, FA_ERR_WORKSPACE = 0, -1, -2, -3, -4
FA_FP16, FA_BF16 = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))


def lib_path() -> str:
    """libfa.so, or with FA_DEBUG=1 in the environment libfa_debug.so: the same
    kernels built with FA_DEBUG (cu_seqlens checked on the host before each
    launch, a synchronisation after each launch)."""
    return os.path.join(_HERE, "libfa_debug.so" if os.environ.get("FA_DEBUG") == "1"
                        else "libfa.so")


class FaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {fa_status_string(status)} ({status})")


# C signatures of the exported functions (include/fa.h), for ctypes: pointer
# arguments (device pointers, streams) are void*; fa_dtype and the status are int.
_VP, _I, _F, _SZ, _U64 = (ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t,
                          ctypes.c_uint64)
_FWD_HEAD = [_VP] * 5 + [_I] * 5 + [_F]                 # q k v o lse  B Hq Hkv N d  scale
_BWD_HEAD = [_VP] * 9 + [_I] * 5 + [_F]                 # q k v o dout lse dq dk dv  B..d  scale
_BWD_TAIL = [_VP, _I, _VP, _SZ, _VP]                    # cu_seqlens dtype workspace bytes stream
_KVC_HEAD = [_VP] * 6 + [_I] * 6 + [_F, _I]             # q kc vc lens o lse  B Hq Hkv Nq Nk d  scale causal
_WS_TAIL = [_VP, _SZ, _VP]                              # workspace bytes stream
_SIGS = {
    "fa_fwd": (_I, _FWD_HEAD + [_I, _VP, _I, _VP]),
    "fa_bwd": (_I, _BWD_HEAD + [_I] + _BWD_TAIL),
    "fa_bwd_num_stages": (_I, []),
    "fa_bwd_workspace_size": (_SZ, [_I] * 5),
    "fa_bwd_noalloc": (_I, _BWD_HEAD + [_I, _VP, _I, _VP]),
    "fa_fwd_window": (_I, _FWD_HEAD + [_I, _I, _VP, _I, _VP]),
    "fa_bwd_window": (_I, _BWD_HEAD + [_I, _I] + _BWD_TAIL),
    "fa_fwd_window_softcap": (_I, _FWD_HEAD + [_I, _I, _F, _VP, _I, _VP]),
    "fa_bwd_window_softcap": (_I, _BWD_HEAD + [_I, _I, _F] + _BWD_TAIL),
    "fa_fwd_softcap": (_I, _FWD_HEAD + [_I, _F, _VP, _I, _VP]),
    "fa_bwd_softcap": (_I, _BWD_HEAD + [_I, _F] + _BWD_TAIL),
    "fa_fwd_dropout": (_I, _FWD_HEAD + [_I, _F, _U64, _VP, _I, _VP]),
    "fa_bwd_dropout": (_I, _BWD_HEAD + [_I, _F, _U64] + _BWD_TAIL),
    "fa_fwd_kvlen": (_I, [_VP] * 5 + [_I] * 6 + [_F, _I, _VP, _VP, _I, _VP]),
    "fa_bwd_kvlen": (_I, [_VP] * 9 + [_I] * 6 + [_F, _I, _VP, _VP, _I, _VP, _SZ, _VP]),
    "fa_fwd_fp8": (_I, _FWD_HEAD + [_I, _VP, _F, _F, _F, _I, _VP]),
    "fa_fwd_kvcache": (_I, _KVC_HEAD + [_I, _I] + _WS_TAIL),
    "fa_fwd_kvcache_local": (_I, _KVC_HEAD + [_I, _F, _I, _I] + _WS_TAIL),
    "fa_fwd_kvcache_fp8": (_I, _KVC_HEAD + [_F, _F, _I, _I] + _WS_TAIL),
    "fa_fwd_kvcache_num_stages": (_I, []),
    "fa_kvcache_num_splits": (_I, [_I] * 6),
    "fa_kvcache_fp8_num_splits": (_I, [_I] * 6),
    "fa_fwd_kvcache_workspace_size": (_SZ, [_I] * 7),
    "fa_status_string": (ctypes.c_char_p, [_I]),
    "fa_check_cu_seqlens": (_I, [_VP, _I, _I]),
    "fa_fwd_ex": (_I, _FWD_HEAD + [_VP, _VP, _I, _VP]),      # ... scale  opts cu_seqlens dtype stream
    "fa_bwd_ex": (_I, _BWD_HEAD + [_VP] + _BWD_TAIL),       # ... scale  opts cu_seqlens dtype ws bytes stream
}
# each staged entry point takes a leading stage index, then its parent's arguments
for _n in ("fa_bwd", "fa_bwd_window", "fa_bwd_window_softcap", "fa_bwd_softcap",
           "fa_bwd_dropout", "fa_bwd_kvlen", "fa_fwd_kvcache", "fa_fwd_kvcache_fp8"):
    _SIGS[_n + "_stage"] = (_I, [_I] + _SIGS[_n][1])


FA_MASK_NONE, FA_MASK_CAUSAL, FA_MASK_WINDOW = 0, 1, 2


class FaAttnOptions(ctypes.Structure):
    """fa_attn_options of include/fa.h (the argument of fa_fwd_ex / fa_bwd_ex)."""
    _fields_ = [("struct_size", ctypes.c_size_t), ("mask", ctypes.c_int),
                ("window_left", ctypes.c_int), ("window_right", ctypes.c_int),
                ("softcap", ctypes.c_float), ("dropout_p", ctypes.c_float),
                ("dropout_seed", ctypes.c_uint64)]


def attn_options(mask=FA_MASK_NONE, window=(-1, -1), softcap=0.0, dropout_p=0.0,
                 dropout_seed=0) -> FaAttnOptions:
    """An fa_attn_options with struct_size filled in; pass ctypes.addressof(...)
    (keep the object alive across the call)."""
    return FaAttnOptions(ctypes.sizeof(FaAttnOptions), int(mask), int(window[0]),
                         int(window[1]), float(softcap), float(dropout_p), int(dropout_seed))


def _load():
    path = lib_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python exact_io_aware_12_amd/build.py --all` "
                          "(there is no non-HIP fallback)")
    # torch bundles its own HIP runtime under the same soname (libamdhip64.so.7).
    # Loading torch first makes libfa.so bind to that runtime, so the tensors torch
    # allocates and the kernels libfa.so launches live in one runtime; loading
    # libfa.so first would pull in a second runtime that cannot see torch's memory.
    import torch  # noqa: F401
    L = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(L, name)
        fn.restype, fn.argtypes = res, args
    return L


lib = _load()

# ---- raw C entry points: the library's functions themselves, C names and
# argument order (pointers as ints or None), returning the status or size
for _n in _SIGS:
    if _n != "fa_status_string":
        globals()[_n] = getattr(lib, _n)


def fa_status_string(status: int) -> str:
    return lib.fa_status_string(status).decode()


__all__ = (["FA_OK", "FA_ERR_INVALID_ARG", "FA_ERR_UNSUPPORTED", "FA_ERR_HIP", "FA_ERR_WORKSPACE",
            "FA_FP16", "FA_BF16", "FA_MASK_NONE", "FA_MASK_CAUSAL", "FA_MASK_WINDOW",
            "FaAttnOptions", "attn_options", "FaError", "lib", "lib_path", "flash_attn_func",
            "flash_attn_backward", "flash_attn_func_fp8", "flash_attn_kvlen_func",
            "flash_attn_kvlen_backward", "flash_attn_with_kvcache"] + sorted(_SIGS))

# ---- tensor helpers ----------------------------------------------------------
def _dropout_args(dropout_p, dropout_seed, causal_window, softcap):
    """(p, seed) for the dropout entry points, or None when dropout_p is 0."""
    if not dropout_p:
        return None
    if dropout_seed is None:
        raise ValueError("dropout needs dropout_seed (the backward regenerates the same decisions)")
    if causal_window is not None or softcap:
        raise NotImplementedError("dropout with a sliding window or a soft cap is not implemented")
    seed = int(dropout_seed)
    if not 0 <= seed < 2 ** 64:
        raise ValueError("dropout_seed must be a 64-bit unsigned integer")
    return float(dropout_p), seed


def _dtype_code(t):
    import torch
    if t.dtype == torch.float16:
        return FA_FP16
    if t.dtype == torch.bfloat16:
        return FA_BF16
    raise TypeError(f"fa supports float16 and bfloat16 tensors, got {t.dtype}")


def _shape(q, k, cu_seqlens, max_seqlen):
    """(B, N, T, Hq, Hkv, d) from (B, N, H, d) tensors or packed [T, H, d] + cu_seqlens."""
    if cu_seqlens is None:
        if q.dim() != 4 or k.dim() != 4:
            raise ValueError("fixed-length inputs are (batch, seq, heads, head_dim)")
        B, N, Hq, d = q.shape
        if k.shape[0] != B or k.shape[1] != N or k.shape[3] != d:
            raise ValueError(f"q {tuple(q.shape)} and k {tuple(k.shape)} do not match")
        return B, N, B * N, Hq, k.shape[2], d
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("varlen inputs are packed (total_tokens, heads, head_dim)")
    if max_seqlen is None:
        raise ValueError("varlen needs max_seqlen (the longest sequence)")
    T, Hq, d = q.shape
    if k.shape[0] != T or k.shape[2] != d:
        raise ValueError(f"q {tuple(q.shape)} and k {tuple(k.shape)} do not match")
    return cu_seqlens.numel() - 1, int(max_seqlen), T, Hq, k.shape[1], d


def _check_cu(cu_seqlens, T, max_seqlen, validate=True, what="cu_seqlens"):
    """A packed batch's prefix sums: int32 on the GPU, and (unless validate is
    False, or the stream is being captured into a graph) consistent with the
    packed tensors: cu[0] = 0, non-decreasing, cu[-1] = T and no sequence
    longer than max_seqlen. The kernels index the LSE with stride cu[-1] and
    size their grid by max_seqlen, so a mismatch would misplace rows or leave
    them unwritten. The check reads the B+1 entries back (one small copy)."""
    import torch
    _check_dev(cu_seqlens)
    if cu_seqlens.dtype != torch.int32:
        raise TypeError(f"{what} must be int32")
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError(f"{what} must be a 1-d tensor of B+1 prefix sums")
    if not validate or torch.cuda.is_current_stream_capturing():
        return
    cu = cu_seqlens.cpu().tolist()
    lens = [b - a for a, b in zip(cu[:-1], cu[1:])]
    if cu[0] != 0 or any(n < 0 for n in lens):
        raise ValueError(f"{what} must start at 0 and never decrease")
    if cu[-1] != T:
        raise ValueError(f"{what}[-1] = {cu[-1]} but the packed tensors hold {T} tokens")
    if lens and max(lens) > int(max_seqlen):
        raise ValueError(f"a sequence of {max(lens)} tokens exceeds max_seqlen = {max_seqlen}")


def _check_dev(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("fa tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("fa tensors must be contiguous")


def _nbytes(t):
    return t.numel() * t.element_size()


def _stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


def _window(causal, window_size):
    """(left, right) for the window entry points, or None for the plain mask."""
    wl, wr = (int(x) for x in window_size)
    if wl < -1 or wr < -1:
        raise ValueError(f"window_size bounds must be >= -1, got {window_size}")
    if (wl, wr) == (-1, -1):
        return None
    if causal:
        wr = 0 if wr < 0 else min(wr, 0)
    return wl, wr


def flash_attn_func(q, k, v, causal=False, softmax_scale=None, cu_seqlens=None, max_seqlen=None,
                    dropout_p=0.0, window_size=(-1, -1), softcap=0.0, dropout_seed=None,
                    validate=True):
    """Forward. Returns (o, lse); lse is float32 [Hq, T] (natural log).

    cu_seqlens (int32, B+1 prefix sums) with max_seqlen: a packed batch of
    [T, H, d] tensors; validate=False skips reading cu_seqlens back to check it
    against T and max_seqlen (no host synchronisation).
    window_size = (left, right): query i sees keys i − left .. i + right of its
    sequence (−1: unbounded); with causal the right side is 0.
    softcap = c > 0: logits c·tanh(scale·q·k / c) (with or without a window).
    dropout_p > 0: dropout on the softmax weights, decisions from the Philox
    stream of dropout_seed (required; pass the same pair to the backward)."""
    import torch
    B, N, T, Hq, Hkv, d = _shape(q, k, cu_seqlens, max_seqlen)
    if v.shape != k.shape:
        raise ValueError("k and v must have the same shape")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    _check_dev(q, k, v)
    if cu_seqlens is not None:
        _check_cu(cu_seqlens, T, N, validate)
    scale = softmax_scale if softmax_scale is not None else 1.0 / math.sqrt(d)
    o = torch.empty_like(q)
    lse = torch.empty((Hq, T), dtype=torch.float32, device=q.device)
    cu = cu_seqlens.data_ptr() if cu_seqlens is not None else None
    w = _window(causal, window_size)
    drop = _dropout_args(dropout_p, dropout_seed, w, softcap)
    if drop is not None:
        st = lib.fa_fwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                lse.data_ptr(), B, Hq, Hkv, N, d, float(scale),
                                int(bool(causal)), drop[0], drop[1], cu, _dtype_code(q),
                                _stream())
        if st != FA_OK:
            raise FaError(st, "fa_fwd_dropout")
        return o, lse
    if softcap and w is not None:
        st = lib.fa_fwd_window_softcap(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                       lse.data_ptr(), B, Hq, Hkv, N, d, float(scale), w[0], w[1],
                                       float(softcap), cu, _dtype_code(q), _stream())
        if st != FA_OK:
            raise FaError(st, "fa_fwd_window_softcap")
        return o, lse
    if softcap:
        st = lib.fa_fwd_softcap(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                lse.data_ptr(), B, Hq, Hkv, N, d, float(scale),
                                int(bool(causal)), float(softcap), cu, _dtype_code(q), _stream())
        if st != FA_OK:
            raise FaError(st, "fa_fwd_softcap")
        return o, lse
    if w is None:
        st = lib.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                        B, Hq, Hkv, N, d, float(scale), int(bool(causal)), cu, _dtype_code(q),
                        _stream())
    else:
        st = lib.fa_fwd_window(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                               lse.data_ptr(), B, Hq, Hkv, N, d, float(scale), w[0], w[1], cu,
                               _dtype_code(q), _stream())
    if st != FA_OK:
        raise FaError(st, "fa_fwd" if w is None else "fa_fwd_window")
    return o, lse


def flash_attn_kvlen_func(q, k, v, causal=False, softmax_scale=None, cu_seqlens_q=None,
                          cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None,
                          validate=True):
    """Forward with queries and keys of different lengths (chunked prefill).
    Returns (o, lse); lse is float32 [Hq, Tq].

    Fixed length: q [B, Nq, Hq, d], k, v [B, Nk, Hkv, d]. Varlen: q [Tq, Hq, d] with
    cu_seqlens_q and max_seqlen_q, k, v [Tk, Hkv, d] with cu_seqlens_k and
    max_seqlen_k (int32, B+1 entries each). The queries of a sequence are its last
    positions: with causal, query i sees keys j <= i + Lk - Lq; a query that sees no
    key gets o = 0 and lse = -inf (see fa_fwd_kvlen in include/fa.h)."""
    import torch
    if v.shape != k.shape:
        raise ValueError("k and v must have the same shape")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    if (cu_seqlens_q is None) != (cu_seqlens_k is None):
        raise ValueError("give both cu_seqlens_q and cu_seqlens_k, or neither")
    if cu_seqlens_q is None:
        if q.dim() != 4 or k.dim() != 4:
            raise ValueError("fixed-length inputs are (batch, seq, heads, head_dim)")
        B, Nq, Hq, d = q.shape
        if k.shape[0] != B or k.shape[3] != d:
            raise ValueError(f"q {tuple(q.shape)} and k {tuple(k.shape)} do not match")
        Nk, Hkv, Tq = k.shape[1], k.shape[2], B * Nq
    else:
        if q.dim() != 3 or k.dim() != 3:
            raise ValueError("varlen inputs are packed (total_tokens, heads, head_dim)")
        if max_seqlen_q is None or max_seqlen_k is None:
            raise ValueError("varlen needs max_seqlen_q and max_seqlen_k")
        if cu_seqlens_q.numel() != cu_seqlens_k.numel():
            raise ValueError("cu_seqlens_q and cu_seqlens_k need the same number of entries")
        Tq, Hq, d = q.shape
        if k.shape[2] != d:
            raise ValueError(f"q {tuple(q.shape)} and k {tuple(k.shape)} do not match")
        B, Nq, Nk, Hkv = cu_seqlens_q.numel() - 1, int(max_seqlen_q), int(max_seqlen_k), k.shape[1]
        _check_cu(cu_seqlens_q, Tq, Nq, validate, "cu_seqlens_q")
        _check_cu(cu_seqlens_k, k.shape[0], Nk, validate, "cu_seqlens_k")
    _check_dev(q, k, v)
    scale = softmax_scale if softmax_scale is not None else 1.0 / math.sqrt(d)
    o = torch.empty_like(q)
    lse = torch.empty((Hq, Tq), dtype=torch.float32, device=q.device)
    cq = cu_seqlens_q.data_ptr() if cu_seqlens_q is not None else None
    ck = cu_seqlens_k.data_ptr() if cu_seqlens_k is not None else None
    st = lib.fa_fwd_kvlen(q.data_ptr(), k.data_ptr() or None, v.data_ptr() or None, o.data_ptr(),
                          lse.data_ptr(), B, Hq, Hkv, Nq, Nk, d, float(scale), int(bool(causal)),
                          cq, ck, _dtype_code(q), _stream())
    if st != FA_OK:
        raise FaError(st, "fa_fwd_kvlen")
    return o, lse


def flash_attn_kvlen_backward(dout, q, k, v, o, lse, causal=False, softmax_scale=None,
                              cu_seqlens_q=None, cu_seqlens_k=None, max_seqlen_q=None,
                              max_seqlen_k=None, workspace=None, validate=True):
    """Backward of flash_attn_kvlen_func (same layouts and arguments; o, lse its
    outputs). Returns (dq, dk, dv) shaped like q, k, v (see fa_bwd_kvlen)."""
    import torch
    if v.shape != k.shape:
        raise ValueError("k and v must have the same shape")
    if not (q.dtype == k.dtype == v.dtype == o.dtype == dout.dtype):
        raise TypeError("q, k, v, o and dout must share one dtype")
    if o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("o and dout must have q's shape")
    if (cu_seqlens_q is None) != (cu_seqlens_k is None):
        raise ValueError("give both cu_seqlens_q and cu_seqlens_k, or neither")
    if cu_seqlens_q is None:
        if q.dim() != 4 or k.dim() != 4:
            raise ValueError("fixed-length inputs are (batch, seq, heads, head_dim)")
        B, Nq, Hq, d = q.shape
        if k.shape[0] != B or k.shape[3] != d:
            raise ValueError(f"q {tuple(q.shape)} and k {tuple(k.shape)} do not match")
        Nk, Hkv, Tq = k.shape[1], k.shape[2], B * Nq
    else:
        if q.dim() != 3 or k.dim() != 3:
            raise ValueError("varlen inputs are packed (total_tokens, heads, head_dim)")
        if max_seqlen_q is None or max_seqlen_k is None:
            raise ValueError("varlen needs max_seqlen_q and max_seqlen_k")
        if cu_seqlens_q.numel() != cu_seqlens_k.numel():
            raise ValueError("cu_seqlens_q and cu_seqlens_k need the same number of entries")
        Tq, Hq, d = q.shape
        if k.shape[2] != d:
            raise ValueError(f"q {tuple(q.shape)} and k {tuple(k.shape)} do not match")
        B, Nq, Nk, Hkv = cu_seqlens_q.numel() - 1, int(max_seqlen_q), int(max_seqlen_k), k.shape[1]
    if lse.dtype != torch.float32 or tuple(lse.shape) != (Hq, Tq):
        raise ValueError(f"lse must be float32 of shape ({Hq}, {Tq})")
    _check_dev(dout, q, k, v, o, lse)
    if cu_seqlens_q is not None:
        _check_cu(cu_seqlens_q, Tq, Nq, validate, "cu_seqlens_q")
        _check_cu(cu_seqlens_k, k.shape[0], Nk, validate, "cu_seqlens_k")
    scale = softmax_scale if softmax_scale is not None else 1.0 / math.sqrt(d)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    need = fa_bwd_workspace_size(B, Hq, Hkv, Nq, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    else:
        _check_dev(workspace)
    cq = cu_seqlens_q.data_ptr() if cu_seqlens_q is not None else None
    ck = cu_seqlens_k.data_ptr() if cu_seqlens_k is not None else None
    ptr = lambda t: t.data_ptr() if t.numel() else None   # noqa: E731  (empty side: NULL)
    st = lib.fa_bwd_kvlen(ptr(q), ptr(k), ptr(v), ptr(o), ptr(dout), ptr(lse), ptr(dq), ptr(dk),
                          ptr(dv), B, Hq, Hkv, Nq, Nk, d, float(scale), int(bool(causal)), cq, ck,
                          _dtype_code(q), workspace.data_ptr(), _nbytes(workspace), _stream())
    if st != FA_OK:
        raise FaError(st, "fa_bwd_kvlen")
    return dq, dk, dv


def flash_attn_func_fp8(q, k, v, descale_q=1.0, descale_k=1.0, descale_v=1.0, causal=False,
                        softmax_scale=None, cu_seqlens=None, max_seqlen=None, out_dtype=None,
                        validate=True):
    """FP8 forward: q, k, v are e4m3fn codes (torch.float8_e4m3fn or uint8 tensors)
    with per-tensor descales (real value = code value × descale). Returns (o, lse):
    o in out_dtype (bfloat16 by default, or float16), lse float32 [Hq, T]."""
    import torch
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    B, N, T, Hq, Hkv, d = _shape(q, k, cu_seqlens, max_seqlen)
    if v.shape != k.shape:
        raise ValueError("k and v must have the same shape")
    for t in (q, k, v):
        if t.dtype not in (torch.float8_e4m3fn, torch.uint8):
            raise TypeError(f"fp8 inputs must be float8_e4m3fn or uint8 codes, got {t.dtype}")
    _check_dev(q, k, v)
    if cu_seqlens is not None:
        _check_cu(cu_seqlens, T, N, validate)
    scale = softmax_scale if softmax_scale is not None else 1.0 / math.sqrt(d)
    o = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    lse = torch.empty((Hq, T), dtype=torch.float32, device=q.device)
    cu = cu_seqlens.data_ptr() if cu_seqlens is not None else None
    st = lib.fa_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                        B, Hq, Hkv, N, d, float(scale), int(bool(causal)), cu, float(descale_q),
                        float(descale_k), float(descale_v), _dtype_code(o), _stream())
    if st != FA_OK:
        raise FaError(st, "fa_fwd_fp8")
    return o, lse


def flash_attn_backward(dout, q, k, v, o, lse, causal=False, softmax_scale=None, cu_seqlens=None,
                        max_seqlen=None, workspace=None, window_size=(-1, -1), softcap=0.0,
                        dropout_p=0.0, dropout_seed=None, validate=True):
    """Backward. Returns (dq, dk, dv) shaped like q, k, v (window_size, softcap,
    dropout_p, dropout_seed, cu_seqlens and validate as in the forward, which
    produced o and lse). workspace: optional device buffer of at least
    fa_bwd_workspace_size(B, Hq, Hkv, N, d) bytes."""
    import torch
    B, N, T, Hq, Hkv, d = _shape(q, k, cu_seqlens, max_seqlen)
    if v.shape != k.shape:
        raise ValueError("k and v must have the same shape")
    if not (q.dtype == k.dtype == v.dtype == o.dtype == dout.dtype):
        raise TypeError("q, k, v, o and dout must share one dtype")
    if o.shape != q.shape or dout.shape != q.shape:
        raise ValueError(f"o {tuple(o.shape)} and dout {tuple(dout.shape)} must have q's shape "
                         f"{tuple(q.shape)}")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (Hq, T):
        raise ValueError(f"lse must be float32 of shape ({Hq}, {T}), got {lse.dtype} "
                         f"{tuple(lse.shape)}")
    _check_dev(dout, q, k, v, o, lse)
    if cu_seqlens is not None:
        _check_cu(cu_seqlens, T, N, validate)
    if workspace is not None:
        _check_dev(workspace)
    scale = softmax_scale if softmax_scale is not None else 1.0 / math.sqrt(d)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    need = fa_bwd_workspace_size(B, Hq, Hkv, N, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    cu = cu_seqlens.data_ptr() if cu_seqlens is not None else None
    w = _window(causal, window_size)
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
            lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr())
    drop = _dropout_args(dropout_p, dropout_seed, w, softcap)
    if drop is not None:
        st = lib.fa_bwd_dropout(*ptrs, B, Hq, Hkv, N, d, float(scale), int(bool(causal)),
                                drop[0], drop[1], cu, _dtype_code(q), workspace.data_ptr(),
                                _nbytes(workspace), _stream())
        if st != FA_OK:
            raise FaError(st, "fa_bwd_dropout")
        return dq, dk, dv
    if softcap and w is not None:
        st = lib.fa_bwd_window_softcap(*ptrs, B, Hq, Hkv, N, d, float(scale), w[0], w[1],
                                       float(softcap), cu, _dtype_code(q), workspace.data_ptr(),
                                       _nbytes(workspace), _stream())
        if st != FA_OK:
            raise FaError(st, "fa_bwd_window_softcap")
        return dq, dk, dv
    if softcap:
        st = lib.fa_bwd_softcap(*ptrs, B, Hq, Hkv, N, d, float(scale), int(bool(causal)),
                                float(softcap), cu, _dtype_code(q), workspace.data_ptr(),
                                _nbytes(workspace), _stream())
        if st != FA_OK:
            raise FaError(st, "fa_bwd_softcap")
        return dq, dk, dv
    if w is None:
        st = lib.fa_bwd(*ptrs, B, Hq, Hkv, N, d, float(scale), int(bool(causal)), cu,
                        _dtype_code(q), workspace.data_ptr(), _nbytes(workspace), _stream())
    else:
        st = lib.fa_bwd_window(*ptrs, B, Hq, Hkv, N, d, float(scale), w[0], w[1], cu,
                               _dtype_code(q), workspace.data_ptr(), _nbytes(workspace),
                               _stream())
    if st != FA_OK:
        raise FaError(st, "fa_bwd" if w is None else "fa_bwd_window")
    return dq, dk, dv


def flash_attn_with_kvcache(q, k_cache, v_cache, cache_seqlens, causal=False, softmax_scale=None,
                            num_splits=0, workspace=None, descale_k=1.0, descale_v=1.0,
                            window_left=-1, softcap=0.0):
    """Decode over a key/value cache. Returns (o, lse); lse is float32 [Hq, B·Nq].

    q [B, Nq, Hq, d]; k_cache, v_cache [B, Nk, Hkv, d]; cache_seqlens int32 [B]
    (valid positions per entry). The queries are the newest Nq positions of
    each sequence (see fa_fwd_kvcache in include/fa.h). Caches of dtype
    float8_e4m3fn (or uint8 codes) take the FP8 path, fa_fwd_kvcache_fp8, with
    cached value = code × descale_k (K) or × descale_v (V); o has q's dtype.
    window_left >= 0 (keys at most that far behind each query) or softcap > 0
    take fa_fwd_kvcache_local (16-bit caches).
    """
    import torch
    if q.dim() != 4 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("q is (B, Nq, Hq, d); k_cache and v_cache are (B, Nk, Hkv, d)")
    B, Nq, Hq, d = q.shape
    if k_cache.shape[0] != B or k_cache.shape[3] != d:
        raise ValueError(f"q {tuple(q.shape)} and k_cache {tuple(k_cache.shape)} do not match")
    Nk, Hkv = k_cache.shape[1], k_cache.shape[2]
    fp8 = (torch.float8_e4m3fn, torch.uint8)
    kv8 = k_cache.dtype in fp8
    if kv8:
        if v_cache.dtype not in fp8:
            raise TypeError("an fp8 k_cache needs an fp8 v_cache")
        _dtype_code(q)
    elif not (q.dtype == k_cache.dtype == v_cache.dtype):
        raise TypeError("q, k_cache, v_cache must share one dtype")
    _check_dev(q, k_cache, v_cache, cache_seqlens)
    if cache_seqlens.dtype != torch.int32 or cache_seqlens.numel() != B:
        raise TypeError("cache_seqlens must be int32 with one entry per batch entry")
    scale = softmax_scale if softmax_scale is not None else 1.0 / math.sqrt(d)
    o = torch.empty_like(q)
    lse = torch.empty((Hq, B * Nq), dtype=torch.float32, device=q.device)
    need = fa_fwd_kvcache_workspace_size(B, Hq, Hkv, Nq, Nk, d, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ptrs = (q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), cache_seqlens.data_ptr(),
            o.data_ptr(), lse.data_ptr())
    if window_left != -1 or softcap:
        if kv8:
            raise NotImplementedError("a window or soft cap over an fp8 cache is not implemented")
        st = lib.fa_fwd_kvcache_local(*ptrs, B, Hq, Hkv, Nq, Nk, d, float(scale),
                                      int(bool(causal)), int(window_left), float(softcap),
                                      int(num_splits), _dtype_code(q), workspace.data_ptr(),
                                      _nbytes(workspace), _stream())
        if st != FA_OK:
            raise FaError(st, "fa_fwd_kvcache_local")
        return o, lse
    if kv8:
        st = lib.fa_fwd_kvcache_fp8(*ptrs, B, Hq, Hkv, Nq, Nk, d, float(scale), int(bool(causal)),
                                    float(descale_k), float(descale_v), int(num_splits),
                                    _dtype_code(q), workspace.data_ptr(), _nbytes(workspace),
                                    _stream())
        if st != FA_OK:
            raise FaError(st, "fa_fwd_kvcache_fp8")
        return o, lse
    st = lib.fa_fwd_kvcache(*ptrs, B, Hq, Hkv, Nq, Nk, d, float(scale), int(bool(causal)),
                            int(num_splits), _dtype_code(q), workspace.data_ptr(), _nbytes(workspace),
                            _stream())
    if st != FA_OK:
        raise FaError(st, "fa_fwd_kvcache")
    return o, lse
