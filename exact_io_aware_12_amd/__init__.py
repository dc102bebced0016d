"""Python binding of libfa.so: exact fused attention on MI355X (gfx950).

Argument marshalling only. Every step of the computation runs in the HIP
kernels of libfa.so; torch supplies device memory and the current stream.
If the library has not been built, importing the binding raises: there is no
fallback implementation.

Raw entry points with the C names and arguments (pointers as ints):
    fa_fwd, fa_bwd, fa_bwd_stage, fa_bwd_num_stages, fa_bwd_workspace_size,
    fa_fwd_window, fa_bwd_window, fa_bwd_window_stage,
    fa_fwd_softcap, fa_bwd_softcap, fa_bwd_softcap_stage,
    fa_fwd_dropout, fa_bwd_dropout, fa_bwd_dropout_stage, fa_fwd_fp8,
    fa_fwd_kvcache, fa_fwd_kvcache_stage, fa_fwd_kvcache_num_stages,
    fa_kvcache_num_splits, fa_fwd_kvcache_workspace_size,
    fa_status_string
Tensor-level helpers:
    flash_attn_func(q, k, v, causal=False, softmax_scale=None,
                    cu_seqlens=None, max_seqlen=None, dropout_p=0.0,
                    window_size=(-1, -1), softcap=0.0, dropout_seed=None) -> (o, lse)
    flash_attn_backward(dout, q, k, v, o, lse, causal=False, softmax_scale=None,
                        cu_seqlens=None, max_seqlen=None, workspace=None,
                        window_size=(-1, -1), softcap=0.0, dropout_p=0.0,
                        dropout_seed=None) -> (dq, dk, dv)
    flash_attn_func_fp8(q, k, v, descale_q, descale_k, descale_v, ...) -> (o, lse)
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

__all__ = ["FA_OK", "FA_ERR_INVALID_ARG", "FA_ERR_UNSUPPORTED", "FA_ERR_HIP", "FA_ERR_WORKSPACE",
           "FA_FP16", "FA_BF16", "FaError", "lib", "lib_path", "fa_fwd", "fa_bwd",
           "fa_bwd_workspace_size", "fa_status_string", "flash_attn_func",
           "flash_attn_backward", "fa_bwd_stage", "fa_bwd_num_stages", "fa_fwd_kvcache",
           "fa_kvcache_num_splits", "fa_fwd_kvcache_workspace_size", "flash_attn_with_kvcache",
           "fa_fwd_kvcache_stage", "fa_fwd_kvcache_num_stages", "fa_fwd_kvcache_fp8",
           "fa_fwd_kvcache_fp8_stage", "fa_kvcache_fp8_num_splits",
           "fa_fwd_kvlen", "flash_attn_kvlen_func", "fa_fwd_kvcache_local"]

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_HIP, FA_ERR_WORKSPACE = 0, -1, -2, -3, -4
FA_FP16, FA_BF16 = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))


def lib_path() -> str:
    return os.path.join(_HERE, "libfa.so")


class FaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {fa_status_string(status)} ({status})")


def _load():
    path = lib_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python exact_io_aware_12_amd/build.py` "
                          "(there is no non-HIP fallback)")
    # torch bundles its own HIP runtime under the same soname (libamdhip64.so.7).
    # Loading torch first makes libfa.so bind to that runtime, so the tensors torch
    # allocates and the kernels libfa.so launches live in one runtime; loading
    # libfa.so first would pull in a second runtime that cannot see torch's memory.
    import torch  # noqa: F401
    L = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, i, vp]
    L.fa_fwd.restype = i
    L.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, i, vp, sz, vp]
    L.fa_bwd.restype = i
    L.fa_bwd_stage.argtypes = [i] + L.fa_bwd.argtypes
    L.fa_bwd_stage.restype = i
    L.fa_bwd_num_stages.argtypes = []
    L.fa_bwd_num_stages.restype = i
    L.fa_bwd_workspace_size.argtypes = [i, i, i, i, i]
    L.fa_bwd_workspace_size.restype = sz
    L.fa_fwd_window.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp, i, vp]
    L.fa_fwd_window.restype = i
    L.fa_bwd_window.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp, i,
                                vp, sz, vp]
    L.fa_bwd_window.restype = i
    L.fa_bwd_window_stage.argtypes = [i] + L.fa_bwd_window.argtypes
    L.fa_bwd_window_stage.restype = i
    L.fa_fwd_window_softcap.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, f, vp, i, vp]
    L.fa_fwd_window_softcap.restype = i
    L.fa_bwd_window_softcap.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i,
                                        f, vp, i, vp, sz, vp]
    L.fa_bwd_window_softcap.restype = i
    L.fa_bwd_window_softcap_stage.argtypes = [i] + L.fa_bwd_window_softcap.argtypes
    L.fa_bwd_window_softcap_stage.restype = i
    L.fa_fwd_softcap.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, f, vp, i, vp]
    L.fa_fwd_softcap.restype = i
    L.fa_bwd_softcap.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, f, vp, i,
                                 vp, sz, vp]
    L.fa_bwd_softcap.restype = i
    L.fa_bwd_softcap_stage.argtypes = [i] + L.fa_bwd_softcap.argtypes
    L.fa_bwd_softcap_stage.restype = i
    u64 = ctypes.c_uint64
    L.fa_fwd_dropout.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, f, u64, vp, i, vp]
    L.fa_fwd_dropout.restype = i
    L.fa_bwd_dropout.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, f, u64,
                                 vp, i, vp, sz, vp]
    L.fa_bwd_dropout.restype = i
    L.fa_bwd_dropout_stage.argtypes = [i] + L.fa_bwd_dropout.argtypes
    L.fa_bwd_dropout_stage.restype = i
    L.fa_fwd_kvlen.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, vp, i, vp]
    L.fa_fwd_kvlen.restype = i
    L.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, f, f, f, i, vp]
    L.fa_fwd_fp8.restype = i
    L.fa_fwd_kvcache.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, i, vp, sz, vp]
    L.fa_fwd_kvcache.restype = i
    L.fa_fwd_kvcache_stage.argtypes = [i] + L.fa_fwd_kvcache.argtypes
    L.fa_fwd_kvcache_stage.restype = i
    L.fa_fwd_kvcache_local.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, f, i, i,
                                       vp, sz, vp]
    L.fa_fwd_kvcache_local.restype = i
    L.fa_fwd_kvcache_fp8.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, f, f, i, i, vp,
                                     sz, vp]
    L.fa_fwd_kvcache_fp8.restype = i
    L.fa_fwd_kvcache_fp8_stage.argtypes = [i] + L.fa_fwd_kvcache_fp8.argtypes
    L.fa_fwd_kvcache_fp8_stage.restype = i
    L.fa_fwd_kvcache_num_stages.argtypes = []
    L.fa_fwd_kvcache_num_stages.restype = i
    L.fa_kvcache_num_splits.argtypes = [i, i, i, i, i, i]
    L.fa_kvcache_num_splits.restype = i
    L.fa_kvcache_fp8_num_splits.argtypes = [i, i, i, i, i, i]
    L.fa_kvcache_fp8_num_splits.restype = i
    L.fa_fwd_kvcache_workspace_size.argtypes = [i, i, i, i, i, i, i]
    L.fa_fwd_kvcache_workspace_size.restype = sz
    L.fa_status_string.argtypes = [i]
    L.fa_status_string.restype = ctypes.c_char_p
    return L


lib = _load()


# ---- raw C entry points ------------------------------------------------------
def fa_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, causal, cu_seqlens, dtype, stream) -> int:
    return lib.fa_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, causal, cu_seqlens, dtype, stream)


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, N, d, scale, causal, cu_seqlens, dtype,
           workspace, workspace_bytes, stream) -> int:
    return lib.fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, N, d, scale, causal,
                      cu_seqlens, dtype, workspace, workspace_bytes, stream)


def fa_bwd_stage(stage, q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, N, d, scale, causal,
                 cu_seqlens, dtype, workspace, workspace_bytes, stream) -> int:
    return lib.fa_bwd_stage(stage, q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, N, d, scale,
                            causal, cu_seqlens, dtype, workspace, workspace_bytes, stream)


def fa_fwd_window(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, window_left, window_right, cu_seqlens,
                  dtype, stream) -> int:
    return lib.fa_fwd_window(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, window_left, window_right,
                             cu_seqlens, dtype, stream)


def fa_bwd_window(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, N, d, scale, window_left,
                  window_right, cu_seqlens, dtype, workspace, workspace_bytes, stream) -> int:
    return lib.fa_bwd_window(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, N, d, scale,
                             window_left, window_right, cu_seqlens, dtype, workspace,
                             workspace_bytes, stream)


def fa_bwd_window_stage(stage, q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, N, d, scale,
                        window_left, window_right, cu_seqlens, dtype, workspace, workspace_bytes,
                        stream) -> int:
    return lib.fa_bwd_window_stage(stage, q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, N, d,
                                   scale, window_left, window_right, cu_seqlens, dtype, workspace,
                                   workspace_bytes, stream)


def fa_fwd_softcap(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, causal, softcap, cu_seqlens, dtype,
                   stream) -> int:
    return lib.fa_fwd_softcap(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, causal, softcap,
                              cu_seqlens, dtype, stream)


def fa_bwd_softcap(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, N, d, scale, causal, softcap,
                   cu_seqlens, dtype, workspace, workspace_bytes, stream) -> int:
    return lib.fa_bwd_softcap(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, N, d, scale, causal,
                              softcap, cu_seqlens, dtype, workspace, workspace_bytes, stream)


def fa_bwd_softcap_stage(stage, q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, N, d, scale,
                         causal, softcap, cu_seqlens, dtype, workspace, workspace_bytes,
                         stream) -> int:
    return lib.fa_bwd_softcap_stage(stage, q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, N, d,
                                    scale, causal, softcap, cu_seqlens, dtype, workspace,
                                    workspace_bytes, stream)


def fa_fwd_dropout(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, causal, dropout_p, seed, cu_seqlens,
                   dtype, stream) -> int:
    return lib.fa_fwd_dropout(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, causal, dropout_p, seed,
                              cu_seqlens, dtype, stream)


def fa_bwd_dropout(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, N, d, scale, causal, dropout_p,
                   seed, cu_seqlens, dtype, workspace, workspace_bytes, stream) -> int:
    return lib.fa_bwd_dropout(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, N, d, scale, causal,
                              dropout_p, seed, cu_seqlens, dtype, workspace, workspace_bytes,
                              stream)


def fa_bwd_dropout_stage(stage, q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, N, d, scale,
                         causal, dropout_p, seed, cu_seqlens, dtype, workspace, workspace_bytes,
                         stream) -> int:
    return lib.fa_bwd_dropout_stage(stage, q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, N, d,
                                    scale, causal, dropout_p, seed, cu_seqlens, dtype, workspace,
                                    workspace_bytes, stream)


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


def fa_fwd_kvlen(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, cu_seqlens_q,
                 cu_seqlens_k, dtype, stream) -> int:
    return lib.fa_fwd_kvlen(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, cu_seqlens_q,
                            cu_seqlens_k, dtype, stream)


def fa_fwd_fp8(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, causal, cu_seqlens, descale_q,
               descale_k, descale_v, out_dtype, stream) -> int:
    return lib.fa_fwd_fp8(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, causal, cu_seqlens,
                          descale_q, descale_k, descale_v, out_dtype, stream)


def fa_bwd_num_stages() -> int:
    return lib.fa_bwd_num_stages()


def fa_bwd_workspace_size(B, Hq, Hkv, N, d) -> int:
    return lib.fa_bwd_workspace_size(B, Hq, Hkv, N, d)


def fa_fwd_kvcache(q, k_cache, v_cache, cache_seqlens, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal,
                   num_splits, dtype, workspace, workspace_bytes, stream) -> int:
    return lib.fa_fwd_kvcache(q, k_cache, v_cache, cache_seqlens, o, lse, B, Hq, Hkv, Nq, Nk, d,
                              scale, causal, num_splits, dtype, workspace, workspace_bytes, stream)


def fa_fwd_kvcache_stage(stage, q, k_cache, v_cache, cache_seqlens, o, lse, B, Hq, Hkv, Nq, Nk, d,
                         scale, causal, num_splits, dtype, workspace, workspace_bytes,
                         stream) -> int:
    return lib.fa_fwd_kvcache_stage(stage, q, k_cache, v_cache, cache_seqlens, o, lse, B, Hq, Hkv,
                                    Nq, Nk, d, scale, causal, num_splits, dtype, workspace,
                                    workspace_bytes, stream)


def fa_fwd_kvcache_fp8(q, k_cache, v_cache, cache_seqlens, o, lse, B, Hq, Hkv, Nq, Nk, d, scale,
                       causal, descale_k, descale_v, num_splits, dtype, workspace,
                       workspace_bytes, stream) -> int:
    return lib.fa_fwd_kvcache_fp8(q, k_cache, v_cache, cache_seqlens, o, lse, B, Hq, Hkv, Nq, Nk,
                                  d, scale, causal, descale_k, descale_v, num_splits, dtype,
                                  workspace, workspace_bytes, stream)


def fa_fwd_kvcache_local(q, k_cache, v_cache, cache_seqlens, o, lse, B, Hq, Hkv, Nq, Nk, d, scale,
                         causal, window_left, softcap, num_splits, dtype, workspace,
                         workspace_bytes, stream) -> int:
    return lib.fa_fwd_kvcache_local(q, k_cache, v_cache, cache_seqlens, o, lse, B, Hq, Hkv, Nq,
                                    Nk, d, scale, causal, window_left, softcap, num_splits, dtype,
                                    workspace, workspace_bytes, stream)


def fa_fwd_kvcache_fp8_stage(stage, q, k_cache, v_cache, cache_seqlens, o, lse, B, Hq, Hkv, Nq,
                             Nk, d, scale, causal, descale_k, descale_v, num_splits, dtype,
                             workspace, workspace_bytes, stream) -> int:
    return lib.fa_fwd_kvcache_fp8_stage(stage, q, k_cache, v_cache, cache_seqlens, o, lse, B, Hq,
                                        Hkv, Nq, Nk, d, scale, causal, descale_k, descale_v,
                                        num_splits, dtype, workspace, workspace_bytes, stream)


def fa_fwd_kvcache_num_stages() -> int:
    return lib.fa_fwd_kvcache_num_stages()


def fa_kvcache_num_splits(B, Hq, Hkv, Nq, Nk, d) -> int:
    return lib.fa_kvcache_num_splits(B, Hq, Hkv, Nq, Nk, d)


def fa_kvcache_fp8_num_splits(B, Hq, Hkv, Nq, Nk, d) -> int:
    return lib.fa_kvcache_fp8_num_splits(B, Hq, Hkv, Nq, Nk, d)


def fa_fwd_kvcache_workspace_size(B, Hq, Hkv, Nq, Nk, d, num_splits) -> int:
    return lib.fa_fwd_kvcache_workspace_size(B, Hq, Hkv, Nq, Nk, d, num_splits)


def fa_status_string(status: int) -> str:
    return lib.fa_status_string(status).decode()


# ---- tensor helpers ----------------------------------------------------------
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


def _check_dev(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("fa tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("fa tensors must be contiguous")


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
                    dropout_p=0.0, window_size=(-1, -1), softcap=0.0, dropout_seed=None):
    """Forward. Returns (o, lse); lse is float32 [Hq, T] (natural log).

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
        _check_dev(cu_seqlens)
        if cu_seqlens.dtype != torch.int32:
            raise TypeError("cu_seqlens must be int32")
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
                          cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None):
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
        for c in (cu_seqlens_q, cu_seqlens_k):
            _check_dev(c)
            if c.dtype != torch.int32:
                raise TypeError("cu_seqlens must be int32")
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


def flash_attn_func_fp8(q, k, v, descale_q=1.0, descale_k=1.0, descale_v=1.0, causal=False,
                        softmax_scale=None, cu_seqlens=None, max_seqlen=None, out_dtype=None):
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
        _check_dev(cu_seqlens)
        if cu_seqlens.dtype != torch.int32:
            raise TypeError("cu_seqlens must be int32")
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
                        dropout_p=0.0, dropout_seed=None):
    """Backward. Returns (dq, dk, dv) shaped like q, k, v (window_size, softcap,
    dropout_p and dropout_seed as in the forward, which produced o and lse)."""
    import torch
    B, N, T, Hq, Hkv, d = _shape(q, k, cu_seqlens, max_seqlen)
    _check_dev(dout, q, k, v, o, lse)
    if cu_seqlens is not None:
        _check_dev(cu_seqlens)
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
                                workspace.numel(), _stream())
        if st != FA_OK:
            raise FaError(st, "fa_bwd_dropout")
        return dq, dk, dv
    if softcap and w is not None:
        st = lib.fa_bwd_window_softcap(*ptrs, B, Hq, Hkv, N, d, float(scale), w[0], w[1],
                                       float(softcap), cu, _dtype_code(q), workspace.data_ptr(),
                                       workspace.numel(), _stream())
        if st != FA_OK:
            raise FaError(st, "fa_bwd_window_softcap")
        return dq, dk, dv
    if softcap:
        st = lib.fa_bwd_softcap(*ptrs, B, Hq, Hkv, N, d, float(scale), int(bool(causal)),
                                float(softcap), cu, _dtype_code(q), workspace.data_ptr(),
                                workspace.numel(), _stream())
        if st != FA_OK:
            raise FaError(st, "fa_bwd_softcap")
        return dq, dk, dv
    if w is None:
        st = lib.fa_bwd(*ptrs, B, Hq, Hkv, N, d, float(scale), int(bool(causal)), cu,
                        _dtype_code(q), workspace.data_ptr(), workspace.numel(), _stream())
    else:
        st = lib.fa_bwd_window(*ptrs, B, Hq, Hkv, N, d, float(scale), w[0], w[1], cu,
                               _dtype_code(q), workspace.data_ptr(), workspace.numel(),
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
                                      workspace.numel(), _stream())
        if st != FA_OK:
            raise FaError(st, "fa_fwd_kvcache_local")
        return o, lse
    if kv8:
        st = lib.fa_fwd_kvcache_fp8(*ptrs, B, Hq, Hkv, Nq, Nk, d, float(scale), int(bool(causal)),
                                    float(descale_k), float(descale_v), int(num_splits),
                                    _dtype_code(q), workspace.data_ptr(), workspace.numel(),
                                    _stream())
        if st != FA_OK:
            raise FaError(st, "fa_fwd_kvcache_fp8")
        return o, lse
    st = lib.fa_fwd_kvcache(*ptrs, B, Hq, Hkv, Nq, Nk, d, float(scale), int(bool(causal)),
                            int(num_splits), _dtype_code(q), workspace.data_ptr(), workspace.numel(),
                            _stream())
    if st != FA_OK:
        raise FaError(st, "fa_fwd_kvcache")
    return o, lse
