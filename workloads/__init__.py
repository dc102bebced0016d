"""Seeded synthetic inputs for the attention workloads.

This module is shared by the oracle tests, the GPU parity tests and the
benchmark. It only draws random numbers and describes shapes; it holds none
of the attention arithmetic, so neither side of a parity check can borrow a
computation from the other through it.

The workloads are the ones the pages time: random normal fp16/bf16 Q, K, V
tensors in the (batch, seq, heads, head_dim) order of the ``flash_attn_func``
example (Llama-Factory page, first code sample) and the N sweep
{512 … 8192} at batch 4, 32 heads, head_dim 128 of the A/B harness
(mlqm.cn evaluation page, section 三). Two further workloads use the
Llama-3-8B head shape (32 query heads sharing 8 KV heads) over a padding-free
packed batch, and a 16k-token causal training step.

Recipe (one generator per workload, NumPy PCG64):
  1. ``rng = numpy.random.default_rng(seed)``
  2. varlen only: ``lens = rng.integers(1024, 8192, size=8, endpoint=True)``
  3. Q, K, V, then dO, each ``rng.standard_normal(shape, dtype=float32)``
     with shapes [T, Hq, d] / [T, Hkv, d] / [T, Hkv, d] / [T, Hq, d]
  4. the caller rounds to fp16 / bf16 (round to nearest even).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int            # fixed length, or the longest sequence for varlen
    d: int
    dtype: str        # "fp16" | "bf16"
    causal: bool
    seed: int
    varlen: bool = False
    backward: bool = False
    lens: Optional[tuple] = None   # varlen sequence lengths
    window: Optional[tuple] = None  # sliding window (left, right), -1 = unbounded
    softcap: float = 0.0            # soft cap c of the logits (0: none)
    dropout_p: float = 0.0          # dropout on the softmax weights (0: none)
    dropout_seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def seq_lens(self) -> List[int]:
        if self.varlen:
            return list(self.lens)
        return [self.N] * self.B

    @property
    def T(self) -> int:
        return int(sum(self.seq_lens))

    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.seq_lens)]).astype(np.int32)

    def fwd_flop(self) -> float:
        """4·Hq·L²·d per sequence, halved when causal (the metric's convention).

        With a sliding window: 4·Hq·d per visible (query, key) pair, counted
        exactly (the dense L² has no meaning for a band)."""
        if self.window is None:
            f = sum(4.0 * self.Hq * L * L * self.d for L in self.seq_lens)
            return f / 2 if self.causal else f
        return 4.0 * self.Hq * self.d * sum(self.visible_pairs(L) for L in self.seq_lens)

    def visible_pairs(self, L: int) -> int:
        """Number of (query, key) pairs of a length-L sequence inside the window."""
        wl, wr = self.window
        if self.causal:
            wr = 0 if wr < 0 else min(wr, 0)
        i = np.arange(L, dtype=np.int64)
        lo = np.maximum(0, i - wl) if wl >= 0 else np.zeros_like(i)
        hi = np.minimum(L - 1, i + wr) if wr >= 0 else np.full_like(i, L - 1)
        return int(np.maximum(hi - lo + 1, 0).sum())

    def bwd_flop(self) -> float:
        return 2.5 * self.fwd_flop()

    def fwd_bytes(self) -> int:
        """Compulsory HBM bytes of the forward: read Q, K, V once, write O and LSE."""
        e = 2
        T = self.T
        return (2 * T * self.Hq * self.d * e          # Q in, O out
                + 2 * T * self.Hkv * self.d * e       # K, V in
                + 4 * T * self.Hq)                    # LSE out

    def bwd_bytes(self) -> int:
        """Read Q, K, V, O, dO, LSE; write dQ, dK, dV (plus the fp32 D row)."""
        e = 2
        T = self.T
        return (4 * T * self.Hq * self.d * e          # Q, O, dO in, dQ out
                + 4 * T * self.Hkv * self.d * e       # K, V in, dK, dV out
                + 4 * T * self.Hq * 2)                # LSE in, D out


def varlen_lengths(seed: int, count: int = 8, lo: int = 1024, hi: int = 8192) -> List[int]:
    rng = np.random.default_rng(seed)
    return [int(x) for x in rng.integers(lo, hi, size=count, endpoint=True)]


def _sweep(N: int, causal: bool) -> Workload:
    return Workload(f"sweep_N{N}_{'causal' if causal else 'full'}", B=4, Hq=32, Hkv=32,
                    N=N, d=128, dtype="fp16", causal=causal, seed=3)


def _build() -> Dict[str, Workload]:
    w = {
        "tiny": Workload("tiny", B=1, Hq=2, Hkv=2, N=128, d=64, dtype="fp16",
                         causal=False, seed=1),
        "causal_d64": Workload("causal_d64", B=1, Hq=16, Hkv=16, N=2048, d=64,
                               dtype="fp16", causal=True, seed=2),
    }
    for N in (512, 1024, 2048, 4096, 8192):
        for c in (False, True):
            s = _sweep(N, c)
            w[s.name] = s
    lens = tuple(varlen_lengths(4))
    w["gqa_varlen"] = Workload("gqa_varlen", B=len(lens), Hq=32, Hkv=8, N=max(lens), d=128,
                               dtype="bf16", causal=True, seed=4, varlen=True, lens=lens)
    w["train_16k"] = Workload("train_16k", B=2, Hq=16, Hkv=16, N=16384, d=128, dtype="bf16",
                              causal=True, seed=5, backward=True)
    # head dim 256 (forward only), the sweep's shape with half the heads
    w["fwd_d256_N4096"] = Workload("fwd_d256_N4096", B=4, Hq=16, Hkv=16, N=4096, d=256,
                                   dtype="bf16", causal=False, seed=8)
    # the training step's shape with a 4096-key sliding window (each query sees
    # itself and the 4095 keys before it): the band mask, forward and backward
    w["window_16k"] = Workload("window_16k", B=2, Hq=16, Hkv=16, N=16384, d=128, dtype="bf16",
                               causal=False, seed=9, backward=True, window=(4095, 0))
    # the training step's shape with soft-capped logits, c = 50 (the attention
    # soft cap published for Gemma-2); FLOP by the same convention (tanh not counted)
    w["softcap_16k"] = Workload("softcap_16k", B=2, Hq=16, Hkv=16, N=16384, d=128,
                                dtype="bf16", causal=True, seed=10, backward=True, softcap=50.0)
    # head dim 256 forward and backward (the pages' envelope ends at 256)
    w["train_d256"] = Workload("train_d256", B=4, Hq=16, Hkv=16, N=4096, d=256, dtype="bf16",
                               causal=True, seed=12, backward=True)
    # head dim 256 with logits capped at 50 and GQA 16/8 (the Gemma-2 attention setting)
    w["softcap_d256"] = Workload("softcap_d256", B=4, Hq=16, Hkv=8, N=4096, d=256,
                                 dtype="bf16", causal=True, seed=14, backward=True, softcap=50.0)
    # the training step's shape with dropout p = 0.1 on the softmax weights
    w["dropout_16k"] = Workload("dropout_16k", B=2, Hq=16, Hkv=16, N=16384, d=128,
                                dtype="bf16", causal=True, seed=11, backward=True,
                                dropout_p=0.1, dropout_seed=0x5EED)
    return w


WORKLOADS: Dict[str, Workload] = _build()


def custom(B, Hq, Hkv, N, d, dtype="fp16", causal=False, seed=0, lens=None,
           backward=False) -> Workload:
    """A workload of any shape (used for small parity cases and edge cases)."""
    if lens is not None:
        lens = tuple(int(x) for x in lens)
        return Workload(f"custom_varlen", B=len(lens), Hq=Hq, Hkv=Hkv,
                        N=max(lens) if lens else 0, d=d, dtype=dtype, causal=causal,
                        seed=seed, varlen=True, lens=lens, backward=backward)
    return Workload("custom", B=B, Hq=Hq, Hkv=Hkv, N=N, d=d, dtype=dtype, causal=causal,
                    seed=seed, backward=backward)


def generate(w: Workload, with_grad: Optional[bool] = None):
    """Draw float32 Q, K, V (and dO) for a workload, in the recipe's order.

    Returns a dict of NumPy float32 arrays with token-major shapes
    q [T, Hq, d], k/v [T, Hkv, d], do [T, Hq, d] and cu_seqlens int32 [B+1].
    A varlen workload whose lengths are drawn (``lens`` from
    :func:`varlen_lengths`) consumes the same generator stream first.
    """
    if with_grad is None:
        with_grad = w.backward
    rng = np.random.default_rng(w.seed)
    if w.varlen and w.name == "gqa_varlen":
        drawn = rng.integers(1024, 8192, size=8, endpoint=True)
        assert tuple(int(x) for x in drawn) == tuple(w.lens)
    T = w.T
    out = {
        "q": rng.standard_normal((T, w.Hq, w.d), dtype=np.float32),
        "k": rng.standard_normal((T, w.Hkv, w.d), dtype=np.float32),
        "v": rng.standard_normal((T, w.Hkv, w.d), dtype=np.float32),
    }
    if with_grad:
        out["do"] = rng.standard_normal((T, w.Hq, w.d), dtype=np.float32)
    out["cu_seqlens"] = w.cu_seqlens()
    return out


def quantize_e4m3(arrays, names=("q", "k", "v"), v_shift: float = 0.0):
    """FP8 inputs: each named float32 array as e4m3fn codes plus one descale.

    Recipe: descale = max|x| / 448 (the largest e4m3fn value), codes = x /
    descale rounded to e4m3fn (nearest even) by torch's float8_e4m3fn cast;
    ``v_shift`` is added to V first (a non-zero mean makes O far from zero).
    Returns {name: uint8 codes of the same shape, "descale_<name>": float}.
    """
    import torch
    out = {}
    for name in names:
        x = arrays[name].astype(np.float32)
        if name == "v" and v_shift:
            x = x + np.float32(v_shift)
        amax = float(np.abs(x).max()) if x.size else 1.0
        ds = amax / 448.0 if amax > 0 else 1.0
        codes = torch.from_numpy(x / np.float32(ds)).to(torch.float8_e4m3fn)
        out[name] = codes.view(torch.uint8).numpy()
        out["descale_" + name] = ds
    if "cu_seqlens" in arrays:
        out["cu_seqlens"] = arrays["cu_seqlens"]
    return out


def to_torch(arrays, dtype: str, device="cpu"):
    """Round float32 arrays to fp16/bf16 (nearest even) as torch tensors."""
    import torch
    td = {"fp16": torch.float16, "bf16": torch.bfloat16}[dtype]
    res = {}
    for name, a in arrays.items():
        if name == "cu_seqlens":
            res[name] = torch.from_numpy(a).to(device)
        else:
            res[name] = torch.from_numpy(a).to(td).to(device)
    return res


# ---------------------------------------------------------------------------
# Decode over a key/value cache: Nq new queries per batch entry against a
# cache of capacity Nk with L_b valid positions per entry.
#
# Recipe (one generator per workload, NumPy PCG64):
#   1. rng = numpy.random.default_rng(seed)
#   2. lengths: the given list, else all Nk ("full"), else
#      rng.integers(lo, Nk, size=B, endpoint=True) for lens="draw:lo"
#   3. q [B, Nq, Hq, d], then k, v [B, Nk, Hkv, d], each
#      rng.standard_normal(shape, dtype=float32); cache slots past L_b hold
#      random values too (they must never be read into the result)
#   4. the caller rounds to fp16 / bf16 (round to nearest even); with
#      kv_cache="e4m3" the caches are instead quantised by quantize_e4m3
#      (names k and v: one descale each, max|x| / 448), see decode_fp8_inputs
@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    dtype: str = "bf16"
    causal: bool = True
    seed: int = 0
    lens: object = "full"        # "full", "draw:<lo>", or a tuple of B lengths
    kv_cache: str = "same"       # cache element: "same" (dtype) or "e4m3" (FP8 codes)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def cache_lens(self) -> List[int]:
        if isinstance(self.lens, (tuple, list)):
            return [int(x) for x in self.lens]
        if self.lens == "full":
            return [self.Nk] * self.B
        lo = int(str(self.lens).split(":")[1])
        return [int(x) for x in np.random.default_rng(self.seed).integers(
            lo, self.Nk, size=self.B, endpoint=True)]

    def kv_elem_bytes(self) -> int:
        return 1 if self.kv_cache == "e4m3" else 2

    def kv_bytes(self) -> int:
        """K and V bytes of the valid cache positions (what one call must read)."""
        return 2 * sum(self.cache_lens()) * self.Hkv * self.d * self.kv_elem_bytes()

    def io_bytes(self) -> int:
        """Compulsory HBM bytes of one call: valid K/V, q and o, lse."""
        qo = 2 * self.B * self.Nq * self.Hq * self.d * 2
        return self.kv_bytes() + qo + 4 * self.Hq * self.B * self.Nq + 4 * self.B

    def flop(self) -> float:
        """4·d FLOP per (query, visible key) pair (the forward convention)."""
        tot = 0
        for L in self.cache_lens():
            for i in range(self.Nq):
                vis = min(L, max(0, L - self.Nq + i + 1)) if self.causal else L
                tot += vis
        return 4.0 * self.d * self.Hq * tot


DECODE_WORKLOADS: Dict[str, DecodeWorkload] = {
    # Llama-3-8B heads decoding one token per sequence over 8k-token caches
    "decode_llama": DecodeWorkload("decode_llama", B=16, Hq=32, Hkv=8, Nq=1, Nk=8192, d=128,
                                   dtype="bf16", causal=True, seed=6),
    # four new tokens per sequence (draft verification), ragged cache lengths
    # decode_llama over an FP8 (e4m3fn) cache: the same inputs quantised, half the cache bytes
    "decode_llama_fp8": DecodeWorkload("decode_llama_fp8", B=16, Hq=32, Hkv=8, Nq=1, Nk=8192,
                                       d=128, dtype="bf16", causal=True, seed=6, kv_cache="e4m3"),
    "decode_multi": DecodeWorkload("decode_multi", B=4, Hq=32, Hkv=8, Nq=4, Nk=4096, d=128,
                                   dtype="bf16", causal=True, seed=7, lens="draw:1024"),
}


# ---------------------------------------------------------------------------
# Forward with queries and keys of different lengths (chunked prefill): Nq new
# tokens per batch entry attend to Nk keys, the new tokens being the last Nq
# positions. Recipe: rng = numpy.random.default_rng(seed); q [B, Nq, Hq, d],
# then k, v [B, Nk, Hkv, d], each rng.standard_normal(shape, dtype=float32);
# the caller rounds to fp16 / bf16 (nearest even).
@dataclasses.dataclass(frozen=True)
class KvlenWorkload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    dtype: str = "bf16"
    causal: bool = True
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def visible_pairs(self) -> int:
        """(query, key) pairs that enter the result, per (entry, query head)."""
        if not self.causal:
            return self.Nq * self.Nk
        off = self.Nk - self.Nq
        return sum(max(0, min(self.Nk, i + off + 1)) for i in range(self.Nq))

    def fwd_flop(self) -> float:
        """4·d FLOP per visible (query, key) pair (the forward convention)."""
        return 4.0 * self.d * self.B * self.Hq * self.visible_pairs()


KVLEN_WORKLOADS: Dict[str, KvlenWorkload] = {
    # a 2048-token chunk of new tokens over an 8192-key context (6144 cached + the
    # chunk), Llama-3-8B heads
    "prefill_chunk": KvlenWorkload("prefill_chunk", B=4, Hq=32, Hkv=8, Nq=2048, Nk=8192, d=128,
                                   dtype="bf16", causal=True, seed=8),
}


def generate_kvlen(w: KvlenWorkload):
    """float32 q [B, Nq, Hq, d] and k, v [B, Nk, Hkv, d]."""
    rng = np.random.default_rng(w.seed)
    return {
        "q": rng.standard_normal((w.B, w.Nq, w.Hq, w.d), dtype=np.float32),
        "k": rng.standard_normal((w.B, w.Nk, w.Hkv, w.d), dtype=np.float32),
        "v": rng.standard_normal((w.B, w.Nk, w.Hkv, w.d), dtype=np.float32),
    }


def decode_custom(B, Hq, Hkv, Nq, Nk, d, dtype="bf16", causal=True, seed=0, lens="full",
                  kv_cache="same"):
    if isinstance(lens, list):
        lens = tuple(lens)
    return DecodeWorkload("decode_custom", B=B, Hq=Hq, Hkv=Hkv, Nq=Nq, Nk=Nk, d=d, dtype=dtype,
                          causal=causal, seed=seed, lens=lens, kv_cache=kv_cache)


def decode_fp8_inputs(w: DecodeWorkload):
    """generate_decode's arrays with k and v replaced by e4m3fn codes (uint8) and
    their descales "descale_k", "descale_v" (quantize_e4m3); q stays float32."""
    a = generate_decode(w)
    qa = quantize_e4m3(a, names=("k", "v"))
    a["k"], a["v"] = qa["k"], qa["v"]
    a["descale_k"], a["descale_v"] = qa["descale_k"], qa["descale_v"]
    return a


def generate_decode(w: DecodeWorkload):
    """float32 q [B, Nq, Hq, d], k/v [B, Nk, Hkv, d] and int32 cache_seqlens [B]."""
    lens = w.cache_lens()
    rng = np.random.default_rng(w.seed)
    if isinstance(w.lens, str) and w.lens.startswith("draw:"):
        rng.integers(int(w.lens.split(":")[1]), w.Nk, size=w.B, endpoint=True)
    return {
        "q": rng.standard_normal((w.B, w.Nq, w.Hq, w.d), dtype=np.float32),
        "k": rng.standard_normal((w.B, w.Nk, w.Hkv, w.d), dtype=np.float32),
        "v": rng.standard_normal((w.B, w.Nk, w.Hkv, w.d), dtype=np.float32),
        "cache_seqlens": np.asarray(lens, dtype=np.int32),
    }
