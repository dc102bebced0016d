"""Shared helpers for the GPU parity tests: running the HIP path through the
C ABI on seeded inputs, and the tolerance rules.

Tolerances (written once, here):
  O     max |O_gpu − O_ref| ≤ 2e-3 (fp16) / 1e-2 (bf16), O_ref the unrounded
        float64 oracle. An element whose own rounding floor |rne(O_ref) − O_ref|
        already exceeds the tolerance is judged against tol + ½ ulp(O_ref) and
        counted as an exception (a perfect kernel could not do better).
  LSE   max |LSE_gpu − LSE_ref| ≤ 1e-3.
  grads per tensor max |g − g_ref| / max |g_ref| ≤ 2e-2.
"""
from __future__ import annotations

import sys

import numpy as np

TOL_O = {"fp16": 2e-3, "bf16": 1e-2}
TOL_LSE = 1e-3
TOL_GRAD = 2e-2
_MANT = {"fp16": 10, "bf16": 7}
_EMIN = {"fp16": -14, "bf16": -126}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch_dtype(name):
    import torch
    return {"fp16": torch.float16, "bf16": torch.bfloat16}[name]


def half_ulp(x, dtype):
    ax = np.maximum(np.abs(x), 1e-300)
    e = np.maximum(np.floor(np.log2(ax)), _EMIN[dtype])
    return 2.0 ** (e - _MANT[dtype]) / 2


def rne(x, dtype):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch_dtype(dtype)).double().numpy()


def check_o(o_gpu, o_ref, dtype, what="O"):
    """Assert the O tolerance rule; returns (max_err, floor, n_exceptions)."""
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    err = np.abs(o_gpu - o_ref)
    floor = np.abs(rne(o_ref, dtype) - o_ref)
    tol = TOL_O[dtype]
    allowed = np.where(floor > tol, tol + half_ulp(o_ref, dtype), tol)
    bad = err > allowed
    assert np.isfinite(o_gpu).all(), f"{what}: non-finite values"
    if bad.any():
        idx = np.unravel_index(np.argmax(err - allowed), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} elements over tolerance; worst at {idx}: "
                             f"gpu {o_gpu[idx]!r} ref {o_ref[idx]!r} err {err[idx]:.3e} "
                             f"allowed {allowed[idx]:.3e}")
    return float(err.max(initial=0.0)), float(floor.max(initial=0.0)), int((floor > tol).sum())


def check_lse(lse_gpu, lse_ref, what="LSE"):
    lse_gpu = np.asarray(lse_gpu, dtype=np.float64)
    err = np.abs(lse_gpu - lse_ref)
    assert np.isfinite(lse_gpu).all(), f"{what}: non-finite values"
    m = float(err.max(initial=0.0))
    assert m <= TOL_LSE, f"{what}: max err {m:.3e} > {TOL_LSE}"
    return m


def check_grad(g_gpu, g_ref, what):
    g_gpu = np.asarray(g_gpu, dtype=np.float64)
    assert np.isfinite(g_gpu).all(), f"{what}: non-finite values"
    scale = float(np.abs(g_ref).max(initial=0.0))
    err = float(np.abs(g_gpu - g_ref).max(initial=0.0))
    rel = err / scale if scale > 0 else err
    fro = float(np.linalg.norm(g_gpu - g_ref) / max(np.linalg.norm(g_ref), 1e-300))
    assert rel <= TOL_GRAD, f"{what}: max-abs/max|ref| = {rel:.3e} > {TOL_GRAD} (frob {fro:.2e})"
    return rel, fro


def to_device(arrays, dtype):
    """float32 NumPy arrays -> rounded torch tensors on cuda:0 (inputs only)."""
    import torch
    out = {}
    for n, a in arrays.items():
        if n == "cu_seqlens":
            out[n] = torch.from_numpy(a).to("cuda")
        else:
            out[n] = torch.from_numpy(a).to(torch_dtype(dtype)).to("cuda")
    return out


def bits_equal(a, b) -> bool:
    """Bitwise equality of two tensors of one dtype (distinguishes -0 from +0)."""
    import torch
    if a.shape != b.shape or a.dtype != b.dtype:
        return False
    iv = {2: torch.int16, 4: torch.int32}[a.element_size()]
    return bool((a.contiguous().view(iv) == b.contiguous().view(iv)).all())


def host64(t):
    return t.detach().float().cpu().double().numpy() if t.dtype != np.float64 else t


def host32(t):
    """A device tensor of 16-bit values as a float32 NumPy array (exact)."""
    return t.detach().float().cpu().numpy()


def tile_rows(rng, L, tile, n_random=2):
    """Positions that cover a sequence's first, one inner and last tile of
    `tile` rows: each tile's first two and last positions, plus random rows."""
    if L <= 0:
        return []
    nt = (L + tile - 1) // tile
    inner = int(rng.integers(0, nt))
    rows = set()
    for t0 in (0, inner * tile, (nt - 1) * tile):
        rows.update(r for r in (t0, t0 + 1, min(t0 + tile, L) - 1) if 0 <= r < L)
    rows.update(int(x) for x in rng.integers(0, L, size=n_random))
    return sorted(rows)


def map_units(fn, units, workers=8):
    """fn(unit) for every unit on a thread pool (NumPy releases the GIL in its
    large array operations); returns the results in the units' order."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max(1, min(workers, len(units)))) as ex:
        return list(ex.map(fn, units))
