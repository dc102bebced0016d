"""GPU parity of fa_fwd against the float64 oracle (through the C ABI).

Small shapes compare every element (several tiles plus a ragged tail); the
full-size workloads compare sampled rows, which the oracle computes one by
one, in the launch configuration the benchmark times.
"""
import numpy as np
import pytest

import workloads as W
from oracle import attention_fwd, attention_fwd_rows
from parity_util import (bits_equal, check_lse, check_o, host32, host64, map_units, say,
                         tile_rows, to_device)

pytestmark = pytest.mark.gpu


def _fa():
    import exact_io_aware_12_amd as fa   # raises if libfa.so is missing: no fallback
    return fa


def run_fwd(w: W.Workload, arrays=None):
    """Run fa_fwd on the workload's seeded inputs; returns (o [T,Hq,d], lse [Hq,T], inputs)."""
    import torch
    fa = _fa()
    arrays = W.generate(w, with_grad=False) if arrays is None else arrays
    t = to_device(arrays, w.dtype)
    say(f"[fa_fwd] {w.name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} d={w.d} {w.dtype} "
        f"causal={w.causal} varlen={w.varlen} T={w.T}")
    if w.varlen:
        o, lse = fa.flash_attn_func(t["q"], t["k"], t["v"], causal=w.causal, softmax_scale=w.scale,
                                    cu_seqlens=t["cu_seqlens"], max_seqlen=w.N)
    else:
        shp = (w.B, w.N)
        o, lse = fa.flash_attn_func(t["q"].view(*shp, w.Hq, w.d), t["k"].view(*shp, w.Hkv, w.d),
                                    t["v"].view(*shp, w.Hkv, w.d), causal=w.causal,
                                    softmax_scale=w.scale)
        o = o.view(w.T, w.Hq, w.d)
    torch.cuda.synchronize()
    return o, lse, t


def compare_whole(w, arrays=None):
    o, lse, t = run_fwd(w, arrays)
    cu = t["cu_seqlens"].cpu().numpy()
    o_ref, lse_ref = attention_fwd(host64(t["q"]), host64(t["k"]), host64(t["v"]), w.scale,
                                   w.causal, cu)
    e, floor, exc = check_o(host64(o), o_ref, w.dtype)
    el = check_lse(host64(lse), lse_ref)
    say(f"   max|dO|={e:.2e} floor={floor:.2e} exceptions={exc} max|dLSE|={el:.2e}")
    return o, lse


# ---- whole-tensor parity on small shapes -------------------------------------
def test_tiny_workload():
    compare_whole(W.WORKLOADS["tiny"])


def test_causal_d64_workload():
    compare_whole(W.WORKLOADS["causal_d64"])


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 7, 64, 65, 130, 257])
def test_ragged_lengths(dtype, d, causal, N):
    compare_whole(W.custom(B=2, Hq=2, Hkv=2, N=N, d=d, dtype=dtype, causal=causal,
                           seed=100 + N))


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 65, 200])
def test_head_dim_256(dtype, causal, N):
    """d = 256, the top of the pages' envelope (forward and decode only)."""
    compare_whole(W.custom(B=2, Hq=4, Hkv=2, N=N, d=256, dtype=dtype, causal=causal,
                           seed=500 + N))


def test_head_dim_256_varlen():
    compare_whole(W.custom(B=0, Hq=4, Hkv=1, N=0, d=256, dtype="bf16", causal=True, seed=510,
                           lens=[300, 0, 129]))


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_gqa(dtype, causal):
    compare_whole(W.custom(B=1, Hq=8, Hkv=2, N=200, d=128, dtype=dtype, causal=causal, seed=7))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_with_empty_and_short(d, causal):
    w = W.custom(B=0, Hq=4, Hkv=2, N=0, d=d, dtype="bf16", causal=causal, seed=8,
                 lens=[0, 1, 5, 128, 129, 300, 64, 0])
    compare_whole(w)


STRESS = ["peaked", "offset", "monotone_max", "steep_max"]


def stress_arrays(w, kind):
    a = W.generate(w)
    if kind == "peaked":
        a["q"] = a["q"] * 4.0
    elif kind == "offset":
        u = np.random.default_rng(90).standard_normal(w.d).astype(np.float32)
        a["k"] = a["k"] + 8.0 * u
        a["q"] = a["q"] + 0.5 * u     # positive correlation with u: large positive logits
    else:
        # the running max grows every tile; steeply enough in "steep_max" that
        # the row max ends ~127 (in log2 units) above that of the first tile
        top = 30.0 if kind == "monotone_max" else 1000.0
        a["k"][:, :, 0] = np.linspace(0, top, w.T, dtype=np.float32)[:, None]
        a["q"][:, :, 0] = 1.0
    return a


@pytest.mark.parametrize("kind", STRESS)
def test_stress_inputs(kind):
    """Large logits, shifted keys and a running max that grows every tile."""
    w = W.custom(B=1, Hq=2, Hkv=2, N=700, d=128, dtype="fp16", causal=True, seed=9)
    compare_whole(w, stress_arrays(w, kind))


# ---- long ragged sequences (d = 128, N >= 2048: many key tiles, ragged ends) ---
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [2048, 2111, 2367])
def test_long_ragged(dtype, causal, N):
    compare_whole(W.custom(B=1, Hq=2, Hkv=1, N=N, d=128, dtype=dtype, causal=causal,
                           seed=N + (1 if causal else 0)))


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("kind", STRESS)
@pytest.mark.parametrize("causal", [False, True])
def test_long_stress(dtype, kind, causal):
    """Stress inputs over many key tiles; 'steep_max' raises the row maximum in
    every tile, so the lazily raised reference max is rescaled again and again
    (in both fp16 and bf16)."""
    w = W.custom(B=1, Hq=2, Hkv=2, N=2100, d=128, dtype=dtype, causal=causal, seed=19)
    compare_whole(w, stress_arrays(w, kind))


def test_long_gqa_varlen():
    w = W.custom(B=0, Hq=8, Hkv=2, N=0, d=128, dtype="bf16", causal=True, seed=20,
                 lens=[2100, 0, 5, 700, 2048, 1])
    compare_whole(w)


def test_long_deterministic():
    w = W.custom(B=1, Hq=2, Hkv=2, N=2200, d=128, dtype="fp16", causal=False, seed=21)
    a = W.generate(w)
    o1, l1, _ = run_fwd(w, a)
    o2, l2, _ = run_fwd(w, a)
    assert bits_equal(o1, o2) and bits_equal(l1, l2)


# ---- invariants that hold exactly for this kernel ----------------------------
def test_deterministic():
    w = W.custom(B=1, Hq=4, Hkv=4, N=1000, d=128, dtype="bf16", causal=True, seed=10)
    a = W.generate(w)
    o1, l1, _ = run_fwd(w, a)
    o2, l2, _ = run_fwd(w, a)
    assert bits_equal(o1, o2) and bits_equal(l1, l2)


def test_varlen_equals_separate_runs():
    lens = [300, 129, 1, 64]
    w = W.custom(B=0, Hq=4, Hkv=1, N=0, d=128, dtype="fp16", causal=True, seed=11, lens=lens)
    a = W.generate(w)
    o, lse, _ = run_fwd(w, a)
    cu = w.cu_seqlens()
    for s, L in enumerate(lens):
        ws = W.custom(B=1, Hq=4, Hkv=1, N=L, d=128, dtype="fp16", causal=True, seed=11)
        sub = {n: a[n][cu[s]:cu[s + 1]] for n in ("q", "k", "v")}
        sub["cu_seqlens"] = ws.cu_seqlens()
        os_, ls, _ = run_fwd(ws, sub)
        assert bits_equal(o[cu[s]:cu[s + 1]], os_), f"sequence {s}"
        assert bits_equal(lse[:, cu[s]:cu[s + 1]], ls), f"sequence {s}"


def test_gqa_equals_repeated_mha():
    w = W.custom(B=2, Hq=8, Hkv=2, N=333, d=64, dtype="bf16", causal=False, seed=12)
    a = W.generate(w)
    o, lse, _ = run_fwd(w, a)
    wm = W.custom(B=2, Hq=8, Hkv=8, N=333, d=64, dtype="bf16", causal=False, seed=12)
    am = dict(a, k=np.repeat(a["k"], 4, axis=1), v=np.repeat(a["v"], 4, axis=1))
    o2, lse2, _ = run_fwd(wm, am)
    assert bits_equal(o, o2) and bits_equal(lse, lse2)


def test_causal_prefix():
    w = W.custom(B=1, Hq=2, Hkv=2, N=777, d=128, dtype="fp16", causal=True, seed=13)
    a = W.generate(w)
    o, lse, _ = run_fwd(w, a)
    M = 300
    wp = W.custom(B=1, Hq=2, Hkv=2, N=M, d=128, dtype="fp16", causal=True, seed=13)
    ap = {n: a[n][:M] for n in ("q", "k", "v")}
    ap["cu_seqlens"] = wp.cu_seqlens()
    op, lp, _ = run_fwd(wp, ap)
    assert bits_equal(o[:M], op) and bits_equal(lse[:, :M], lp)


def test_constant_values_exact():
    """V constant across keys: every output row equals that row (rounded once)."""
    w = W.custom(B=1, Hq=2, Hkv=2, N=500, d=64, dtype="bf16", causal=True, seed=14)
    a = W.generate(w)
    a["v"][:] = a["v"][:1]
    o, _, t = run_fwd(w, a)
    want = np.broadcast_to(host64(t["v"][:1]), o.shape)
    check_o(host64(o), want, w.dtype, "O with constant V")


# ---- parity at the full workload sizes: every (sequence, head) unit ----------
# The launch configuration (tile order, XCD remapping, heavy-first causal order,
# sequence-fastest indexing) only takes its full form at these sizes, so every
# unit is checked, on rows from its first, one inner and its last query tile.
def compare_every_unit(w, o, lse, t, seed=0):
    import torch
    rng = np.random.default_rng(seed)
    cu = w.cu_seqlens()
    q, k, v = host32(t["q"]), host32(t["k"]), host32(t["v"])
    units = [(s, h) for s in range(len(cu) - 1) for h in range(w.Hq) if cu[s + 1] > cu[s]]
    rows = {u: tile_rows(rng, int(cu[u[0] + 1] - cu[u[0]]), 128) for u in units}
    toks = np.concatenate([cu[s] + np.array(rows[(s, h)]) for s, h in units])
    heads = np.concatenate([np.full(len(rows[u]), u[1]) for u in units])
    ti = torch.as_tensor(toks, device=o.device)
    hi = torch.as_tensor(heads, device=o.device)
    o_g, l_g = host64(o[ti, hi]), host64(lse[hi, ti])
    refs = map_units(lambda u: attention_fwd_rows(q, k, v, w.scale, w.causal, cu, u[0], u[1],
                                                  rows[u]), units)
    o_ref = np.concatenate([r[0] for r in refs])
    l_ref = np.concatenate([r[1] for r in refs])
    e, _, _ = check_o(o_g, o_ref, w.dtype, f"O ({len(units)} units)")
    el = check_lse(l_g, l_ref, f"LSE ({len(units)} units)")
    say(f"   every unit ({len(units)}, {len(toks)} rows): max|dO|={e:.2e} max|dLSE|={el:.2e}")


@pytest.mark.parametrize("N", [512, 1024, 2048, 4096, 8192])
def test_sweep_every_unit(N):
    base = W.WORKLOADS[f"sweep_N{N}_full"]
    a = W.generate(base)
    for causal in (False, True):
        w = W.WORKLOADS[f"sweep_N{N}_{'causal' if causal else 'full'}"]
        o, lse, t = run_fwd(w, a)
        compare_every_unit(w, o, lse, t, seed=N + causal)
        del o, lse, t


def test_gqa_varlen_every_unit():
    w = W.WORKLOADS["gqa_varlen"]
    o, lse, t = run_fwd(w)
    compare_every_unit(w, o, lse, t, seed=4)


def test_train_16k_forward_every_unit():
    w = W.WORKLOADS["train_16k"]
    o, lse, t = run_fwd(w)
    compare_every_unit(w, o, lse, t, seed=5)
