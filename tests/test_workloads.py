"""The seeded workload generator: reproducibility, shapes and the work model."""
import numpy as np

import workloads as W


def test_varlen_lengths_pinned():
    # seed 4 reproduces these lengths; none is a multiple of 128, so tail tiles are exercised
    w = W.WORKLOADS["gqa_varlen"]
    assert list(w.lens) == [6231, 7784, 7342, 4689, 7766, 8022, 7979, 1603]
    assert w.T == 51416 and w.N == 8022
    assert all(L % 128 for L in w.lens)
    assert list(w.cu_seqlens()[[0, -1]]) == [0, 51416]


def test_generate_is_seeded_and_ordered():
    w = W.custom(B=2, Hq=4, Hkv=2, N=16, d=8, seed=11, backward=True)
    a, b = W.generate(w), W.generate(w)
    for n in ("q", "k", "v", "do"):
        np.testing.assert_array_equal(a[n], b[n])
    rng = np.random.default_rng(11)
    np.testing.assert_array_equal(a["q"], rng.standard_normal((32, 4, 8), dtype=np.float32))
    np.testing.assert_array_equal(a["k"], rng.standard_normal((32, 2, 8), dtype=np.float32))
    assert a["cu_seqlens"].tolist() == [0, 16, 32]


def test_flop_model():
    s = W.WORKLOADS["sweep_N4096_full"]
    assert s.fwd_flop() == 4 * 4 * 32 * 4096 ** 2 * 128
    assert W.WORKLOADS["sweep_N4096_causal"].fwd_flop() == s.fwd_flop() / 2
    t = W.WORKLOADS["train_16k"]
    assert abs(t.fwd_flop() - 2.199e12) / 2.199e12 < 1e-3
    assert t.bwd_flop() == 2.5 * t.fwd_flop()
    g = W.WORKLOADS["gqa_varlen"]
    assert g.fwd_flop() == 4 * 32 * 366204992 * 128 / 2


def test_rounding_is_nearest_even():
    torch = __import__("torch")
    x = np.array([1.0 + 2 ** -11, 1.0 + 3 * 2 ** -11], dtype=np.float32)   # fp16 ties
    t = W.to_torch({"q": x}, "fp16")["q"].float().numpy()
    assert t.tolist() == [1.0, 1.0 + 2 ** -9]
