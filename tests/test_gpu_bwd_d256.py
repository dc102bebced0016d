"""GPU parity of fa_bwd at head dimension 256 against the float64 oracle.

d = 256 runs its own dK/dV kernel (two passes, dV then dK, one wave per SIMD
holding one accumulator set) and the dQ kernel at one workgroup per CU; the
cases span ragged lengths around the 64-query and 128-key tiles, both masks,
fp16 and bf16, varlen with GQA and empty or one-token sequences, and the
forward at d = 256 feeding it as in training.
"""
import pytest

import workloads as W
from parity_util import bits_equal
from test_gpu_bwd import compare_whole, run_fwd_bwd

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 33, 64, 129, 300])
def test_d256_ragged_lengths(dtype, causal, N):
    compare_whole(W.custom(B=2, Hq=2, Hkv=2, N=N, d=256, dtype=dtype, causal=causal,
                           seed=400 + N, backward=True))


@pytest.mark.parametrize("causal", [False, True])
def test_d256_gqa_varlen(causal):
    w = W.custom(B=0, Hq=8, Hkv=2, N=0, d=256, dtype="bf16", causal=causal, seed=421,
                 lens=[0, 1, 77, 128, 200, 64, 513], backward=True)
    compare_whole(w)


def test_d256_long():
    compare_whole(W.custom(B=1, Hq=2, Hkv=1, N=1100, d=256, dtype="fp16", causal=True, seed=422,
                           backward=True))


def test_d256_deterministic():
    w = W.custom(B=1, Hq=4, Hkv=2, N=400, d=256, dtype="bf16", causal=True, seed=423,
                 backward=True)
    a = W.generate(w, with_grad=True)
    g1, _ = run_fwd_bwd(w, a)
    g2, _ = run_fwd_bwd(w, a)
    assert all(bits_equal(x, y) for x, y in zip(g1, g2))
