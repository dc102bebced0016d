"""Property-based check of the host-side cu_seqlens validator (no GPU needed).

Hypothesis draws packed-batch descriptions, valid and invalid, and
fa_check_cu_seqlens must accept exactly those that satisfy its documented
condition: entry 0 is 0 and every sequence length lies in [0, N]. The rule
is restated here as a plain predicate, so a wrong comparison, an off-by-one
in the loop bound or a missed first entry in the C code shows up as a
counterexample. Derandomized: every run draws the same cases.
"""
import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st


def _fa():
    import exact_io_aware_12_amd as fa
    return fa


def holds(cu, N):
    if cu[0] != 0:
        return False
    return all(0 <= int(cu[s + 1]) - int(cu[s]) <= N for s in range(len(cu) - 1))


@st.composite
def packed(draw):
    N = draw(st.integers(0, 64))
    B = draw(st.integers(0, 8))
    lens = draw(st.lists(st.integers(-3, N + 3), min_size=B, max_size=B))
    first = draw(st.sampled_from([0, 0, 0, 1, -1]))
    cu = np.cumsum([first] + lens).astype(np.int32)
    return cu, B, N


@settings(max_examples=400, deadline=None, derandomize=True, database=None,
          suppress_health_check=list(HealthCheck))
@given(case=packed())
def test_check_cu_seqlens_matches_rule(case):
    fa = _fa()
    cu, B, N = case
    cu = np.ascontiguousarray(cu)
    st_ = fa.fa_check_cu_seqlens(cu.ctypes.data, B, N)
    want = fa.FA_OK if holds(cu, N) else fa.FA_ERR_INVALID_ARG
    assert st_ == want, (cu.tolist(), B, N, st_)


@settings(max_examples=200, deadline=None, derandomize=True, database=None,
          suppress_health_check=list(HealthCheck))
@given(B=st.integers(1, 16), N=st.integers(1, 70000), hkv=st.sampled_from([1, 2, 8]),
       group=st.sampled_from([1, 2, 4]), d=st.sampled_from([64, 128, 256]))
def test_backward_workspace_covers_two_rows_per_token(B, N, hkv, group, d):
    """The backward's workspace holds D and LSE·log2 e (float32) for every
    (query head, token), so it can never be smaller than 8·Hq·B·N bytes."""
    fa = _fa()
    hq = hkv * group
    n = fa.fa_bwd_workspace_size(B, hq, hkv, N, d)
    assert n >= 8 * hq * B * N
