"""Randomised pins of the oracle (CPU): the layout invariants and the merge
identity over drawn shapes, beside the fixed cases of the other oracle tests."""

import math

import numpy as np
from hypothesis import given, settings, strategies as st

from oracle import attention as A
from oracle import layout as L

SCALE = 1.0 / math.sqrt(192.0)


@settings(max_examples=60, deadline=None)
@given(N=st.integers(1, 9), I=st.sampled_from([1, 2, 3, 4, 16, 64, 128]), x=st.integers(0, 3000),
       a=st.integers(0, 2000), n=st.integers(0, 700))
def test_layout_counts_and_rows(N, I, x, a, n):
    c = L.local_counts(x, N, I)
    assert c.sum() == x and c.min() >= 0
    assert c.max() - c.min() <= I                               # at most one run apart
    share = L.interval_counts(a, n, N, I)
    assert share.sum() == n
    assert (share == L.local_counts(a + n, N, I) - L.local_counts(a, N, I)).all()
    # every owned position's row is its index in the rank's list
    lists = L.stripe_positions(x, N, I)
    for r in range(N):
        assert len(lists[r]) == c[r]
        if len(lists[r]):
            p = int(lists[r][-1])
            assert L.owner_row_walk(p, N, I) == (r, len(lists[r]) - 1)


@settings(max_examples=25, deadline=None)
@given(N=st.integers(1, 8), I=st.sampled_from([1, 2, 5, 32]), S=st.integers(1, 90), q_len=st.integers(1, 4),
       base=st.sampled_from(["e", "2"]), seed=st.integers(0, 2 ** 31 - 1))
def test_stripes_merge_to_full_attention(N, I, S, q_len, base, seed):
    q_len = min(q_len, S)
    rng = np.random.default_rng(seed)
    H, D = 2, 576
    q = rng.standard_normal((q_len, H, D))
    kv = rng.standard_normal((S, D)) * 0.5
    o_full, l_full = A.full_attention(q, kv, S, SCALE)
    parts = [A.stripe_attention(q, kv, S, pos, SCALE) for pos in L.stripe_positions(S, N, I)]
    o, lse = A.lse_merge(np.stack([p[0] for p in parts]), np.stack([A.to_base(p[1], base) for p in parts]), base)
    assert np.allclose(o, o_full, rtol=1e-11, atol=1e-13)
    assert np.allclose(lse, A.to_base(l_full, base), rtol=1e-11, atol=1e-11)
