"""Pins for the oracle's attention, stripe attention and LSE merge (CPU only).

Each check pins the float64 oracle to something other than itself: a
pure-Python brute force on tiny inputs, torch's scaled_dot_product_attention
and logsumexp on the same special case (a different library routine), closed
forms (q = 0, one dominant key), the pages' two-token counterexample, and the
merge identity / monoid laws the pages derive.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import layout as L

SCALE = 1.0 / math.sqrt(192.0)
D = 576
V = 512
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_case(rng, S, H, q_len, kv_std=0.5):
    q = rng.standard_normal((q_len, H, D))
    kv = rng.standard_normal((S, D)) * kv_std
    return q, kv


# ---- brute force ------------------------------------------------------------

def brute_attention(q_row, kv, kv_pos, q_pos, scale):
    """Definition evaluated term by term with math.fsum."""
    vis = [i for i in range(len(kv)) if kv_pos[i] <= q_pos]
    if not vis:
        return [0.0] * V, -math.inf
    s = [scale * math.fsum(float(q_row[d]) * float(kv[i][d]) for d in range(D)) for i in vis]
    m = max(s)
    e = [math.exp(x - m) for x in s]
    Z = math.fsum(e)
    o = [math.fsum(e[j] * float(kv[vis[j]][c]) for j in range(len(vis))) / Z for c in range(V)]
    return o, m + math.log(Z)


@pytest.mark.parametrize("S,q_len", [(1, 1), (5, 1), (16, 1), (9, 3), (4, 4)])
def test_full_attention_against_brute_force(S, q_len):
    rng = np.random.default_rng(S * 10 + q_len)
    H = 2
    q, kv = rand_case(rng, S, H, q_len, kv_std=1.0)
    o, lse = A.full_attention(q, kv, S, SCALE)
    for t in range(q_len):
        for h in range(H):
            bo, bl = brute_attention(q[t, h], kv, list(range(S)), S - q_len + t, SCALE)
            assert np.allclose(o[t, h], bo, rtol=1e-12, atol=1e-13)
            assert abs(lse[t, h] - bl) <= 1e-12 * max(1.0, abs(bl))


@pytest.mark.parametrize("N,I", [(1, 1), (2, 1), (3, 1), (4, 1), (8, 1), (2, 2), (3, 4), (4, 2)])
def test_stripe_attention_against_brute_force(N, I):
    rng = np.random.default_rng(100 + N * 7 + I)
    S, H, q_len = 13, 2, 2
    q, kv = rand_case(rng, S, H, q_len, kv_std=1.0)
    lists = L.stripe_positions(S, N, I)
    for r in range(N):
        o, lse = A.stripe_attention(q, kv, S, lists[r], SCALE)
        for t in range(q_len):
            for h in range(H):
                pos = lists[r].tolist()
                bo, bl = brute_attention(q[t, h], [kv[p] for p in pos], pos, S - q_len + t, SCALE)
                assert np.allclose(o[t, h], bo, rtol=1e-12, atol=1e-13)
                if math.isinf(bl):
                    assert lse[t, h] == -math.inf
                else:
                    assert abs(lse[t, h] - bl) <= 1e-12 * max(1.0, abs(bl))


# ---- library routine on a special case -----------------------------------------

@pytest.mark.parametrize("S,H,q_len", [(37, 4, 1), (200, 16, 1), (64, 3, 4), (5, 8, 4)])
def test_against_torch_sdpa_fp64(S, H, q_len):
    rng = np.random.default_rng(S + H + q_len)
    q, kv = rand_case(rng, S, H, q_len)
    o, lse = A.full_attention(q, kv, S, SCALE)
    qt = torch.from_numpy(q.reshape(q_len * H, D)).view(1, 1, q_len * H, D)
    kt = torch.from_numpy(kv).view(1, 1, S, D)
    vt = torch.from_numpy(np.ascontiguousarray(kv[:, :V])).view(1, 1, S, V)
    qpos = torch.arange(S - q_len, S).repeat_interleave(H)
    mask = torch.arange(S)[None, :] <= qpos[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask.view(1, 1, -1, S), scale=SCALE)
    scores = (qt[0, 0] @ kt[0, 0].T) * SCALE
    ref_lse = torch.logsumexp(scores.masked_fill(~mask, -math.inf), dim=-1)
    assert np.allclose(o.reshape(q_len * H, V), ref[0, 0].numpy(), rtol=1e-12, atol=1e-13)
    assert np.allclose(lse.reshape(-1), ref_lse.numpy(), rtol=1e-12, atol=1e-13)


# ---- closed forms -----------------------------------------------------------------

@pytest.mark.parametrize("N,I,q_len", [(1, 1, 1), (8, 1, 1), (8, 64, 4), (4, 1, 4), (3, 2, 2)])
def test_zero_query_gives_mean_and_log_count(N, I, q_len):
    rng = np.random.default_rng(3)
    S, H = 300, 2
    _, kv = rand_case(rng, S, H, q_len)
    q = np.zeros((q_len, H, D))
    o, lse = A.full_attention(q, kv, S, SCALE)
    for t in range(q_len):
        vis = S - q_len + t + 1
        assert np.allclose(o[t], kv[:vis, :V].mean(axis=0)[None], rtol=1e-12, atol=1e-14)
        assert np.allclose(lse[t], math.log(vis), rtol=1e-14)
    lists = L.stripe_positions(S, N, I)
    for r in range(N):
        o_r, lse_r = A.stripe_attention(q, kv, S, lists[r], SCALE)
        for t in range(q_len):
            mine = lists[r][lists[r] <= S - q_len + t]
            if len(mine) == 0:
                assert (o_r[t] == 0).all() and (lse_r[t] == -np.inf).all()
            else:
                assert np.allclose(o_r[t], kv[mine, :V].mean(axis=0)[None], rtol=1e-12, atol=1e-14)
                assert np.allclose(lse_r[t], math.log(len(mine)), rtol=1e-14)


def test_one_dominant_key_returns_its_value():
    rng = np.random.default_rng(4)
    S, H = 50, 3
    _, kv = rand_case(rng, S, H, 1)
    q = np.zeros((1, H, D))
    for h, target in enumerate([0, 17, 49]):
        q[0, h] = kv[target] * 400.0          # score of the target dominates by a wide margin
    o, _ = A.full_attention(q, kv, S, SCALE)
    for h, target in enumerate([0, 17, 49]):
        assert np.allclose(o[0, h], kv[target, :V], atol=1e-9)
        # the rope dims take part in the score but never in the value
        assert o.shape[-1] == V


def test_rope_dims_enter_the_score():
    """Keys that differ only in the last 64 dims get different weights."""
    S = 2
    kv = np.zeros((S, D))
    kv[0, 0] = 1.0
    kv[1, 1] = 1.0
    kv[1, 512:] = 0.5
    q = np.zeros((1, 1, D))
    q[0, 0, 512:] = 1.0
    o, lse = A.full_attention(q, kv, S, SCALE)
    s1 = SCALE * 64 * 0.5
    w1 = math.exp(s1) / (1 + math.exp(s1))
    assert abs(o[0, 0, 1] - w1) < 1e-14 and abs(o[0, 0, 0] - (1 - w1)) < 1e-14
    assert abs(lse[0, 0] - math.log(1 + math.exp(s1))) < 1e-14


# ---- the pages' counterexample ------------------------------------------------------

def test_two_token_counterexample():
    g = json.load(open(os.path.join(GOLDEN, "two_token_counterexample.json")))
    v0, v1 = g["values"][1], g["values"][0]      # token 0 carries 0, token 1 carries 1
    for gap in (-4.0, 0.0, 4.0):
        kv = np.zeros((2, D))
        kv[0, 0] = v0
        kv[1, 0] = v1
        # scores: s0 = 0, s1 = gap (via a rope dim that only token 1 has)
        kv[1, 575] = 1.0
        q = np.zeros((1, 1, D))
        q[0, 0, 575] = gap / SCALE
        lists = L.stripe_positions(2, 2, 1)
        parts = [A.stripe_attention(q, kv, 2, lists[r], SCALE) for r in range(2)]
        local = [parts[r][0][0, 0, 0] for r in range(2)]
        assert local == g["local_outputs"][::-1]           # shard 0 holds the 0, shard 1 the 1
        naive = 0.5 * (parts[0][0] + parts[1][0])
        assert naive[0, 0, 0] == g["naive_mean_of_local_outputs"]
        true = 1.0 / (1.0 + math.exp(-gap))
        o, _ = A.lse_merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
        assert abs(o[0, 0, 0] - true) < 1e-14
        full, _ = A.full_attention(q, kv, 2, SCALE)
        assert abs(full[0, 0, 0] - true) < 1e-14


# ---- merge identity and monoid laws ------------------------------------------------

CASES = [
    # (S, H, q_len, N, I): small analogues of the five workloads plus fuzz shapes
    (1024, 16, 1, 4, 1),
    (512, 8, 1, 8, 1),
    (700, 6, 1, 8, 1),
    (3, 4, 1, 8, 1),
    (7, 4, 1, 8, 1),
    (1000, 4, 4, 8, 1),
    (1000, 4, 4, 8, 64),
    (130, 3, 2, 3, 2),
    (200, 1, 1, 2, 1),
]


@pytest.mark.parametrize("S,H,q_len,N,I", CASES)
@pytest.mark.parametrize("base", ["e", "2"])
def test_merged_stripes_equal_full_attention(S, H, q_len, N, I, base):
    rng = np.random.default_rng(S * 31 + N)
    q, kv = rand_case(rng, S, H, q_len)
    o_full, lse_full = A.full_attention(q, kv, S, SCALE)
    lists = L.stripe_positions(S, N, I)
    parts = [A.stripe_attention(q, kv, S, lists[r], SCALE) for r in range(N)]
    o_parts = np.stack([p[0] for p in parts])
    lse_parts = np.stack([A.to_base(p[1], base) for p in parts])
    o, lse = A.lse_merge(o_parts, lse_parts, base)
    assert np.allclose(o, o_full, rtol=1e-12, atol=1e-13)
    assert np.allclose(lse, A.to_base(lse_full, base), rtol=1e-12, atol=1e-13)


def test_one_stripe_is_the_identity():
    rng = np.random.default_rng(9)
    S, H, q_len = 77, 5, 3
    q, kv = rand_case(rng, S, H, q_len)
    o_full, lse_full = A.full_attention(q, kv, S, SCALE)
    o1, lse1 = A.stripe_attention(q, kv, S, L.stripe_positions(S, 1, 1)[0], SCALE)
    assert (o1 == o_full).all() and (lse1 == lse_full).all()
    o, lse = A.lse_merge(o1[None], lse1[None])
    assert np.allclose(o, o1, rtol=1e-15, atol=0) and np.allclose(lse, lse1, rtol=1e-15, atol=0)


def _merge_tree(rng, o_parts, lse_parts, base):
    items = [(o_parts[i], lse_parts[i]) for i in range(len(o_parts))]
    while len(items) > 1:
        i, j = sorted(rng.choice(len(items), size=2, replace=False))
        a, b = items[i], items[j]
        m = A.lse_merge(np.stack([a[0], b[0]]), np.stack([a[1], b[1]]), base)
        items = [it for k, it in enumerate(items) if k not in (i, j)] + [m]
    return items[0]


@pytest.mark.parametrize("base", ["e", "2"])
def test_merge_is_order_and_tree_independent(base):
    rng = np.random.default_rng(11)
    N, R = 8, 20
    o_parts = rng.standard_normal((N, R, 16))
    lse_parts = rng.standard_normal((N, R)) * 30
    lse_parts[2, :5] = -np.inf                            # some empty stripes
    ref_o, ref_l = A.lse_merge(o_parts, lse_parts, base)
    for perm in itertools.islice(itertools.permutations(range(N)), 0, 40000, 997):
        o, l = A.lse_merge(o_parts[list(perm)], lse_parts[list(perm)], base)
        assert np.allclose(o, ref_o, rtol=1e-12, atol=1e-13) and np.allclose(l, ref_l, rtol=1e-13)
    for _ in range(20):
        o, l = _merge_tree(rng, o_parts, lse_parts, base)
        assert np.allclose(o, ref_o, rtol=1e-12, atol=1e-13) and np.allclose(l, ref_l, rtol=1e-13)


def test_merge_base_pairing():
    rng = np.random.default_rng(12)
    o_parts = rng.standard_normal((5, 7, 8))
    lse_e = rng.standard_normal((5, 7)) * 10
    oe, le = A.lse_merge(o_parts, lse_e, "e")
    o2, l2 = A.lse_merge(o_parts, lse_e / math.log(2), "2")
    assert np.allclose(oe, o2, rtol=1e-13) and np.allclose(le, l2 * math.log(2), rtol=1e-13)
    # mixing the bases (2^x weights on natural-log lse) gives wrong weights
    o_bad, _ = A.lse_merge(o_parts, lse_e, "2")
    assert not np.allclose(o_bad, oe, rtol=1e-3)


def test_merge_empty_stripes_carry_zero_weight():
    o_parts = np.array([[[1.0, 2.0]], [[np.nan, np.nan]] , [[5.0, 7.0]]])
    o_parts[1] = 123.0                                    # junk in an empty stripe
    lse_parts = np.array([[0.5], [-np.inf], [0.5]])
    o, lse = A.lse_merge(o_parts, lse_parts)
    assert np.allclose(o, [[3.0, 4.5]]) and np.allclose(lse, [0.5 + math.log(2)])
    o, lse = A.lse_merge(o_parts[1:2], lse_parts[1:2])
    assert (o == 0).all() and (lse == -np.inf).all()


def test_large_lse_does_not_overflow():
    o_parts = np.array([[[1.0]], [[3.0]]])
    lse_parts = np.array([[1000.0], [1000.0 + math.log(3)]])
    o, lse = A.lse_merge(o_parts, lse_parts)
    assert np.allclose(o, [[2.5]]) and np.allclose(lse, [1000.0 + math.log(4)])


def test_chunked_evaluation_is_the_same_sum():
    rng = np.random.default_rng(13)
    S, H, q_len = 1000, 4, 4
    q, kv = rand_case(rng, S, H, q_len)
    o1, l1 = A.full_attention(q, kv, S, SCALE)
    o2, l2 = A.full_attention(q, kv, S, SCALE, chunk=97)
    assert np.allclose(o1, o2, rtol=1e-12, atol=1e-14) and np.allclose(l1, l2, rtol=1e-14)


# ---- mergeable variants: sliding window, logit softcap, attention sink ------
# (page "DCP", "conditions for merging and where they fail")

def brute_variant(q_row, kv, kv_pos, q_pos, scale, window=0, softcap=0.0, sink=None, slope=0.0):
    """The variant definitions evaluated term by term with math.fsum."""
    vis = [i for i in range(len(kv))
           if kv_pos[i] <= q_pos and (window <= 0 or kv_pos[i] > q_pos - window)]
    s = []
    for i in vis:
        x = scale * math.fsum(float(q_row[d]) * float(kv[i][d]) for d in range(D))
        x = softcap * math.tanh(x / softcap) if softcap > 0 else x
        s.append(x + slope * (kv_pos[i] - q_pos))
    terms = s + ([sink] if sink is not None else [])
    if not terms:
        return [0.0] * V, -math.inf
    m = max(terms)
    e = [math.exp(x - m) for x in s]
    Z = math.fsum(e + ([math.exp(sink - m)] if sink is not None else []))
    o = [math.fsum(e[j] * float(kv[vis[j]][c]) for j in range(len(vis))) / Z for c in range(V)]
    return o, m + math.log(Z)


VARIANTS = [dict(window=3), dict(window=1), dict(softcap=0.5), dict(sinks=[0.7, -1.3]),
            dict(window=4, softcap=1.0, sinks=[2.0, 0.1]), dict(slopes=[0.25, 0.0625]),
            dict(slopes=[0.5, 1.0], softcap=2.0, sinks=[0.0, 1.0])]


def _close(o, lse, bo, bl):
    assert np.allclose(o, bo, rtol=1e-12, atol=1e-13)
    if math.isinf(bl):
        assert lse == -math.inf
    else:
        assert abs(lse - bl) <= 1e-12 * max(1.0, abs(bl))


@pytest.mark.parametrize("var", VARIANTS)
def test_variants_against_brute_force(var):
    rng = np.random.default_rng(7)
    S, H, q_len = 11, 2, 2
    q, kv = rand_case(rng, S, H, q_len, kv_std=1.0)
    o, lse = A.full_attention(q, kv, S, SCALE, **var)
    sinks = var.get("sinks")
    slopes = var.get("slopes", [0.0] * H)
    for t in range(q_len):
        for h in range(H):
            bo, bl = brute_variant(q[t, h], kv, list(range(S)), S - q_len + t, SCALE, var.get("window", 0),
                                   var.get("softcap", 0.0), None if sinks is None else sinks[h], slopes[h])
            _close(o[t, h], lse[t, h], bo, bl)
    # one stripe of a block round-robin layout, the sink on this stripe
    pos = L.stripe_positions(S, 3, 2)[1]
    o, lse = A.stripe_attention(q, kv, S, pos, SCALE, **var)
    for t in range(q_len):
        for h in range(H):
            bo, bl = brute_variant(q[t, h], [kv[p] for p in pos.tolist()], pos.tolist(), S - q_len + t, SCALE,
                                   var.get("window", 0), var.get("softcap", 0.0),
                                   None if sinks is None else sinks[h], slopes[h])
            _close(o[t, h], lse[t, h], bo, bl)


def test_window_of_one_sees_only_the_query_position():
    rng = np.random.default_rng(8)
    S, H, q_len = 9, 3, 3
    q, kv = rand_case(rng, S, H, q_len)
    o, lse = A.full_attention(q, kv, S, SCALE, window=1)
    for t in range(q_len):
        p = S - q_len + t
        for h in range(H):
            assert np.allclose(o[t, h], kv[p, :V], rtol=0, atol=1e-15)
            assert abs(lse[t, h] - SCALE * float(q[t, h] @ kv[p])) < 1e-12


def test_window_covering_the_context_changes_nothing():
    rng = np.random.default_rng(9)
    S, H, q_len = 20, 2, 4
    q, kv = rand_case(rng, S, H, q_len)
    o0, l0 = A.full_attention(q, kv, S, SCALE)
    o1, l1 = A.full_attention(q, kv, S, SCALE, window=S)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
    # W = S - q_len + 1: query t sees p >= t, so the first query keeps every
    # position and the last one loses positions 0 .. q_len - 2
    o2, l2 = A.full_attention(q, kv, S, SCALE, window=S - q_len + 1)
    assert np.array_equal(o2[0], o0[0]) and np.array_equal(l2[0], l0[0])
    assert not np.allclose(o2[-1], o0[-1], rtol=1e-6, atol=0)
    o3, l3 = A.full_attention(q[-1:], kv[q_len - 1:], S - q_len + 1, SCALE)   # the last query on what it keeps
    assert np.allclose(o2[-1], o3[0], rtol=1e-12, atol=1e-14) and np.allclose(l2[-1], l3[0], rtol=1e-12)


def test_softcap_saturates_to_a_two_level_softmax():
    # q along dim 0 only, huge: every capped score is +c or -c to fp64 rounding,
    # so the weights are e^c for keys with kv[.,0] > 0 and e^-c for the others
    rng = np.random.default_rng(10)
    S, c = 12, 1.5
    kv = rng.standard_normal((S, D)) * 0.5
    sign = np.where(rng.random(S) < 0.4, 1.0, -1.0)
    kv[:, 0] = sign
    q = np.zeros((1, 1, D))
    q[0, 0, 0] = 1e6
    o, lse = A.full_attention(q, kv, S, SCALE, softcap=c)
    wp, wm = math.exp(c), math.exp(-c)
    Z = wp * (sign > 0).sum() + wm * (sign < 0).sum()
    want = (wp * kv[sign > 0, :V].sum(axis=0) + wm * kv[sign < 0, :V].sum(axis=0)) / Z
    assert np.allclose(o[0, 0], want, rtol=1e-12, atol=1e-14)
    assert abs(lse[0, 0] - math.log(Z)) < 1e-12


def test_softcap_far_above_the_scores_is_the_plain_softmax():
    rng = np.random.default_rng(11)
    S, H, q_len = 15, 2, 2
    q, kv = rand_case(rng, S, H, q_len)
    o0, l0 = A.full_attention(q, kv, S, SCALE)
    o1, l1 = A.full_attention(q, kv, S, SCALE, softcap=1e7)
    assert np.allclose(o0, o1, rtol=1e-11, atol=1e-13) and np.allclose(l0, l1, rtol=1e-11, atol=1e-12)


def test_sink_with_zero_query_closed_form():
    # every score is 0: o = n / (n + e^sigma) * mean(v), lse = log(n + e^sigma)
    rng = np.random.default_rng(12)
    S, H, q_len = 10, 2, 3
    kv = rng.standard_normal((S, D))
    q = np.zeros((q_len, H, D))
    sinks = np.array([0.3, -2.0])
    o, lse = A.full_attention(q, kv, S, SCALE, sinks=sinks)
    for t in range(q_len):
        n = S - q_len + t + 1
        for h in range(H):
            f = n / (n + math.exp(sinks[h]))
            assert np.allclose(o[t, h], f * kv[:n, :V].mean(axis=0), rtol=1e-12, atol=1e-14)
            assert abs(lse[t, h] - math.log(n + math.exp(sinks[h]))) < 1e-12


def test_sink_alone_and_minus_infinite_sink():
    rng = np.random.default_rng(13)
    S, H = 6, 2
    q, kv = rand_case(rng, S, H, 1)
    o0, l0 = A.full_attention(q, kv, S, SCALE)
    o1, l1 = A.full_attention(q, kv, S, SCALE, sinks=[-np.inf, -np.inf])
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
    # a stripe with no visible row but the sink: o = 0, lse = sigma
    o2, l2 = A.stripe_attention(q, kv, S, np.array([], dtype=np.int64), SCALE, sinks=[1.5, -0.5])
    assert np.array_equal(o2, np.zeros_like(o2)) and np.allclose(l2[0], [1.5, -0.5], rtol=0, atol=0)


@pytest.mark.parametrize("var", VARIANTS)
@pytest.mark.parametrize("N,I", [(2, 1), (3, 2), (4, 1), (8, 1)])
def test_variant_stripes_merge_to_full(var, N, I):
    # the page's claim: with the sink added in exactly one shard, the merge of
    # the stripes is the unsharded variant
    rng = np.random.default_rng(N * 13 + I)
    S, H, q_len = 37, 2, 3
    q, kv = rand_case(rng, S, H, q_len)
    o_full, l_full = A.full_attention(q, kv, S, SCALE, **var)
    lists = L.stripe_positions(S, N, I)
    parts = []
    for r in range(N):
        v = dict(var)
        if r != N - 1:
            v.pop("sinks", None)
        parts.append(A.stripe_attention(q, kv, S, lists[r], SCALE, **v))
    o, lse = A.lse_merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    assert np.allclose(o, o_full, rtol=1e-12, atol=1e-14)
    assert np.allclose(lse, l_full, rtol=1e-12, atol=1e-12)


def test_sink_added_on_every_stripe_is_counted_every_time():
    # the merge adds up the partition functions: a sink on all N stripes
    # enters N times, Z = Z_plain + N e^sigma
    rng = np.random.default_rng(14)
    S, H, N = 24, 2, 4
    q, kv = rand_case(rng, S, H, 1)
    sinks = np.array([0.4, 1.1])
    _, l_plain = A.full_attention(q, kv, S, SCALE)
    lists = L.stripe_positions(S, N, 1)
    parts = [A.stripe_attention(q, kv, S, lists[r], SCALE, sinks=sinks) for r in range(N)]
    _, lse = A.lse_merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    want = np.log(np.exp(l_plain[0]) + N * np.exp(sinks))
    assert np.allclose(lse[0], want, rtol=1e-12, atol=1e-12)


# ---- head-return exchange (packed bf16 output + fp32 lse) --------------------

def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(21)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 20000),
                        np.array([0.0, -0.0, np.inf, -np.inf, 1e-40, -1e-40, 3.4e38, 1.0 + 2 ** -8,
                                  1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, 65504.0], dtype=np.float32)]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(A.to_bf16_bits(x), want)
    assert np.isnan(A.bf16_bits_to_float(A.to_bf16_bits(np.array([np.nan], dtype=np.float32)))).all()


def test_pack_layout_and_round_trip():
    rng = np.random.default_rng(22)
    rows, H, N, v = 5, 12, 4, 8
    o = rng.standard_normal((rows, H, v)).astype(np.float32)
    lse = (rng.standard_normal((rows, H)) * 30).astype(np.float32)
    lse[0, 3] = -np.inf
    buf = A.pack_heads(o, lse, N)
    assert buf.shape == (N, rows, H // N, v + 4)
    for h in range(H):
        d, j = divmod(h, H // N)
        assert np.array_equal(A.bf16_bits_to_float(buf[d, :, j, :v]), A.bf16_bits_to_float(A.to_bf16_bits(o[:, h])))
        bits = buf[d, :, j, v].astype(np.uint32) | (buf[d, :, j, v + 1].astype(np.uint32) << 16)
        assert np.array_equal(bits.view(np.float32), lse[:, h])            # the lse travels exactly
        assert (buf[d, :, j, v + 2:] == 0).all()
    # the page's payload at B = 64, H = 96, v = 512: 64 x 96 x (512 + 4) x 2 bytes
    assert A.pack_heads(np.zeros((64, 96, 512)), np.zeros((64, 96)), 8).nbytes == 64 * 96 * (512 + 4) * 2


def test_head_return_merge_equals_full_attention_within_bf16():
    # stripes -> per-rank packing -> all-to-all -> each owner merges its heads:
    # every head of the full result, up to the bf16 rounding of the partials
    rng = np.random.default_rng(23)
    S, H, q_len, N = 53, 8, 2, 4
    q, kv = rand_case(rng, S, H, q_len)
    o_full, l_full = A.full_attention(q, kv, S, SCALE)
    lists = L.stripe_positions(S, N, 1)
    sends = []
    for r in range(N):
        o_r, l_r = A.stripe_attention(q, kv, S, lists[r], SCALE)
        sends.append(A.pack_heads(o_r.reshape(q_len, H, V), l_r.reshape(q_len, H), N))
    Hl = H // N
    for d in range(N):
        recv = np.stack([sends[r][d] for r in range(N)])                   # what rank d receives
        o, lse = A.unpack_merge(recv)
        heads = slice(d * Hl, (d + 1) * Hl)
        ref = o_full[:, heads]
        # a convex combination of parts, each within half a bf16 ulp (2^-8 relative) of its value
        bound = 2.0 ** -8 * np.max(np.abs(np.stack([A.stripe_attention(q, kv, S, lists[r], SCALE)[0][:, heads]
                                                    for r in range(N)])), axis=0) + 1e-12
        assert (np.abs(o - ref) <= bound).all()
        assert np.allclose(lse, l_full[:, heads], rtol=0, atol=1e-5)     # lse exact up to float32


def test_position_bias_with_zero_query_is_geometric():
    # every score is 0: position p of a query at t has weight exp(-lam (t - p)),
    # a geometric series over p = 0..t
    rng = np.random.default_rng(15)
    S, H, q_len = 12, 2, 2
    kv = rng.standard_normal((S, D))
    q = np.zeros((q_len, H, D))
    lam = np.array([0.3, 1.7])
    o, lse = A.full_attention(q, kv, S, SCALE, slopes=lam)
    for t in range(q_len):
        pq = S - q_len + t
        for h in range(H):
            r = math.exp(-lam[h])
            w = np.array([r ** (pq - p) for p in range(pq + 1)])
            assert np.allclose(o[t, h], (w[:, None] * kv[:pq + 1, :V]).sum(axis=0) / w.sum(), rtol=1e-12, atol=1e-14)
            assert abs(lse[t, h] - math.log((1 - r ** (pq + 1)) / (1 - r))) < 1e-12


def test_position_bias_uses_global_positions_on_a_stripe():
    # on a stripe the bias of a row is its GLOBAL distance: with q = 0 and
    # token round robin, rank r's weights are exp(-lam (t - p)) over its own p
    rng = np.random.default_rng(16)
    S, N, lam = 20, 4, 0.4
    kv = rng.standard_normal((S, D))
    q = np.zeros((1, 1, D))
    for r, pos in enumerate(L.stripe_positions(S, N, 1)):
        o, lse = A.stripe_attention(q, kv, S, pos, SCALE, slopes=[lam])
        w = np.exp(-lam * (S - 1 - pos))
        assert np.allclose(o[0, 0], (w[:, None] * kv[pos, :V]).sum(axis=0) / w.sum(), rtol=1e-12, atol=1e-14)
        assert abs(lse[0, 0] - math.log(w.sum())) < 1e-12


# ---- sparse attention over a global top-k selection ---------------------------

def _random_topk(rng, S, q_len, K):
    out = np.full((q_len, K), -1, dtype=np.int64)
    for t in range(q_len):
        qp = S - q_len + t
        n = min(K, qp + 1)
        out[t, :n] = rng.choice(qp + 1, size=n, replace=False)
    return out


def test_sparse_selecting_everything_is_full_attention():
    rng = np.random.default_rng(31)
    S, H, q_len = 30, 2, 3
    q, kv = rand_case(rng, S, H, q_len)
    topk = np.stack([np.concatenate([rng.permutation(S - q_len + t + 1), np.full(q_len - 1 - t, -1)])
                     for t in range(q_len)])
    o, lse = A.sparse_attention(q, kv, S, topk, SCALE)
    of, lf = A.full_attention(q, kv, S, SCALE)
    assert np.allclose(o, of, rtol=1e-12, atol=1e-14) and np.allclose(lse, lf, rtol=1e-12, atol=1e-12)


def test_sparse_against_brute_force_and_single_selection():
    rng = np.random.default_rng(32)
    S, H, q_len, K = 17, 2, 2, 5
    q, kv = rand_case(rng, S, H, q_len, kv_std=1.0)
    topk = _random_topk(rng, S, q_len, K)
    topk[1, 0] = S + 3                                          # a position past the query: never seen
    o, lse = A.sparse_attention(q, kv, S, topk, SCALE)
    for t in range(q_len):
        sel = [int(p) for p in topk[t] if 0 <= p <= S - q_len + t]
        for h in range(H):
            bo, bl = brute_attention(q[t, h], [kv[p] for p in sel], sel, S - q_len + t, SCALE)
            _close(o[t, h], lse[t, h], bo, bl)
    one = np.array([[4], [-1]])
    o1, l1 = A.sparse_attention(q, kv, S, one, SCALE)
    assert np.allclose(o1[0], kv[4, :V][None], rtol=0, atol=1e-15) and np.isneginf(l1[1]).all()


@pytest.mark.parametrize("N,I", [(2, 1), (4, 1), (8, 1), (3, 4)])
def test_sparse_stripes_merge_to_the_global_selection(N, I):
    # the page's condition: select globally, each rank attends to the selected
    # tokens it owns, the LSE merge gives the unsharded sparse result
    rng = np.random.default_rng(33 + N)
    S, H, q_len, K = 64, 2, 4, 12
    q, kv = rand_case(rng, S, H, q_len)
    topk = _random_topk(rng, S, q_len, K)
    o_full, l_full = A.sparse_attention(q, kv, S, topk, SCALE)
    parts = [A.sparse_attention(q, kv, S, topk, SCALE, positions=pos) for pos in L.stripe_positions(S, N, I)]
    o, lse = A.lse_merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    assert np.allclose(o, o_full, rtol=1e-12, atol=1e-14) and np.allclose(lse, l_full, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("S,N,k", [(300, 1, 4), (999, 3, 5), (2048, 8, 4), (77, 4, 16)])
def test_bf16_chunk_partials_merge_within_half_an_ulp(S, N, k):
    # a stripe's rows cut into k contiguous chunks (as the kernel cuts them),
    # each chunk's (o, lse) with o rounded to bf16 and lse to float32, merged:
    # a convex combination of the rounded parts, so within 2^-8 of the largest
    # |o| of a part (half a bf16 ulp, relative) of the stripe's exact o; the
    # lse is exact up to float32
    rng = np.random.default_rng(S + 7 * N + k)
    H, q_len = 4, 2
    q, kv = rand_case(rng, S, H, q_len)
    for r in range(N):
        pos = L.stripe_positions(S, N, 1)[r]
        o_ref, l_ref = A.stripe_attention(q, kv, S, pos, SCALE)
        cs = -(-len(pos) // k)
        parts = [A.stripe_attention(q, kv, S, pos[c * cs:(c + 1) * cs], SCALE) for c in range(k)]
        o_p = np.stack([p[0] for p in parts])
        l_p = np.stack([p[1] for p in parts])
        o, lse = A.merge_bf16_parts(o_p, l_p)
        bound = 2.0 ** -8 * np.abs(o_p).max(axis=0) + 1e-12
        assert (np.abs(o - o_ref) <= bound).all()
        assert np.allclose(lse, l_ref, rtol=0, atol=1e-5)
        # without the rounding the same merge is the stripe itself
        o_x, l_x = A.lse_merge(o_p, l_p)
        assert np.allclose(o_x, o_ref, rtol=1e-12, atol=1e-13) and np.allclose(l_x, l_ref, rtol=1e-12, atol=1e-12)


def test_bf16_single_part_is_its_rounding():
    # one part (and an empty part: o = 0, lse = -inf) merge to the part's own bf16 value
    rng = np.random.default_rng(3)
    o = rng.standard_normal((1, 5, V))
    l = rng.standard_normal((1, 5))
    got, lse = A.merge_bf16_parts(np.concatenate([o, np.zeros_like(o)]),
                                  np.concatenate([l, np.full_like(l, -np.inf)]))
    want = A.bf16_bits_to_float(A.to_bf16_bits(o[0].astype(np.float32)))
    assert np.array_equal(got, want)
    assert np.array_equal(lse, l[0].astype(np.float32).astype(np.float64))
