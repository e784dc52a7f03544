"""Pins for the oracle's token striping, counts and slot mapping (CPU only).

The oracle produces the striping by simulating the round-robin hand-out.  Here
it is checked against (a) the values the pages print for their worked
examples (tests/golden), (b) the closed forms the pages give, written out
below from the pages, and (c) invariants the pages state.
"""

import json
import os

import numpy as np
import pytest

from oracle import layout as L

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---- closed forms from the pages (used only as pins) -----------------------

def token_rr(p, N):
    """Page "DCP", core abstraction, idea one: owner = p mod N, row = p div N."""
    return p % N, p // N


def block_rr(p, N, I):
    """Page "PCP/DCP", section 6: owner = (t div B) mod P,
    local index = (t div (B*P))*B + t mod B (P = DCP size, B = block size)."""
    return (p // I) % N, (p // (I * N)) * I + p % I


def block_rr_local_len(n, r, N, I):
    """Page "PCP/DCP", section 6: local_len(n, r)."""
    return (n // (N * I)) * I + np.clip(n % (N * I) - r * I, 0, I)


def virtual_block(x, N, I, block_size):
    """vLLM-Ascend CP design, section "block table": virtual block of
    block_size*cp_size tokens, local block index, target rank and the offset
    inside the rank's block; the local row is taken as
    (virtual block index) * block_size + that offset."""
    vbs = block_size * N
    vb = x // vbs
    off = x % vbs
    lbi = off // I
    rank = lbi % N
    inner = (lbi // N) * I + off % I
    return rank, vb * block_size + inner


# ---- printed worked examples ------------------------------------------------

def test_token_rr_worked_example():
    g = golden("token_rr_dcp8.json")
    lists = L.stripe_positions(64, g["N"], g["interleave"])
    for r, prefix in g["rank_prefixes"].items():
        assert lists[int(r)][: len(prefix)].tolist() == prefix


def test_block_rr_worked_example():
    g = golden("block_rr_dcp4_b4.json")
    N, I = g["N"], g["interleave"]
    owner, _ = L.owner_and_row_table(24, N, I)
    for lo, hi, r in g["runs"]:
        assert (owner[lo:hi + 1] == r).all()
    for x, counts in g["counts_after"].items():
        assert L.local_counts(int(x), N, I).tolist() == counts


def test_page_expansion_worked_example():
    g = golden("page_expansion.json")
    P = g["page_size"]
    rows = np.arange(P * len(g["pages"]))
    slots = L.page_slot(np.array(g["pages"]), rows, P)
    want = np.concatenate([np.arange(lo, hi + 1) for lo, hi in g["slot_ranges"]])
    assert slots.tolist() == want.tolist()


def test_rank1_extraction_worked_example():
    g = golden("rank1_extraction.json")
    N, r, n, P = g["N"], g["rank"], g["length"], g["page_size"]
    pos = L.stripe_positions(n, N, 1)[r]
    assert pos[: len(g["positions_head"])].tolist() == g["positions_head"]
    assert pos[-1] == g["positions_last"]
    assert len(pos) == g["tokens_received"]
    # The prefill side is unsharded (DCP1): request position t sits at row t.
    src = L.page_slot(np.array(g["source_pages"]), pos, P)
    assert src.tolist() == g["source_slots"]
    for bad in g["not_in_source_slots"]:
        assert bad not in src.tolist()
    # The decode side stores the received rows compactly in page 10.
    _, row, dst = L.slot_map(pos, np.zeros_like(pos), N, 1, P, r, np.array([[g["dest_page"]]]))
    assert row.tolist() == list(range(len(pos)))
    lo, hi = g["dest_slot_range"]
    assert dst.tolist() == list(range(lo, hi + 1))


# ---- closed forms -----------------------------------------------------------

@pytest.mark.parametrize("N", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("I", [1, 2, 4, 16, 64, 128])
def test_simulation_equals_closed_forms(N, I):
    S = 5000
    owner, row = L.owner_and_row_table(S, N, I)
    p = np.arange(S)
    o3, r3 = block_rr(p, N, I)
    assert (owner == o3).all() and (row == r3).all()
    if I == 1:
        o1, r1 = token_rr(p, N)
        assert (owner == o1).all() and (row == r1).all()
    for block_size in (I, 2 * I, 64 if 64 % I == 0 else I):
        o4, r4 = virtual_block(p, N, I, block_size)
        assert (owner == o4).all() and (row == r4).all()


@pytest.mark.parametrize("N,I", [(1, 1), (3, 1), (8, 1), (4, 4), (8, 64), (3, 16), (8, 128)])
def test_local_counts_equal_local_len(N, I):
    for x in list(range(0, 300)) + [1000, 1333, 4097, 65535]:
        got = L.local_counts(x, N, I)
        want = np.array([block_rr_local_len(x, r, N, I) for r in range(N)])
        assert (got == want).all(), (x, got, want)


def test_owner_row_walk_matches_simulation_and_large_positions():
    for N, I in [(1, 1), (8, 1), (8, 64), (3, 4)]:
        owner, row = L.owner_and_row_table(4096, N, I)
        for p in range(0, 4096, 7):
            assert L.owner_row_walk(p, N, I) == (owner[p], row[p])
    rng = np.random.default_rng(5)
    for p in rng.integers(0, 1 << 40, size=200):
        for N, I in [(8, 1), (8, 64), (5, 2)]:
            assert L.owner_row_walk(int(p), N, I) == tuple(int(v) for v in block_rr(int(p), N, I))


# ---- invariants the pages state ---------------------------------------------

@pytest.mark.parametrize("N,I", [(1, 1), (2, 1), (8, 1), (4, 4), (8, 64), (3, 2)])
def test_count_invariants(N, I):
    for x in range(0, 700, 3):
        c = L.local_counts(x, N, I)
        assert c.sum() == x
        # token RR: counts differ by at most one; block RR: by at most one block
        assert c.max() - c.min() <= (1 if I == 1 else I)
    for a, n in [(0, 0), (0, 17), (1000, 333), (5, 1), (513, 64)]:
        assert L.interval_counts(a, n, N, I).sum() == n


@pytest.mark.parametrize("N,I", [(1, 1), (8, 1), (8, 64), (3, 2), (4, 128)])
def test_owner_row_is_a_bijection_with_compact_rows(N, I):
    S = 2000
    owner, row = L.owner_and_row_table(S, N, I)
    seen = set()
    for p in range(S):
        key = (int(owner[p]), int(row[p]))
        assert key not in seen
        seen.add(key)
    counts = L.local_counts(S, N, I)
    for r in range(N):
        assert sorted(row[owner == r].tolist()) == list(range(counts[r]))
        # rows of one rank follow position order
        assert (np.diff(row[owner == r]) == 1).all()


def test_chunk_interval_counts():
    """count(a+L) - count(a) with global positions, a=1000, L=333, N=8: the
    counts come from the block-RR local_len of page "PCP/DCP" section 6."""
    for I, want in [(1, [42, 42, 42, 42, 42, 41, 41, 41]), (64, [64, 64, 64, 64, 53, 0, 0, 24])]:
        closed = [block_rr_local_len(1333, r, 8, I) - block_rr_local_len(1000, r, 8, I) for r in range(8)]
        assert closed == want
        assert L.interval_counts(1000, 333, 8, I).tolist() == want


# ---- slot map and KV write ------------------------------------------------------

def test_slot_map_against_closed_forms():
    rng = np.random.default_rng(1)
    for N, I, P in [(4, 1, 16), (8, 1, 64), (8, 64, 64), (3, 2, 4)]:
        B = 3
        cols = 40
        tables = rng.permutation(B * cols).reshape(B, cols).astype(np.int32)
        pos = rng.integers(0, 1500, size=400)
        req = rng.integers(0, B, size=400)
        for rank in [-1] + list(range(N)):
            owner, row, slot = L.slot_map(pos, req, N, I, P, rank, tables)
            for i in range(len(pos)):
                o, rr = block_rr(int(pos[i]), N, I)
                assert owner[i] == o and row[i] == rr
                if rank >= 0 and o == rank and rr // P < cols:
                    assert slot[i] == tables[req[i], rr // P] * P + rr % P
                else:
                    assert slot[i] == -1


def test_slot_map_missing_page_gives_minus_one():
    table = np.array([[7, -1]], dtype=np.int32)
    _, row, slot = L.slot_map(np.array([0, 8, 16, 24, 10**6 * 8]), np.zeros(5, dtype=np.int64), 8, 1, 2, 0, table)
    assert row.tolist() == [0, 1, 2, 3, 10**6]
    assert slot.tolist() == [14, 15, -1, -1, -1]


def test_kv_write_owner_filtered_and_chunked_equals_one_shot():
    N, I, P = 8, 1, 4
    S = 1500
    rows = np.arange(S * 3, dtype=np.int64).reshape(S, 3)        # row p holds (3p, 3p+1, 3p+2)
    counts = L.local_counts(S, N, I)
    pages = -(-counts // P)
    cols = int(pages.max())
    for rank in range(N):
        table = np.random.default_rng(rank).permutation(cols + 5)[:cols].reshape(1, cols).astype(np.int32)
        pool = np.full(((cols + 5) * P, 3), -7, dtype=np.int64)
        pos = np.arange(S)
        req = np.zeros(S, dtype=np.int64)
        one = L.kv_write(pool, rows, pos, req, N, I, P, rank, table)
        chunked = pool
        for lo, hi in [(0, 1000), (1000, 1333), (1333, S)]:
            chunked = L.kv_write(chunked, rows[lo:hi], pos[lo:hi], req[lo:hi], N, I, P, rank, table)
        assert (one == chunked).all()
        # every owned position is at its slot, nothing else was touched
        written = (one != -7).all(axis=1)
        assert written.sum() == counts[rank]
        mine = np.arange(S)[np.arange(S) % N == rank]
        for j, p in enumerate(mine):
            slot = table[0, j // P] * P + j % P
            assert (one[slot] == rows[p]).all()
        # the middle chunk wrote exactly its interval share
        mid = L.kv_write(pool, rows[1000:1333], pos[1000:1333], req[1000:1333], N, I, P, rank, table)
        assert (mid != -7).all(axis=1).sum() == L.interval_counts(1000, 333, N, I)[rank]


# ---- prefill (DCP1) -> decode (DCP-N) token relayout -------------------------

def test_relayout_plan_reproduces_the_printed_extraction():
    g = golden("rank1_extraction.json")
    N, r, n, P = g["N"], g["rank"], g["length"], g["page_size"]
    pos, src, dst = L.relayout_plan(0, n, N, 1, r, np.array(g["source_pages"]), P, np.array([g["dest_page"]]), P)
    assert pos[: len(g["positions_head"])].tolist() == g["positions_head"] and pos[-1] == g["positions_last"]
    assert src.tolist() == g["source_slots"] and len(pos) == g["tokens_received"]
    lo, hi = g["dest_slot_range"]
    assert dst.tolist() == list(range(lo, hi + 1))


@pytest.mark.parametrize("N,I", [(8, 1), (4, 2), (8, 64), (3, 128)])
def test_relayout_moves_exactly_the_owned_positions_of_the_chunk(N, I):
    rng = np.random.default_rng(N + I)
    P = 64
    for start, length in [(0, 1), (0, 700), (1000, 333), (129, 64), (5, 0)]:
        end = start + length
        src_row = rng.permutation(64)[: -(-end // P)]
        for r in range(N):
            dst_row = rng.permutation(64)
            pos, src, dst = L.relayout_plan(start, length, N, I, r, src_row, P, dst_row, P)
            # exactly the rank's share of the chunk, in position order, by global position
            assert len(pos) == L.interval_counts(start, length, N, I)[r]
            assert ((pos >= start) & (pos < end)).all() and (np.diff(pos) > 0).all()
            assert all(block_rr(int(p), N, I)[0] == r for p in pos)
            # source slot = the position's row in the dense source pages
            assert (src == src_row[pos // P] * P + pos % P).all()
            # destination = the slot the owner-filtered write would give the same position
            _, _, want = L.slot_map(pos, np.zeros_like(pos), N, I, P, r, dst_row[None, :])
            assert (dst == want).all()


def test_relayout_then_decode_pool_equals_the_owner_filtered_write():
    rng = np.random.default_rng(3)
    N, I, P, S = 4, 2, 16, 150
    rows = rng.standard_normal((S, 5))
    src_row = rng.permutation(20)[: -(-S // P)]
    src_pool = np.full((20 * P, 5), np.nan)
    src_pool[src_row[np.arange(S) // P] * P + np.arange(S) % P] = rows
    for r in range(N):
        dst_row = rng.permutation(30)
        empty = np.full((30 * P, 5), np.nan)
        a = empty
        for start, length in [(0, 61), (61, 40), (101, 49)]:          # chunked transfer
            _, src, dst = L.relayout_plan(start, length, N, I, r, src_row, P, dst_row, P)
            a = L.relayout(a, src_pool, src, dst)
        b = L.kv_write(empty, rows, np.arange(S), np.zeros(S, dtype=np.int64), N, I, P, r, dst_row[None, :])
        assert np.array_equal(a, b, equal_nan=True)


# ---- a rank's share of a global sparse selection -----------------------------

@pytest.mark.parametrize("N,I", [(8, 1), (4, 2), (3, 64)])
def test_sparse_plan_keeps_exactly_the_owned_visible_selections(N, I):
    rng = np.random.default_rng(N * 7 + I)
    S, q_len, K = 500, 3, 40
    topk = np.full((q_len, K), -1, dtype=np.int64)
    for t in range(q_len):
        topk[t, :K - 3] = rng.choice(S + 20, size=K - 3, replace=False)     # some past the token's position
    kept = 0
    for r in range(N):
        rows, bits = L.sparse_plan(topk, S, N, I, r)
        pos = L.stripe_positions(S, N, I)[r]
        want_rows, want_bits = [], []
        for t in range(q_len):
            for p in topk[t]:
                if 0 <= p <= S - q_len + t and block_rr(int(p), N, I)[0] == r:
                    want_rows.append(int(np.searchsorted(pos, p)))            # its index in the rank's list
                    want_bits.append(1 << t)
        assert rows.tolist() == want_rows and bits.tolist() == want_bits
        kept += len(rows)
    assert kept == sum(int(((topk[t] >= 0) & (topk[t] <= S - q_len + t)).sum()) for t in range(q_len))
