"""Host-side replay of the stripe-attention kernel's address arithmetic.

For every workgroup and every tile load of each full-size workload (pools
with no spare pages, exactly as the benchmark allocates them) this checks that
each 16-byte direct-to-LDS load reads a chunk of the tile's own page inside
the pool, and only rows of the split (rows the pool write filled), so no
stale or NaN row reaches the MFMAs; that the vector-memory wait at the top of
each iteration covers exactly the loads still in flight; and that the
epilogue's stores stay inside their buffers.  It mirrors the constants and
index math of csrc/stripe_attn.hip; planted copies of earlier mistakes (no
clamp of the fast path's tail slots, no substitution of rows past the split)
must be caught.
"""

import math
import os
import re

import numpy as np
import pytest

from mla_context_kv_amd import stripes, workloads

import gpu_helpers as H

TILE, ROW_SLOTS, CHUNKS = 32, 73, 72
TILE_SLOTS = TILE * ROW_SLOTS
STAGES, MAX_RB = 4, 3
LAST_BASE = TILE_SLOTS - 64

KERNEL_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                          "mla_context_kv_amd", "csrc", "stripe_attn.hip")


def kernel_constants():
    """The integer constexpr constants of the kernel source, evaluated from
    their definitions (integer literals and earlier constants combined with
    + - * / and parentheses)."""
    src = open(KERNEL_SRC).read()
    env = {}
    for name, expr in re.findall(r"constexpr\s+int\s+(k\w+)\s*=\s*([^;]+);", src):
        e = re.sub(r"//.*", "", expr).strip()
        if not re.fullmatch(r"[\w\s+\-*/()]+", e):
            continue
        e = e.replace("/", "//")
        try:
            env[name] = int(eval(e, {"__builtins__": {}}, dict(env)))
        except (NameError, SyntaxError):
            pass
    return env


def test_replay_constants_are_the_kernels():
    """The replay below re-types the kernel's tile geometry and plan limits;
    a kernel edit that changes any of them without a mirror edit here fails."""
    k = kernel_constants()
    assert k["kTile"] == TILE and k["kRowSlots"] == ROW_SLOTS and k["kChunks"] == CHUNKS
    assert k["kTileSlots"] == TILE_SLOTS and k["kLastBase"] == LAST_BASE
    assert k["kStages"] == STAGES and k["kMaxRB"] == MAX_RB
    assert k["kTileInsts"] == TILE_INSTS and k["kGroupChunkTiles"] == GROUP_CHUNK
    assert k["kChunkGroup"] == CHUNK_GROUP


TILE_INSTS = -(-TILE_SLOTS // 64)                 # 37
CHUNK_GROUP = 4


def load_slots():
    """Tile slot of every lane of every load instruction of the workgroup: the
    loader wave issues instructions g = 0..36, instruction g filling the 64
    slots from min(64 g, 2272)."""
    g = np.arange(TILE_INSTS)
    s0 = np.minimum(64 * g, LAST_BASE)
    return (s0[:, None] + np.arange(64)[None, :]).reshape(-1), s0


def test_loads_cover_every_slot_of_one_stage():
    s, s0 = load_slots()
    assert s.min() == 0 and s.max() == TILE_SLOTS - 1            # never past the stage
    assert set(s.tolist()) == set(range(TILE_SLOTS))             # every slot written
    assert len(s0) <= 63                                         # one tile fits the load counter


def plan(B, M, bt_cols, P, cus=256, num_splits=0):
    # query-row blocks of 32 per workgroup: up to 3; above 96 rows, the count
    # that pads the fewest rows when the rows are cut into groups
    if M <= 32 * MAX_RB:
        W = -(-M // 32)
    else:
        W = min(range(MAX_RB, 0, -1), key=lambda rb: (-(-M // (32 * rb)) * 32 * rb, -rb))
    mgroups = -(-M // (32 * W))
    tiles_max = -(-(bt_cols * P) // TILE)
    if num_splits > 0:
        forced = min(num_splits, tiles_max)
        target = 0
        slots = B * forced
    else:
        forced = 0
        target = max(cus // mgroups, 1)
        slots = target if target > B else target + B
        if target <= B and mgroups > 1:
            slots = max(slots, B * (-(-tiles_max // GROUP_CHUNK) + 1))
    slots = -(-slots // (8 * CHUNK_GROUP)) * 8 * CHUNK_GROUP   # groups of chunks go to the 8 XCDs in turn
    return W, mgroups, slots, forced, target


def block_item(bid, mgroups):
    """The kernel's block order: block bid runs on XCD bid % 8; it is row
    group (bid // 8) % mgroups of the j-th chunk of that XCD, j = bid // 8 //
    mgroups, and groups of CHUNK_GROUP consecutive chunks go to the XCDs in turn."""
    bx, bk = bid & 7, bid >> 3
    j = bk // mgroups
    return ((j // CHUNK_GROUP) * 8 + bx) * CHUNK_GROUP + j % CHUNK_GROUP, bk % mgroups


def test_block_order_is_a_bijection_that_spreads_live_chunks():
    for slots in (32, 64, 256, 512, 416):
        for mgroups in (1, 2, 3, 4):
            items = [block_item(b, mgroups) for b in range(slots * mgroups)]
            assert sorted(items) == [(c, g) for c in range(slots) for g in range(mgroups)]
            # the row groups of a chunk sit on one XCD, in consecutive blocks of it
            for c in range(slots):
                bids = [b for b, it in enumerate(items) if it[0] == c]
                assert len({b % 8 for b in bids}) == 1
                assert sorted(b // 8 for b in bids) == list(range(min(b // 8 for b in bids),
                                                                  min(b // 8 for b in bids) + mgroups))
            # any number of live chunks (the first L) spreads over the 8 XCDs to
            # within one group; a group of consecutive chunks shares an XCD
            for live in (1, 7, 9, slots // 2, slots - 3):
                per_xcd = np.bincount([b % 8 for b, it in enumerate(items) if it[0] < live], minlength=8)
                assert per_xcd.max() - per_xcd.min() <= CHUNK_GROUP * mgroups
            xcd_of = {it[0]: b % 8 for b, it in enumerate(items)}
            assert all(xcd_of[c] == xcd_of[c - c % CHUNK_GROUP] for c in range(slots))


def cdiv(a, b):
    return -(-a // b)


GROUP_CHUNK = 512          # longest chunk when the rows are cut into several groups


def work_list(tiles, forced, target, mgroups=1):
    """The kernel's chunks in chunk order: (request, chunk of it, its chunk
    count, chunk length in tiles).  Every request gets at least one chunk."""
    B = len(tiles)
    if forced > 0:
        n = [cdiv(t, cdiv(t, forced)) if t > 0 else 1 for t in tiles]
    else:
        total = int(sum(tiles))
        chunks_for = lambda C: sum(max(cdiv(t, C), 1) for t in tiles)
        if target <= B:
            C = max(cdiv(total, target), 1)          # chunks of the mean per-unit share
            if mgroups > 1:
                C = min(C, GROUP_CHUNK)
        else:
            C = max(cdiv(total, target), 1)
            if chunks_for(C) > target:               # the shortest length that fits one round, by bisection
                lo, hi = C + 1, max(cdiv(total, target - B), 1)
                while lo < hi:
                    mid = lo + (hi - lo) // 2
                    if chunks_for(mid) <= target:
                        hi = mid
                    else:
                        lo = mid + 1
                C = lo
        n = [max(cdiv(t, C), 1) for t in tiles]
    out = []
    for b, t in enumerate(tiles):
        cs = cdiv(t, n[b]) if t > 0 else 0
        out += [(b, k, n[b], cs) for k in range(n[b])]
    return out


def test_work_list_fits_the_grid_and_partitions_every_request():
    """Over random batches (uniform, log-uniform, empty, huge) the chunks never
    outnumber the grid's slots and tile each request exactly once, and the
    balanced list keeps the longest chunk within twice the mean."""
    rng = np.random.default_rng(5)
    for trial in range(400):
        B = int(rng.integers(1, 300))
        kind = trial % 4
        if kind == 0:
            tiles = np.full(B, int(rng.integers(0, 600)))
        elif kind == 1:
            tiles = np.rint(np.exp(rng.uniform(0, np.log(2048), B))).astype(int)
        elif kind == 2:
            tiles = rng.integers(0, 4, B)
        else:
            tiles = rng.integers(0, 40000, B)
        for mgroups in (1, 2, 4):
            for ns in (0, 1, 3, 8):
                forced = min(ns, 10 ** 6) if ns else 0
                target = 0 if ns else max(256 // mgroups, 1)
                slots = B * forced if ns else (target if target > B else target + B)
                if not ns and target <= B and mgroups > 1:
                    slots = max(slots, B * (-(-int(tiles.max(initial=0)) // GROUP_CHUNK) + 1))
                wl = work_list(list(tiles), forced, target, mgroups)
                assert len(wl) <= slots
                for b in range(B):
                    mine = [(k, n, cs) for (bb, k, n, cs) in wl if bb == b]
                    assert [k for k, _, _ in mine] == list(range(len(mine))) and mine[0][1] == len(mine)
                    cs = mine[0][2]
                    covered = sum(max(0, min((k + 1) * cs, tiles[b]) - k * cs) for k, _, _ in mine)
                    assert covered == tiles[b] and (len(mine) - 1) * cs < max(tiles[b], 1)
                if not ns and tiles.sum() > 0 and target > B:
                    assert max(cs for (_, _, _, cs) in wl) <= 2 * cdiv(int(tiles.sum()), target - B) + 1
                if not ns and tiles.sum() > 0 and target <= B:
                    # no chunk longer than the mean share of a compute unit (nor the group cap)
                    cap = cdiv(int(tiles.sum()), target)
                    assert max(cs for (_, _, _, cs) in wl) <= (min(cap, GROUP_CHUNK) if mgroups > 1 else cap)


def test_one_round_chunk_length_is_the_shortest_that_fits():
    """Fewer requests than workgroups: the balanced list's chunk length is the
    smallest whose chunk count fits one round (brute force over every
    length), whatever the mix of short and long requests."""
    rng = np.random.default_rng(17)
    for trial in range(200):
        B = int(rng.integers(1, 255))
        tiles = [int(x) for x in np.rint(np.exp(rng.uniform(0, np.log(rng.choice([8, 300, 5000])), B)))]
        if trial % 3 == 0:
            tiles[: B // 2] = [1] * (B // 2)
        target = 256
        wl = work_list(tiles, 0, target)
        count = lambda L: sum(max(cdiv(t, L), 1) for t in tiles)
        best = next(L for L in range(1, max(tiles) + 2) if count(L) <= target)
        assert len(wl) == count(best) <= target
        # no chunk longer than that length
        assert max(cs for (_, _, _, cs) in wl) <= best


def chunk_class(cs):
    """The kernel's chunk class: chunks of about 2**(30 - key) tiles; 31 = empty."""
    return 30 - (int(cs).bit_length() - 1) if cs > 0 else 31


def class_order(tiles, target, mgroups=1):
    """The many-request plan (target <= requests): the same chunks as
    work_list, numbered class by class, longest class first, request by
    request inside a class.  Returns [(b, k, n, cs)] in chunk order."""
    wl = work_list(tiles, 0, target, mgroups)
    per_req = {}
    for (b, k, n, cs) in wl:
        per_req.setdefault(b, []).append((b, k, n, cs))
    out = []
    for key in range(32):
        for b in range(len(tiles)):
            chunks = per_req[b]
            if chunk_class(chunks[0][3]) == key:
                out += chunks
    return out


def test_class_order_is_longest_first_and_keeps_requests_together():
    rng = np.random.default_rng(9)
    for trial in range(60):
        B = int(rng.integers(257, 1200))
        tiles = [int(x) for x in np.exp(rng.uniform(0, np.log(300), B)).astype(int)]
        tiles[:7] = [0, 1, 2, 3, 0, 5, 6]
        target = 256
        order = class_order(tiles, target)
        assert sorted(order) == sorted(work_list(tiles, 0, target))       # the same chunks
        keys = [chunk_class(cs) for (_, _, _, cs) in order]
        assert keys == sorted(keys)                                        # longest class first
        # a request's chunks are consecutive, k = 0..n-1
        pos = {}
        for c, (b, k, n, cs) in enumerate(order):
            pos.setdefault(b, []).append((c, k))
        for b, ck in pos.items():
            cs_ = [c for c, _ in ck]
            assert cs_ == list(range(cs_[0], cs_[0] + len(cs_))) and [k for _, k in ck] == list(range(len(ck)))
        assert len(order) <= target + B                                    # the plan's slot bound


def block_find(tiles, target, c, threads=512, plant=None):
    """The workgroup-wide lookup of the many-request plan (above 512
    requests): thread i takes the contiguous run of requests i*q .. i*q+q-1,
    counts the chunks of chunk c's class in its run, and the one thread whose
    prefix range holds c's rank in the class walks its run.  Returns
    (b, k, n, cs) or None past the last chunk."""
    B = len(tiles)
    C = max(cdiv(int(sum(tiles)), target), 1)
    nb = [max(cdiv(t, C), 1) for t in tiles]
    cs = [cdiv(t, n) if t > 0 else 0 for t, n in zip(tiles, nb)]
    key = [chunk_class(x) for x in cs]
    counts = [sum(n for n, k in zip(nb, key) if k == kk) for kk in range(32)]
    incl = np.cumsum(counts)
    hit = [kk for kk in range(32) if incl[kk] - counts[kk] <= c < incl[kk]]
    if not hit:
        return None
    kk = hit[0]
    r = c - (incl[kk] - counts[kk])
    q = cdiv(B, threads)
    runs = [range(i * q, min(i * q + q, B)) for i in range(threads)]
    s = [sum(nb[v] for v in run if key[v] == kk) for run in runs]
    excl = 0
    for i, run in enumerate(runs):
        lo = excl + (1 if plant == "off_by_one" else 0)
        if s[i] > 0 and lo <= r < excl + s[i]:
            acc = excl
            for v in run:
                if key[v] != kk:
                    continue
                if r < acc + nb[v]:
                    return (v, r - acc, nb[v], cs[v])
                acc += nb[v]
        excl += s[i]
    return "lost"


def test_block_find_is_the_class_order():
    """Over random many-request batches (more requests than threads, fewer,
    empty ones), the workgroup-wide lookup finds for every chunk the request
    and chunk that the class order numbers there, and nothing past the end; a
    planted off-by-one in the prefix test is caught."""
    rng = np.random.default_rng(13)
    for trial in range(24):
        B = int(rng.integers(513, 2305)) if trial % 3 else int(rng.integers(257, 600))
        tiles = [int(x) for x in np.exp(rng.uniform(0, np.log(400), B)).astype(int)]
        tiles[:5] = [0, 1, 0, 3, 2]
        order = class_order(tiles, 256)
        for c in list(range(0, len(order), max(1, len(order) // 97))) + [len(order) - 1]:
            assert block_find(tiles, 256, c) == order[c]
        assert block_find(tiles, 256, len(order)) is None
    bad = [block_find(tiles, 256, c, plant="off_by_one") for c in range(len(order))]
    assert any(x != order[c] for c, x in enumerate(bad))


SMALL_PER_LANE = 4          # requests per lane of the register lookup


def register_find(tiles, target, c, plant=None):
    """The one-round lookup from registers (fewer requests than workgroups,
    at most 64 x SMALL_PER_LANE of them): lane l of the wave holds requests
    l, l + 64, ...; the chunk length is found by the same bisection over wave
    sums, then each block of 64 requests is scanned with the previous
    blocks' total carried in, and the first lane whose range holds c wins.
    Returns (b, k, n, cs) or None past the last chunk."""
    B = len(tiles)
    lanes = [[tiles[64 * k + l] if 64 * k + l < B else None for k in range(SMALL_PER_LANE)] for l in range(64)]
    total = sum(t for lane in lanes for t in lane if t is not None)

    def chunks_for(L):
        return sum(max(cdiv(t, L), 1) for lane in lanes for t in lane if t is not None)

    C = max(cdiv(total, target), 1)
    if chunks_for(C) > target:
        lo, hi = C + 1, max(cdiv(total, target - B), 1)
        while lo < hi:
            mid = lo + (hi - lo) // 2
            if chunks_for(mid) <= target:
                hi = mid
            else:
                lo = mid + 1
        C = lo
    carry = 0
    for k in range(SMALL_PER_LANE):
        if 64 * k >= B:
            break
        nb = [max(cdiv(lanes[l][k], C), 1) if lanes[l][k] is not None else 0 for l in range(64)]
        incl = list(np.cumsum(nb) + carry)
        for l in range(64):
            excl = incl[l] - nb[l]
            lo = excl + (1 if plant == "off_by_one" else 0)
            if lanes[l][k] is not None and lo <= c < incl[l]:
                t = lanes[l][k]
                return (64 * k + l, c - excl, nb[l], cdiv(t, nb[l]) if t > 0 else 0)
        carry = incl[63] if plant != "no_carry" else 0
    return None


def test_register_find_is_the_work_list():
    """Over random one-round batches of 1 to 255 requests (empty, short and
    long ones, every block count of the lanes' registers) the register lookup
    finds for every chunk the request and chunk the work list numbers there,
    and nothing past the end; a dropped carry between blocks and an off-by-one
    in the range test are caught.  The kernel takes this path only below the
    lanes' capacity, which is the constant mirrored here."""
    k = kernel_constants()
    assert k["kSmallPerLane"] == SMALL_PER_LANE
    src = open(KERNEL_SRC).read()
    assert "Bv <= 64 * kSmallPerLane" in src and "p.target_chunks > Bv" in src
    rng = np.random.default_rng(23)
    for trial in range(40):
        B = int(rng.integers(1, 256)) if trial > 3 else [1, 64, 65, 255][trial]
        tiles = [int(x) for x in np.rint(np.exp(rng.uniform(0, np.log(rng.choice([4, 400, 9000])), B)))]
        tiles[: min(3, B)] = [0, 1, 0][: min(3, B)]
        wl = work_list(tiles, 0, 256)
        for c in range(len(wl)):
            assert register_find(tiles, 256, c) == wl[c]
        assert register_find(tiles, 256, len(wl)) is None
    tiles = [int(x) for x in rng.integers(1, 50, 200)]
    wl = work_list(tiles, 0, 256)
    for plant in ("off_by_one", "no_carry"):
        assert any(register_find(tiles, 256, c, plant=plant) != wl[c] for c in range(len(wl)))


def chunk_table(tiles, forced, target, slots, mgroups=1, plant=None):
    """The chunk table the combine reads in the many-request plan: each
    request's first chunk, if it has a workgroup (chunk index < slots), writes
    (chunks cut to the slots there are, first chunk); the call is flagged when
    the chunks outnumber the slots."""
    order = class_order(tiles, target, mgroups)
    table, flagged = {}, len(order) > slots
    for c, (b, k, n, cs) in enumerate(order):
        if k == 0 and c < slots:
            fit = n if (c + n <= slots or plant == "no_table_clamp") else slots - c
            flagged |= fit != n
            table[b] = (fit, c)
    return list(table.values()), flagged


def test_chunk_table_never_points_past_the_workspace():
    """Device lengths past the page table's capacity (the plan sizes the
    workspace from the table) on the capped row-group path: every entry the
    combine can read is cut to the slots, so it reads inside the workspace,
    and the call is flagged; within capacity nothing is cut.  (An entry no
    workgroup writes is rejected by the combine's own range check.)"""
    B, cols, P, M = 256, 256, 64, 384                  # 4 row groups of 96 rows: capped chunks
    W, mgroups, slots, forced, target = plan(B, M, cols, P)
    assert mgroups > 1 and target <= B
    fits = [cdiv(cols * P, TILE)] * B                  # every request at the table's capacity
    table, flagged = chunk_table(fits, forced, target, slots, mgroups)
    assert not flagged and len(table) == B and all(c0 + n <= slots for n, c0 in table)
    over = [8 * cdiv(cols * P, TILE)] * B               # lengths 8x the capacity
    over[0] = 3 * GROUP_CHUNK                           # (so that one request's chunks straddle the last slot)
    table, flagged = chunk_table(over, forced, target, slots, mgroups)
    assert flagged and all(c0 + n <= slots for n, c0 in table if n > 0)
    table, _ = chunk_table(over, forced, target, slots, mgroups, plant="no_table_clamp")
    assert any(c0 + n > slots for n, c0 in table)      # what the clamp prevents


def count_rows(x, N, I, r):
    x = np.asarray(x, dtype=np.int64)
    rnd = N * I
    rem = np.clip(x % rnd - r * I, 0, I)
    return np.where(x <= 0, 0, (x // rnd) * I + rem)


def fast_chunks(plant=None):
    """Global chunk (0..2303 of the tile's 36,864 contiguous bytes) each slot of a fast tile loads."""
    s, _ = load_slots()
    q = s * 57457 >> 22
    assert (q == s // 73).all()                       # the kernel's division by 73
    g = s - q
    if plant != "no_fast_clamp":
        g = np.minimum(g, TILE * CHUNKS - 1)
    return g


def general_rows_chunks(rows_left, plant=None):
    """(tile row, chunk) each slot of a general (partial or unaligned) tile loads."""
    s, _ = load_slots()
    tt, c = s // ROW_SLOTS, s % ROW_SLOTS
    if plant != "no_row_substitute":
        tt = np.where(tt < rows_left, tt, 0)
    c = np.minimum(c, CHUNKS - 1)
    return tt, c


def check_waits(ntiles, stages):
    """Each wait allows exactly the loads of the live tiles issued after the tile it
    waits for: tile 0 before the loop, then tile it+1 at the top of iteration it
    (whose PV uses tile it and whose QK^T uses tile it+1); tile it+3 is issued
    after that wait, into the stage of tile it-1."""
    issued = list(range(min(stages - 1, ntiles)))     # prologue

    def wait_for(tile, allowed_tiles):
        later = [t for t in issued if t > tile]
        assert tile in issued
        assert len(later) == allowed_tiles, (ntiles, tile, later, allowed_tiles)

    if ntiles:
        wait_for(0, min(2, ntiles - 1))
    for it in range(ntiles):
        if it + 1 < ntiles:
            wait_for(it + 1, 1 if it + 2 < ntiles else 0)
        else:
            assert [t for t in issued if t > it] == []
        nt = it + stages - 1
        if nt < ntiles:
            assert (nt - (it - 1)) % stages == 0            # reuses the stage of tile it-1
            issued.append(nt)
        # stages in use during iteration it: it (PV), it+1 (QK^T), it+2 and it+3 landing
        live = [t for t in issued if it <= t <= it + 3]
        assert len(live) <= stages


def test_wait_counts_cover_the_tail():
    for ntiles in range(1, 12):
        check_waits(ntiles, STAGES)


def check_workload(w, I, plant=None, num_splits=0, window=0, partials=0):
    lens = workloads.seq_lens(w)
    N, P = w.N, w.page_size
    counts = H.oracle_counts(lens, N, I)
    tables, pool_pages = workloads.make_block_tables(w, stripes.pages_from_counts(counts, P), 0)
    M = w.q_len * w.H
    for r in range(N):
        tab = tables[r]
        B, cols = tab.shape
        W, mgroups, slots, forced, target = plan(B, M, cols, P, num_splits=num_splits)
        g = fast_chunks(plant)
        max_vis = count_rows(lens, N, I, r)
        # with a sliding window a request starts at the tile holding the first
        # row its first query sees
        first = count_rows(lens - w.q_len + 1 - window, N, I, r) if window > 0 else np.zeros_like(max_vis)
        ft = [int(f) // TILE for f in first]
        tiles = [cdiv(int(v), TILE) - ft[b] if v > 0 else 0 for b, v in enumerate(max_vis)]
        if partials:
            # unmerged parts: exactly k per request, ceil(t / k) tiles each
            slots = B * partials
            wl = [(b, c, partials, cdiv(t, partials) if t else 0) for b, t in enumerate(tiles) for c in range(partials)]
        else:
            wl = work_list(tiles, forced, target, mgroups)
        assert len(wl) <= slots                        # every chunk has a workgroup
        for (b, sp, nchunks, cs) in wl:
            if True:
                row_lo = (ft[b] + sp * cs) * TILE
                row_hi = min(row_lo + cs * TILE, int(max_vis[b]))
                ntiles = -(-(row_hi - row_lo) // TILE) if row_hi > row_lo else 0
                for it in range(ntiles):                  # tiles past the split issue no loads
                    J = row_lo + it * TILE
                    rows_left = row_hi - J
                    if P % TILE == 0 and rows_left >= TILE:
                        # fast path: slot s loads chunk g[s] of the tile's 32 contiguous rows
                        pi = J // P
                        assert pi < cols and 0 <= tab[b, pi] < pool_pages
                        assert J % P + TILE <= P                   # the tile lies inside its page
                        assert g.min() >= 0 and g.max() < TILE * CHUNKS, (w.name, r, b, sp, it)
                        continue
                    tt, c = general_rows_chunks(rows_left, plant)
                    j = J + tt
                    assert (j < row_hi).all(), (w.name, r, b, sp, it, "row past the split")
                    pi = j // P
                    assert (pi < cols).all()
                    pg = tab[b, pi]
                    assert (pg >= 0).all() and (pg < pool_pages).all()
                    assert (c < CHUNKS).all()
        # epilogue: partial / final rows stay inside their buffers
        assert mgroups * 32 * W >= M
        assert (slots - 1) * M + (M - 1) < slots * M


@pytest.mark.parametrize("name,I", [("tiny", 1), ("dsv3", 1), ("k3", 1), ("ragged", 1), ("long", 1), ("long", 64),
                                    ("dsv3", 128), ("long", 256)])
def test_dma_loads_stay_in_the_tile_page(name, I):
    check_workload(workloads.WORKLOADS[name], I)


@pytest.mark.parametrize("name,I,k", [("k3", 1, 4), ("ragged", 1, 3), ("long", 64, 7), ("tiny", 1, 5)])
def test_unmerged_parts_stay_in_the_tile_page(name, I, k):
    check_workload(workloads.WORKLOADS[name], I, partials=k)


@pytest.mark.parametrize("name,I,window", [("tiny", 1, 100), ("ragged", 1, 1000), ("dsv3", 1, 4097),
                                           ("long", 64, 70000)])
def test_window_chunks_stay_in_the_tile_page(name, I, window):
    check_workload(workloads.WORKLOADS[name], I, window=window)


def test_planted_missing_fast_clamp_is_caught():
    """Without the clamp, the pad slot of the tile's last row maps to the
    chunk just past the tile's 36,864 bytes."""
    for name in ("dsv3", "k3"):
        with pytest.raises(AssertionError):
            check_workload(workloads.WORKLOADS[name], 1, plant="no_fast_clamp")


def test_planted_missing_row_substitution_is_caught():
    """Without the substitution, a partial tile loads rows past the split's end
    (rows the pool write never filled)."""
    with pytest.raises(AssertionError):
        check_workload(workloads.WORKLOADS["ragged"], 1, plant="no_row_substitute")


def test_plan_matches_library_workspace():
    import ctypes
    from mla_context_kv_amd import dcp
    L = dcp.lib()
    for B, q_len, H_, cols, P, ns in [(64, 1, 96, 256, 64, 4), (32, 1, 128, 16, 64, 8), (8, 4, 96, 2048, 64, 32),
                                      (2, 1, 16, 16, 16, 0 or 1)]:
        a = dcp.dcp_attn_args()
        a.layout = dcp.layout(8, 1, P)
        a.rank, a.batch, a.q_len, a.n_heads, a.head_dim, a.v_dim = 0, B, q_len, H_, 576, 512
        a.num_pages, a.bt_cols, a.num_splits = 10, cols, ns
        n = ctypes.c_size_t(0)
        assert L.dcp_stripe_attn_workspace(ctypes.byref(a), ctypes.byref(n)) == 0
        W, mg, slots, forced, target = plan(B, q_len * H_, cols, P, num_splits=ns)
        part = slots * q_len * H_ * (512 * 2 + 4)       # bf16 o and float32 lse per chunk partial row
        want = 0 if forced == 1 else cdiv(part, 256) * 256 + 2 * B * 4
        assert n.value == want


def part_slot(c, slots, group=CHUNK_GROUP):
    """Workspace slot of chunk c's partial: chunk c mod group of every group of
    consecutive chunks goes to region c mod group, at c / group within it."""
    return (c % group) * (slots // group) + c // group


def test_partial_slots_are_a_bijection_inside_the_workspace():
    """The kernel writes chunk c's partial to slot part_slot(c) and the
    combine reads a request's chunks c0..c0+n-1 through the same map: for
    every slot count the plan can make (a multiple of 8 x kChunkGroup) the map
    is a permutation of the slots, so no two chunks share a slot and no read
    leaves the workspace; the uniform 4-chunk plan lands on the unmerged
    parts' layout (part k of request b at k x B + b).  A map that drops the
    region offset is caught."""
    src = open(KERNEL_SRC).read()
    assert "return (c % kChunkGroup) * (p.slots / kChunkGroup) + c / kChunkGroup;" in src
    for slots in range(8 * CHUNK_GROUP, 8 * CHUNK_GROUP * 40, 8 * CHUNK_GROUP):
        m = [part_slot(c, slots) for c in range(slots)]
        assert sorted(m) == list(range(slots))
    B = 64
    assert all(part_slot(4 * b + k, 4 * B) == k * B + b for b in range(B) for k in range(4))
    bad = [(c % CHUNK_GROUP) + c // CHUNK_GROUP for c in range(256)]
    assert sorted(bad) != list(range(256))
