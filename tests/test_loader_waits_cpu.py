"""Op-level replay of the loader wave's vector-memory counter.

The stripe kernel's loader wave waits for a tile with a hand-counted
`s_waitcnt vmcnt(N)` (N = 37 x the tiles issued after it, capped at 63):
the wait returns once at most N of the wave's vector-memory operations are
outstanding, and the counter drops in issue order.  Besides the 37
direct-to-LDS loads of a tile the wave issues other vector-memory
operations: the page-table load at the start and again when a chunk crosses
64 pages, and on the general path the per-lane row lookups of a tile.  The
compiler waits for each of those before it uses the value (a wait that
completes everything issued before it).

This replay issues the loader's operations in the kernel's order, applies
each wait, and checks that every tile a barrier hands to the other waves has
all 37 of its loads complete -- for the static loader of csrc/stripe_attn.hip
over chunks of every length, with page crossings and general tiles mixed in.
It also models the run-time tile hand-out that was tried and dropped (tiles
taken from a per-request counter by an agent-scope atomic, their start rows
passed to the other waves through a 4-slot LDS ring) to check its waits, its
ring reuse and its partition of the request's tiles.  Planted mistakes (a
tile with fewer loads than counted, a wait that counts a tile never issued)
must be caught.
"""

import numpy as np
import pytest

from test_kernel_bounds_cpu import STAGES, TILE_INSTS, kernel_constants

VMCNT_MAX = 63


class LoaderStream:
    """One wave's vector-memory operations; the counter drops in issue order."""

    def __init__(self):
        self.ops = []          # (kind, tile)
        self.done = 0          # ops[:done] are complete

    def issue(self, kind, tile=None):
        self.ops.append((kind, tile))
        return len(self.ops) - 1

    def consume(self, idx):
        """The compiler's wait for the value of op idx: it and everything before it complete."""
        self.done = max(self.done, idx + 1)

    def vmcnt(self, n):
        self.done = max(self.done, len(self.ops) - n)

    def complete(self, tile):
        return all(i < self.done for i, (k, t) in enumerate(self.ops) if k == "dma" and t == tile)


def issue_tile(ws, tile, dmas=TILE_INSTS, general=False, crosses=False, sparse=False):
    if crosses:                                 # a chunk crossing 64 pages reloads its page ids
        ws.consume(ws.issue("page_table", tile))
    if general:                                 # lanes 0..31 look up their row's address first
        if sparse:
            ws.consume(ws.issue("selection", tile))
        ws.consume(ws.issue("row", tile))
    for _ in range(dmas):
        ws.issue("dma", tile)


def wait_tiles(ws, after, per_tile=TILE_INSTS):
    n = 0 if after <= 0 else (per_tile if after == 1 else min(2 * per_tile, VMCNT_MAX))
    ws.vmcnt(n)


def replay_static(ntiles, general=(), crosses=(), sparse=False, aligned=True, plant=None, extra=()):
    """The static loader: prologue of min(3, ntiles) tiles, a wait for tile 0,
    then per iteration it a wait for tile it+1 and the issue of tile it+3.
    `extra` inserts other vector-memory operations (never waited for) after
    the given tiles' loads.  Returns the tiles found incomplete when handed over."""
    ws = LoaderStream()
    if aligned:
        ws.consume(ws.issue("page_table"))
    bad = []

    def issue(t):
        dmas = TILE_INSTS - 1 if (plant == "short_tile" and t == 2) else TILE_INSTS
        issue_tile(ws, t, dmas=dmas, general=t in general, crosses=t in crosses, sparse=sparse)
        if t in extra:
            ws.issue("extra", t)

    for t in range(min(STAGES - 1, ntiles)):
        issue(t)
    if ntiles:
        wait_tiles(ws, min(2, ntiles - 1))
        if not ws.complete(0):
            bad.append(0)
    for it in range(ntiles):
        after = 1 if it + 2 < ntiles else 0
        if plant == "phantom_tile" and it + 2 == ntiles:
            after = 1                           # counts a tile that is never issued
        wait_tiles(ws, after)
        if it + 1 < ntiles and not ws.complete(it + 1):
            bad.append(it + 1)
        if it + STAGES - 1 < ntiles:
            issue(it + STAGES - 1)
    return bad


def test_constants_are_the_kernels():
    k = kernel_constants()
    assert k["kTileInsts"] == TILE_INSTS and k["kStages"] == STAGES
    assert 2 * TILE_INSTS > VMCNT_MAX >= TILE_INSTS   # the two-tile wait is capped, so it waits for more


@pytest.mark.parametrize("ntiles", list(range(1, 12)) + [64, 129])
def test_static_loader_hands_over_only_landed_tiles(ntiles):
    rng = np.random.default_rng(ntiles)
    for trial in range(20):
        general = set(rng.choice(ntiles, size=rng.integers(0, ntiles + 1), replace=False).tolist())
        crosses = set(rng.choice(ntiles, size=rng.integers(0, 3), replace=False).tolist()) if ntiles > 2 else set()
        for sparse in (False, True):
            for aligned in (True, False):
                assert replay_static(ntiles, general, crosses, sparse, aligned) == [], (ntiles, trial)


def test_extra_operations_only_lengthen_a_wait():
    """Other vector-memory operations in the loader's stream (a counter atomic,
    a page-table load the value of which is not waited for) can only make a
    wait cover more: the counter drops in issue order."""
    rng = np.random.default_rng(7)
    for ntiles in (2, 3, 5, 17):
        for _ in range(30):
            extra = set(rng.choice(ntiles, size=rng.integers(1, ntiles + 1), replace=False).tolist())
            assert replay_static(ntiles, extra=extra) == []


def test_planted_count_mistakes_are_caught():
    # tile 2 with one load fewer than the wait for tile 1 allows in flight:
    # that wait returns while tile 1's last load is still in flight
    assert replay_static(6, plant="short_tile") == [1]
    # a wait that counts a tile never issued (the last tile of a chunk)
    assert replay_static(5, plant="phantom_tile") != []


# ---- the run-time tile hand-out (tried and dropped; not in the library) ----

def replay_handout(req_tiles, n, head_eighths, batch, order_rng, plant=None):
    """n chunks of one request share its tiles: chunk k first takes its equal
    share of the first head_eighths/8 of the tiles, then batches from a
    counter (an atomic whose value the compiler waits for).  Each chunk's
    loader writes the start tile of its i-th tile into LDS slot i % 4 when it
    takes it; every wave reads slot (it+1) % 4 after barrier A(it) and leaves
    the loop when it holds -1.  Chunks interleave their counter atomics in a
    random order.  Returns the tiles each chunk processed."""
    head = (req_tiles * head_eighths // 8) // n
    tail0 = head * n
    ctr = [0]
    state = []
    for k in range(n):
        state.append({"next": k * head, "end": (k + 1) * head, "done": False})

    def grab(k, ws):
        s = state[k]
        if s["done"]:
            return -1
        if s["next"] >= s["end"]:
            ws.consume(ws.issue("atomic"))
            s0 = ctr[0] + tail0
            ctr[0] += batch
            if s0 >= req_tiles:
                s["done"] = True
                return -1
            s["next"], s["end"] = s0, min(s0 + batch, req_tiles)
        t = s["next"]
        s["next"] += 1
        return t

    # each chunk runs as a generator that yields at its counter atomics, so the
    # chunks' atomics interleave
    processed = {k: [] for k in range(n)}

    def chunk(k):
        ws = LoaderStream()
        ring = [None] * STAGES
        written_at = [None] * STAGES               # barrier index of each slot's last write
        issued = []
        for i in range(STAGES - 1):
            yield
            J = grab(k, ws)
            ring[i], written_at[i] = J, -1
            if J >= 0:
                issue_tile(ws, J)
                issued.append(J)
        wait_tiles(ws, min(len(issued) - 1, 2) if issued else 0)
        if ring[0] is None or ring[0] < 0:
            return
        assert ws.complete(ring[0])
        tiles = [ring[0]]
        it = 0
        while True:
            after = 1 if len(issued) > it + 2 else 0
            wait_tiles(ws, after)                  # barrier A(it)
            slot = (it + 1) % STAGES
            Jn = ring[slot]
            assert written_at[slot] is not None and written_at[slot] < it, "slot read before its write"
            if Jn is not None and Jn >= 0:
                assert ws.complete(Jn), ("tile handed over before it landed", k, it, Jn)
            yield
            J3 = grab(k, ws)
            w = (it + STAGES - (2 if plant == "slot_too_early" else 1)) % STAGES
            # the slot written now held the tile of iteration it-1, read at A(it-2)
            ring[w], written_at[w] = J3, it
            if J3 >= 0:
                issue_tile(ws, J3)
                issued.append(J3)
            if Jn is None or Jn < 0:
                break
            tiles.append(Jn)
            it += 1
        processed[k] = tiles

    gens = [chunk(k) for k in range(n)]
    live = list(range(n))
    while live:
        k = live[order_rng.integers(len(live))]
        try:
            next(gens[k])
        except StopIteration:
            live.remove(k)
    return processed


@pytest.mark.parametrize("req_tiles,n", [(1, 2), (7, 4), (64, 4), (129, 4), (512, 4), (33, 8), (3, 8)])
@pytest.mark.parametrize("head_eighths,batch", [(6, 2), (8, 2), (6, 4), (0, 1)])
def test_handout_partitions_tiles_and_hands_over_landed_tiles(req_tiles, n, head_eighths, batch):
    """Under any interleaving of the chunks' atomics, the modelled hand-out
    processes every tile of the request exactly once, each ring slot is read
    only after the loader wrote it and before it is written again, and every
    tile is handed over only after its loads completed.  (The wrong outputs
    the hand-out gave on the GPU are therefore not explained by its load
    accounting or its ring as modelled here; the design stays out of the
    library.)"""
    rng = np.random.default_rng(req_tiles * 31 + n)
    for _ in range(10):
        got = replay_handout(req_tiles, n, head_eighths, batch, rng)
        all_tiles = sorted(t for ts in got.values() for t in ts)
        assert all_tiles == list(range(req_tiles))


def test_planted_ring_reuse_is_caught():
    """Writing the new start row one slot early overwrites a tile the other
    waves have not read yet: the replay loses that tile."""
    rng = np.random.default_rng(3)
    with pytest.raises(AssertionError):
        for _ in range(5):
            got = replay_handout(64, 4, 6, 2, rng, plant="slot_too_early")
            assert sorted(t for ts in got.values() for t in ts) == list(range(64))
