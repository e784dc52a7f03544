"""Oracle: which rank owns a token, where it is stored, and how many each rank holds.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The striping is produced by walking the positions in order and handing them
out, exactly as the pages describe it, rather than from a closed form:

* Page "DCP" (zdszero), section "core abstraction", idea one: rank r owns the
  positions whose residue mod N is r and stores them compactly as local rows
  0, 1, 2, ... in increasing position order.
* Page "PCP/DCP" (obnotes), section 6 "Block RR": with block size I the
  positions are handed out in consecutive runs of I, one run per rank in turn
  (I = 1 is the token round robin of section 5).
* Page "PCP/DCP", section "KV cache management": a row's physical slot is
  page_id * page_size + offset inside the page, the page id coming from the
  request's page (block) table.
* Page "DCP", idea one: the share of the interval [a, a+L) that rank r holds is
  count_r(a+L) - count_r(a), count_r(x) being the number of positions in
  [0, x) that rank r owns (page "PCP/DCP" section 6 states the same with
  global positions).

The closed forms on the pages (p mod N and p div N; the block-RR owner, local
index and local_len; the virtual-block formula of the vLLM-Ascend CP design)
are deliberately not used here: the tests compare this simulation with them.
"""

from __future__ import annotations

import numpy as np


def stripe_positions(S: int, N: int, I: int) -> list[np.ndarray]:
    """Hand out positions 0..S-1 to N ranks in runs of I, round robin.

    Returns N int64 arrays.  Entry j of array r is the global position that
    rank r stores at local row j (rows are compact and in position order).
    """
    if N < 1 or I < 1 or S < 0:
        raise ValueError("need N >= 1, I >= 1, S >= 0")
    lists: list[list[int]] = [[] for _ in range(N)]
    rank = 0
    p = 0
    while p < S:
        run_end = min(p + I, S)
        lists[rank].extend(range(p, run_end))
        p = run_end
        rank += 1
        if rank == N:
            rank = 0
    return [np.asarray(l, dtype=np.int64) for l in lists]


def owner_and_row_table(S: int, N: int, I: int) -> tuple[np.ndarray, np.ndarray]:
    """owner[p] and row[p] for every p < S, read off the simulated hand-out."""
    owner = np.full(S, -1, dtype=np.int32)
    row = np.full(S, -1, dtype=np.int64)
    for r, pos in enumerate(stripe_positions(S, N, I)):
        owner[pos] = r
        row[pos] = np.arange(len(pos), dtype=np.int64)
    return owner, row


def owner_row_walk(p: int, N: int, I: int) -> tuple[int, int]:
    """Owner and local row of one (possibly huge) position.

    One full round of the hand-out covers N*I positions and gives every rank
    exactly I of them, so the rounds completed before p contribute
    (p // (N*I)) * I rows to each rank; the walk then hands out the runs of the
    current round one at a time until it reaches p.
    """
    if p < 0:
        raise ValueError("position must be >= 0")
    round_len = N * I
    rounds_done = p // round_len
    start = rounds_done * round_len
    rank = 0
    run_start = start
    while True:
        run_end = run_start + I
        if p < run_end:
            return rank, rounds_done * I + (p - run_start)
        run_start = run_end
        rank += 1


def local_counts(x: int, N: int, I: int) -> np.ndarray:
    """count_r(x) for every rank r: how many of the positions [0, x) rank r owns."""
    return np.array([len(l) for l in stripe_positions(x, N, I)], dtype=np.int64)


def interval_counts(a: int, L: int, N: int, I: int) -> np.ndarray:
    """Share of each rank in the positions [a, a+L): count_r(a+L) - count_r(a)."""
    return local_counts(a + L, N, I) - local_counts(a, N, I)


def page_slot(block_table_row: np.ndarray, local_row: np.ndarray, page_size: int) -> np.ndarray:
    """Physical slot of a local row: page id of its page times page size plus
    the offset inside the page.  Rows whose page entry is missing or negative
    map to -1."""
    return page_slots(np.asarray(block_table_row)[None, :], np.zeros(np.shape(local_row), dtype=np.int64),
                      local_row, page_size)


def page_slots(block_table: np.ndarray, req: np.ndarray, local_row: np.ndarray, page_size: int) -> np.ndarray:
    """page_slot for many rows at once: row i of request req[i] sits at
    block_table[req[i], local_row[i] // page_size] * page_size + local_row[i] % page_size
    (-1 where the request or page index is outside the table or the entry is negative)."""
    block_table = np.asarray(block_table, dtype=np.int64)
    req = np.asarray(req, dtype=np.int64)
    local_row = np.asarray(local_row, dtype=np.int64)
    page_idx = local_row // page_size
    offset = local_row % page_size
    rows, cols = block_table.shape
    inside = (req >= 0) & (req < rows) & (page_idx >= 0) & (page_idx < cols)
    page = np.full(local_row.shape, -1, dtype=np.int64)
    page[inside] = block_table[req[inside], page_idx[inside]]
    out = np.full(local_row.shape, -1, dtype=np.int64)
    ok = page >= 0
    out[ok] = page[ok] * page_size + offset[ok]
    return out


def slot_map(pos: np.ndarray, req: np.ndarray, N: int, I: int, page_size: int,
             rank: int, block_table: np.ndarray | None):
    """owner, local row and physical slot on ``rank`` of each (request, position).

    slot is -1 when the position is not owned by ``rank`` (or rank < 0, or no
    block table is given, or the table has no page for that row).
    """
    pos = np.asarray(pos, dtype=np.int64)
    req = np.asarray(req, dtype=np.int64)
    n = pos.shape[0]
    owner = np.empty(n, dtype=np.int32)
    row = np.empty(n, dtype=np.int64)
    if n:
        top = int(pos.max()) + 1
        if top <= (1 << 22):
            own_t, row_t = owner_and_row_table(top, N, I)
            owner[:] = own_t[pos]
            row[:] = row_t[pos]
        else:
            for i in range(n):
                o, r = owner_row_walk(int(pos[i]), N, I)
                owner[i] = o
                row[i] = r
    slot = np.full(n, -1, dtype=np.int64)
    if rank >= 0 and block_table is not None:
        mine = owner == rank
        slot[mine] = page_slots(block_table, req[mine], row[mine], page_size)
    return owner, row, slot


def kv_write(pool: np.ndarray, kv_rows: np.ndarray, pos: np.ndarray, req: np.ndarray,
             N: int, I: int, page_size: int, rank: int, block_table: np.ndarray) -> np.ndarray:
    """Owner-filtered paged write (page "MLA 的 DCP", section 4, stage 2).

    ``pool`` is rank ``rank``'s pool viewed as [num_pages * page_size, row_dim]
    (any dtype; it is copied, not modified).  Row i of ``kv_rows`` is stored at
    its slot only if ``rank`` owns ``pos[i]``; rows owned by other ranks are
    skipped.  Returns the new pool.
    """
    out = pool.copy()
    _, _, slot = slot_map(pos, req, N, I, page_size, rank, block_table)
    keep = slot >= 0
    out[slot[keep]] = kv_rows[keep]
    return out


def relayout_plan(start: int, length: int, N: int, I: int, rank: int,
                  src_table_row: np.ndarray, src_page_size: int,
                  dst_table_row: np.ndarray, dst_page_size: int):
    """Token relayout of one request from an unsharded prefill cache (DCP1) to
    rank ``rank``'s striped decode pool.

    Page "PCP/DCP" (obnotes), "PD + DCP: extracting this rank's tokens from
    full source pages": on the prefill side request position t sits at row t
    of the request's pages; the decode rank receives the positions it owns,
    chosen by the request's global position (never by physical slot), read at
    their source slots and stored compactly at its local rows.  SGLang DCP
    docs, "DCP x PD disaggregation": the plan carries the exact token count,
    so rows of a partly filled final page are never moved.

    Positions [start, start + length) are moved (start > 0: a chunk after a
    prefix).  Returns (positions, source slots, destination slots), in
    position order; a slot is -1 where a table has no page for the row.
    """
    mine = stripe_positions(start + length, N, I)[rank]
    rows = np.arange(len(mine), dtype=np.int64)          # local row = index in the rank's list
    keep = mine >= start
    positions, rows = mine[keep], rows[keep]
    src = page_slot(src_table_row, positions, src_page_size)
    dst = page_slot(dst_table_row, rows, dst_page_size)
    return positions, src, dst


def relayout(dst_pool: np.ndarray, src_pool: np.ndarray, src_slots: np.ndarray,
             dst_slots: np.ndarray) -> np.ndarray:
    """Apply a relayout plan: copy source row src_slots[i] to destination row
    dst_slots[i] (pools viewed as [pages * page_size, row_dim]); pairs with a
    missing slot are skipped.  Returns the new destination pool."""
    out = dst_pool.copy()
    ok = (np.asarray(src_slots) >= 0) & (np.asarray(dst_slots) >= 0)
    out[np.asarray(dst_slots)[ok]] = src_pool[np.asarray(src_slots)[ok]]
    return out


def sparse_plan(topk: np.ndarray, S: int, N: int, I: int, rank: int):
    """One rank's share of a global per-token selection of one request.

    topk [q_len, K] global positions (-1 = unused slot).  Page "DCP",
    conditions for merging: with a global top-k each rank attends only to the
    selected tokens it owns.  Walks the slots in (token, slot) order and keeps
    a position p of token t when 0 <= p <= S - q_len + t and the rank owns p.
    Returns (local rows, selecting-token bits 1 << t) of the kept entries."""
    topk = np.asarray(topk, dtype=np.int64)
    q_len = topk.shape[0]
    owner, row = owner_and_row_table(max(S, 1), N, I)
    rows, bits = [], []
    for t in range(q_len):
        for p in topk[t]:
            p = int(p)
            if 0 <= p <= S - q_len + t and owner[p] == rank:
                rows.append(int(row[p]))
                bits.append(1 << t)
    return np.asarray(rows, dtype=np.int64), np.asarray(bits, dtype=np.int64)
