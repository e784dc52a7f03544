"""Host-side replay of the stripe-attention kernel's address arithmetic.

For every workgroup and every tile load of each full-size workload (pools
with no spare pages, exactly as the benchmark allocates them) this checks that
each 16-byte direct-to-LDS load reads either the zero row or a row of the
tile's own page inside the pool, and that the epilogue's stores and the split
combine stay inside their buffers.  It mirrors the constants and index math of
csrc/stripe_attn.hip; a planted copy of an earlier guard (slots past the tile
not excluded) must be caught.
"""

import math

import numpy as np
import pytest

from mla_context_kv_amd import stripes, workloads

import gpu_helpers as H

TILE, ROW_SLOTS, CHUNKS = 32, 73, 72
TILE_SLOTS = TILE * ROW_SLOTS


def shape(W):
    loads = -(-TILE_SLOTS // (64 * W))
    stages = 3 if W == 1 else 4
    return loads, stages


def plan(B, M, bt_cols, P, cus=256, num_splits=0):
    W = 1 if M <= 32 else 2 if M <= 64 else 3 if M <= 96 else 4
    mgroups = -(-M // (32 * W))
    tiles_max = -(-(bt_cols * P) // TILE)
    splits = num_splits or -(-cus // (B * mgroups))
    splits = max(1, min(splits, tiles_max))
    per = -(-tiles_max // splits)
    splits = -(-tiles_max // per)
    return W, mgroups, splits, per * TILE


def count_rows(x, N, I, r):
    x = np.asarray(x, dtype=np.int64)
    rnd = N * I
    rem = np.clip(x % rnd - r * I, 0, I)
    return np.where(x <= 0, 0, (x // rnd) * I + rem)


def slot_rows(W, guard_tile=True):
    """(tt, c, use-mask-independent-of-rows) for every slot one wave set issues per tile."""
    loads, _ = shape(W)
    s = np.arange(loads * 64 * W)
    tt, c = s // ROW_SLOTS, s % ROW_SLOTS
    base_ok = c < CHUNKS
    if guard_tile:
        base_ok &= s < TILE_SLOTS
    return tt, base_ok


def check_workload(w, I, guard_tile=True, num_splits=0):
    lens = workloads.seq_lens(w)
    N, P = w.N, w.page_size
    counts = H.oracle_counts(lens, N, I)
    tables, pool_pages = workloads.make_block_tables(w, stripes.pages_from_counts(counts, P), 0)
    M = w.q_len * w.H
    for r in range(N):
        tab = tables[r]
        B, cols = tab.shape
        W, mgroups, splits, split_rows = plan(B, M, cols, P, num_splits=num_splits)
        loads, stages = shape(W)
        tt, base_ok = slot_rows(W, guard_tile)
        max_vis = count_rows(lens, N, I, r)
        for b in range(B):
            for sp in range(splits):
                row_lo = sp * split_rows
                row_hi = min(row_lo + split_rows, int(max_vis[b]))
                ntiles = -(-(row_hi - row_lo) // TILE) if row_hi > row_lo else 0
                for it in range(ntiles + stages - 1):
                    if it >= ntiles:
                        continue                       # dead tiles load only the zero row
                    J = row_lo + it * TILE
                    rows_left = row_hi - J
                    if P % TILE == 0 and rows_left >= TILE and guard_tile:
                        # fast path: slot s takes chunk min(s - s//73, 2303) of the
                        # 36,864 contiguous bytes of the tile's 32 rows
                        loads, _ = shape(W)
                        s_ = np.arange(loads * 64 * W)
                        g = np.minimum(s_ - (s_ * 57457 >> 22), TILE * CHUNKS - 1)
                        assert ((s_ * 57457 >> 22) == s_ // 73).all()
                        assert g.min() >= 0 and g.max() < TILE * CHUNKS
                        pi = J // P
                        assert pi < cols and 0 <= tab[b, pi] < pool_pages
                        assert J % P + TILE <= P          # the tile's rows lie inside its page
                        continue
                    use = base_ok & (tt < rows_left)
                    if not use.any():
                        continue
                    if P % TILE == 0:
                        pi = J // P
                        pg = tab[b, pi] if pi < cols else -1
                        assert 0 <= pg < pool_pages, "the kernel would flag this page; tables here are valid"
                        rows = pg * P + (J % P) + tt[use]
                        # every row read lies in the tile's own page and inside the pool
                        assert rows.max() < pg * P + P, (w.name, r, b, sp, it)
                        assert rows.max() < pool_pages * P
                    else:
                        j = J + tt[use]
                        pi = j // P
                        assert (pi < cols).all()
                        pg = tab[b, pi]
                        assert (pg >= 0).all() and (pg < pool_pages).all()
        # epilogue: partial / final rows and the combine stay inside their buffers
        assert B * mgroups * 32 * W >= B * M
        ws_floats = splits * B * M * (512 + 1)
        assert (splits - 1) * B * M + (B - 1) * M + (M - 1) < splits * B * M <= ws_floats


@pytest.mark.parametrize("name,I", [("tiny", 1), ("dsv3", 1), ("k3", 1), ("ragged", 1), ("long", 1), ("long", 64)])
def test_dma_loads_stay_in_the_tile_page(name, I):
    check_workload(workloads.WORKLOADS[name], I)


def test_planted_missing_tile_guard_is_caught():
    """Without the slot < tile guard the last load instruction of a full tile
    reads rows 32-34 past the tile: past its page, and past the pool at the
    pool's last page (page-aligned path; the per-row path looks every row up)."""
    for name in ("dsv3", "k3"):
        with pytest.raises(AssertionError):
            check_workload(workloads.WORKLOADS[name], 1, guard_tile=False)


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
        W, mg, splits, _ = plan(B, q_len * H_, cols, P, num_splits=ns)
        want = 0 if splits == 1 else splits * B * q_len * H_ * 513 * 4 + B * mg * 4
        assert n.value == want
