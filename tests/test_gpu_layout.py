"""GPU parity of the integer path: slot map, interval counts and the
owner-filtered paged KV write, bit-exact against the oracle's simulation."""

import numpy as np
import pytest
import torch

from mla_context_kv_amd import dcp, stripes, workloads
from oracle import layout as OL

import gpu_helpers as H

pytestmark = pytest.mark.gpu

CASES = [("tiny", 1), ("dsv3", 1), ("k3", 1), ("ragged", 1), ("long", 1), ("long", 64),
         ("dsv3", 128), ("ragged", 256)]                 # I = 2 and 4 pages of 64


def _tokens(lens):
    pos = np.concatenate([np.arange(int(s), dtype=np.int64) for s in lens])
    req = np.concatenate([np.full(int(s), b, dtype=np.int32) for b, s in enumerate(lens)])
    return pos, req


@pytest.mark.parametrize("name,I", CASES)
def test_slot_map_bit_exact_full_size(name, I):
    w = workloads.WORKLOADS[name]
    dev = H.device()
    lens = workloads.seq_lens(w)
    N, P = w.N, w.page_size
    print(f"slot map: {name} I={I} tokens={int(lens.sum())}", flush=True)
    counts = H.oracle_counts(lens, N, I)
    tables, _ = workloads.make_block_tables(w, stripes.pages_from_counts(counts, P))
    pos, req = _tokens(lens)
    pos_d = torch.from_numpy(pos).to(dev)
    req_d = torch.from_numpy(req).to(dev)
    lay = dcp.layout(N, I, P)
    own_ref, row_ref, _ = OL.slot_map(pos, req, N, I, P, -1, None)
    for r in range(N):
        status = torch.zeros(1, dtype=torch.int32, device=dev)
        bt = torch.from_numpy(tables[r]).to(dev)
        owner, row, slot = dcp.dcp_slot_map(lay, r, pos_d, req_d, bt, status)
        torch.cuda.synchronize()
        _, _, slot_ref = OL.slot_map(pos, req, N, I, P, r, tables[r])
        assert (owner.cpu().numpy() == own_ref).all()
        assert (row.cpu().numpy() == row_ref).all()
        assert (slot.cpu().numpy() == slot_ref).all()
        assert int(status.item()) == 0


def test_slot_map_large_positions_and_errors():
    dev = H.device()
    rng = np.random.default_rng(7)
    pos = rng.integers(0, 1 << 40, size=3000).astype(np.int64)
    for N, I in [(8, 1), (8, 64), (5, 2), (1, 1)]:
        lay = dcp.layout(N, I, 64)
        owner, row, slot = dcp.dcp_slot_map(lay, -1, torch.from_numpy(pos).to(dev))
        torch.cuda.synchronize()
        ref = np.array([OL.owner_row_walk(int(p), N, I) for p in pos])
        assert (owner.cpu().numpy() == ref[:, 0]).all() and (row.cpu().numpy() == ref[:, 1]).all()
        assert (slot.cpu().numpy() == -1).all()
    # an owned row whose page is missing from the table, and a negative position, raise DCP_ERANGE
    lay = dcp.layout(8, 1, 2)
    table = torch.tensor([[7, -1]], dtype=torch.int32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    p = torch.tensor([0, 8, 16, 8 * 10**6], dtype=torch.int64, device=dev)
    _, _, slot = dcp.dcp_slot_map(lay, 0, p, torch.zeros(4, dtype=torch.int32, device=dev), table, status)
    torch.cuda.synchronize()
    assert slot.cpu().tolist() == [14, 15, -1, -1] and int(status.item()) == dcp.DCP_ERANGE
    status.zero_()
    owner, row, slot = dcp.dcp_slot_map(lay, 0, torch.tensor([-5], dtype=torch.int64, device=dev), None, None, status)
    torch.cuda.synchronize()
    assert owner.item() == -1 and row.item() == -1 and int(status.item()) == dcp.DCP_ERANGE


@pytest.mark.parametrize("N,I", [(8, 1), (8, 64), (4, 1), (3, 16), (1, 1), (8, 128)])
def test_local_count_bit_exact(N, I):
    dev = H.device()
    rng = np.random.default_rng(N * 100 + I)
    start = np.concatenate([[0, 1000, 0, 5, 513], rng.integers(0, 70000, size=200)]).astype(np.int64)
    length = np.concatenate([[131072, 333, 0, 1, 64], rng.integers(0, 70000, size=200)]).astype(np.int64)
    got = dcp.dcp_local_count(dcp.layout(N, I, 64 if 64 % I == 0 else I), torch.from_numpy(length).to(dev),
                              torch.from_numpy(start).to(dev)).cpu().numpy()
    for i in range(len(start)):
        assert (got[i] == OL.interval_counts(int(start[i]), int(length[i]), N, I)).all(), (start[i], length[i])
    if (N, I) == (8, 1):
        assert got[1].tolist() == [42, 42, 42, 42, 42, 41, 41, 41]
    if (N, I) == (8, 64):
        assert got[1].tolist() == [64, 64, 64, 64, 53, 0, 0, 24]


def _rows_written(pool):
    """Rows of a pool that are no longer the NaN fill."""
    return ~(pool.view(torch.int16) == 0x7FC0).all(dim=-1)


@pytest.mark.parametrize("name,I", CASES)
def test_kv_write_places_every_owned_row(name, I):
    w = workloads.WORKLOADS[name]
    print(f"kv write: {name} I={I}", flush=True)
    s = H.make_setup(w, I)
    dev = s.q.device
    assert int(s.status.item()) == 0
    pos, req = _tokens(s.lens)
    own_ref, _, _ = OL.slot_map(pos, req, w.N, I, w.page_size, -1, None)
    src_row = np.arange(len(pos), dtype=np.int64)          # row index into s.kv
    for r in range(w.N):
        _, _, slot = OL.slot_map(pos, req, w.N, I, w.page_size, r, s.tables[r])
        mine = slot >= 0
        assert mine.sum() == (own_ref == r).sum()
        flat = s.sp.pools[r].view(-1, workloads.ROW_DIM)
        got = flat[torch.from_numpy(slot[mine]).to(dev)]
        want = s.kv[torch.from_numpy(src_row[mine]).to(dev)]
        assert torch.equal(got.view(torch.int16), want.view(torch.int16))
        written = _rows_written(flat)
        assert int(written.sum().item()) == int(mine.sum())
    del s
    torch.cuda.empty_cache()


def test_chunked_write_equals_one_shot_and_counts():
    """Ragged batch: [0,1000), [1000,1333), [1333,S) in three calls."""
    w = workloads.WORKLOADS["ragged"]
    dev = H.device()
    lens = workloads.seq_lens(w)
    lay = dcp.layout(w.N, 1, w.page_size)
    counts = H.oracle_counts(lens, w.N, 1)
    tables, pool_pages = workloads.make_block_tables(w, stripes.pages_from_counts(counts, w.page_size))
    kv = workloads.make_all_kv(w, lens, dev)
    one = stripes.build_pools(lay, lens, kv, tables, pool_pages, nan_fill=True)
    pos, req = stripes.positions_and_requests(lens, dev)
    pools = torch.empty_like(one.pools)
    workloads.bf16_nan_fill(pools)
    mid_only = torch.empty_like(one.pools)
    workloads.bf16_nan_fill(mid_only)
    for lo, hi in [(0, 1000), (1000, 1333), (1333, 1 << 30)]:
        sel = (pos >= lo) & (pos < hi)
        for r in range(w.N):
            dcp.dcp_kv_write(lay, r, kv[sel].contiguous(), pos[sel].contiguous(), req[sel].contiguous(),
                             one.tables[r], pools[r])
            if lo == 1000:
                dcp.dcp_kv_write(lay, r, kv[sel].contiguous(), pos[sel].contiguous(), req[sel].contiguous(),
                                 one.tables[r], mid_only[r])
    torch.cuda.synchronize()
    assert torch.equal(pools.view(torch.int16), one.pools.view(torch.int16))
    assert int((lens >= 1333).sum()) > 0
    per_rank = np.array([int(_rows_written(mid_only[r].view(-1, workloads.ROW_DIM)).sum().item()) for r in range(w.N)])
    # every request contributes its share of [1000, min(S_b, 1333)); a full chunk is [42]*5 + [41]*3
    want = sum(OL.interval_counts(1000, max(0, min(int(S), 1333) - 1000), w.N, 1) for S in lens)
    assert (per_rank == want).all()


def test_kv_write_out_of_range_page_is_skipped_and_flagged():
    dev = H.device()
    lay = dcp.layout(2, 1, 4)
    pool = torch.zeros((3, 4, 8), dtype=torch.bfloat16, device=dev)
    table = torch.tensor([[0, 5, 1]], dtype=torch.int32, device=dev)     # page 5 does not exist
    kv = torch.ones((24, 8), dtype=torch.bfloat16, device=dev)
    pos = torch.arange(24, dtype=torch.int64, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    dcp.dcp_kv_write(lay, 0, kv, pos, None, table, pool, status)
    torch.cuda.synchronize()
    assert int(status.item()) == dcp.DCP_ERANGE
    # rank 0 owns positions 0,2,..,22 -> rows 0..11: pages 0, 5 (skipped), 1
    assert pool[0].float().sum().item() == 32 and pool[1].float().sum().item() == 32
    assert pool[2].float().sum().item() == 0


# ---- prefill (DCP1) -> decode token relayout ---------------------------------

NAN16 = 0x7FC0      # bfloat16 quiet NaN: rows never written keep it


def _relayout_case(N, I, P, Ps, lens, seed):
    rng = np.random.default_rng(seed)
    B, D = len(lens), workloads.ROW_DIM
    src_need = [-(-int(S) // Ps) for S in lens]
    src_pages = sum(src_need) + 3
    perm = rng.permutation(src_pages)
    src_bt = np.full((B, max(src_need)), -1, dtype=np.int32)
    k = 0
    for b, n in enumerate(src_need):
        src_bt[b, :n] = perm[k:k + n]
        k += n
    g = torch.Generator().manual_seed(seed)
    src = (torch.randn((src_pages, Ps, D), generator=g) * 0.5).to(torch.bfloat16)
    return rng, src_bt, src


@pytest.mark.parametrize("N,I,P,Ps", [(8, 1, 64, 64), (4, 2, 16, 16), (8, 64, 64, 64), (3, 128, 64, 64),
                                      (8, 1, 64, 16)])
def test_relayout_bit_exact_chunked(N, I, P, Ps):
    dev = H.device()
    lens = [1, 700, 1333, 64]
    B, D = len(lens), workloads.ROW_DIM
    print(f"relayout N={N} I={I} P={P} Ps={Ps} lens={lens}", flush=True)
    rng, src_bt, src = _relayout_case(N, I, P, Ps, lens, N * 1000 + I + P)
    src_d = src.to(dev)
    src_bt_d = torch.from_numpy(src_bt).to(dev)
    src16 = src.view(torch.int16).reshape(-1, D).numpy()
    lay = dcp.layout(N, I, P)
    for r in range(N):
        counts = [int(OL.local_counts(int(S), N, I)[r]) for S in lens]
        need = [max(1, -(-c // P)) for c in counts]
        pages = sum(need) + 2
        perm = rng.permutation(pages)
        bt = np.full((B, max(need)), -1, dtype=np.int32)
        k = 0
        for b, n in enumerate(need):
            bt[b, :n] = perm[k:k + n]
            k += n
        pool = torch.full((pages, P, D), NAN16, dtype=torch.int16).view(torch.bfloat16).to(dev)
        want = np.full((pages * P, D), NAN16, dtype=np.int16)
        status = torch.zeros(1, dtype=torch.int32, device=dev)
        # every request moved in two chunks: a prefix and the rest (global positions)
        cut = [int(S) // 3 for S in lens]
        for starts, lengths in [([0] * B, cut), (cut, [int(S) - c for S, c in zip(lens, cut)])]:
            st = torch.tensor(starts, dtype=torch.int64, device=dev)
            ln = torch.tensor(lengths, dtype=torch.int64, device=dev)
            dcp.dcp_relayout(lay, r, src_d, src_bt_d, st, ln, torch.from_numpy(bt).to(dev), pool, status=status)
            for b in range(B):
                _, s_sl, d_sl = OL.relayout_plan(starts[b], lengths[b], N, I, r, src_bt[b], Ps, bt[b], P)
                want = OL.relayout(want, src16, s_sl, d_sl)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        got = pool.view(torch.int16).reshape(-1, D).cpu().numpy()
        assert np.array_equal(got, want), f"rank {r}"


def test_relayout_missing_page_is_skipped_and_flagged():
    dev = H.device()
    N, I, P = 4, 1, 16
    lens = [200]
    rng, src_bt, src = _relayout_case(N, I, P, P, lens, 5)
    src_bt[0, 3] = -1                                        # positions 48..63 have no source page
    D = workloads.ROW_DIM
    pool = torch.full((8, P, D), NAN16, dtype=torch.int16).view(torch.bfloat16).to(dev)
    bt = np.arange(4, dtype=np.int32)[None, :]
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    dcp.dcp_relayout(dcp.layout(N, I, P), 1, src.to(dev), torch.from_numpy(src_bt).to(dev),
                     torch.zeros(1, dtype=torch.int64, device=dev), torch.tensor([200], device=dev),
                     torch.from_numpy(bt).to(dev), pool, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == dcp.DCP_ERANGE
    pos, s_sl, d_sl = OL.relayout_plan(0, 200, N, I, 1, src_bt[0], P, bt[0], P)
    want = OL.relayout(np.full((8 * P, D), NAN16, dtype=np.int16), src.view(torch.int16).reshape(-1, D).numpy(),
                       s_sl, d_sl)
    assert np.array_equal(pool.view(torch.int16).reshape(-1, D).cpu().numpy(), want)
    assert (s_sl < 0).sum() == 4                             # rank 1 owns 49, 53, 57, 61 of that page


@pytest.mark.gpu
def test_measurement_probes_run():
    # the streaming-read and MFMA probes behind the measured peaks: one small
    # launch each, counts as documented, every sink word written
    import torch
    from mla_context_kv_amd import probe as PR
    dev = torch.device("cuda:0")
    src = torch.arange(41 * 36864 // 4, dtype=torch.int32, device=dev)
    for mode in ("lds1", "lds4", "reg"):
        grid = 4
        sink = PR.make_sink(mode, grid, dev)
        sink.fill_(-1)
        got = PR.stream(src, 40 * 36864 + 100, mode, grid, sink, torch.cuda.current_stream(dev).cuda_stream)
        torch.cuda.synchronize()
        assert got == 40 * 36864
        assert not bool((sink == -1).all())
    sink = PR.make_mfma_sink(2, dev)
    flops = PR.mfma(2, 3, sink, torch.cuda.current_stream(dev).cuda_stream)
    torch.cuda.synchronize()
    assert flops == 2 * 8 * 4 * 4 * 32 * 32 * 16 * 2          # 3 rounds run as 4 (pairs)
    assert bool(torch.isfinite(sink).all())
