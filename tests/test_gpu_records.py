"""GPU parity of the packed-record output of dcp_stripe_attn: per (row, head)
the bf16 output (rounded to nearest even) and the float32 lse, written in
head-owner order [N][parts][B*q_len][H/N][516] -- the all-to-all send buffer
of the head-return exchange (page "DCP", "merge: All-to-All"; page "MLA 的
DCP", section 5: (512 + 4) 16-bit slots per (row, head)).

Two checks: the records are exactly the float32 result rounded once (the
same bits dcp_pack_heads gives), and each owner's dcp_merge_heads over what it
receives agrees with the oracle's full attention and with the oracle's merge
of bf16-rounded stripe partials."""

import dataclasses

import numpy as np
import pytest
import torch

from mla_context_kv_amd import dcp, workloads
from oracle import attention as OA
from oracle import layout as OL

import gpu_helpers as H

pytestmark = pytest.mark.gpu

V = workloads.V_DIM

CASES = [
    # B, H, q_len, N, I, P, lens, base, splits, parts
    (3, 16, 1, 4, 1, 64, [300, 2000, 5], "e", 1, False),          # one chunk per request: the kernel writes
    (2, 32, 2, 4, 64, 64, [9000, 700], "2", 4, False),            # several chunks: the chunk combine writes
    (4, 96, 1, 8, 1, 64, [4000, 100, 9, 1], "2", 0, False),       # balanced plan, empty stripes
    (2, 16, 1, 2, 1, 64, [5000, 33], "e", 3, True),               # unmerged parts, some empty
    (2, 24, 3, 4, 2, 16, [90, 31], "e", 2, True),                 # drafts, page 16, interleave 2
]


def custom(B, H_, q_len, N, P, lens, base):
    w = dataclasses.replace(workloads.WORKLOADS["tiny"], name="custom", B=B, H=H_, q_len=q_len, N=N,
                            page_size=P, S=max(lens), lse_base=base, seed=11)
    return w, np.asarray(lens, dtype=np.int64)


def expected_records(o: torch.Tensor, lse: torch.Tensor, N: int) -> torch.Tensor:
    """float32 (o [k, B, q_len, H, V], lse [k, B, q_len, H]) -> int16 records
    [N, k, B*q_len, H/N, V + 4], bf16 by torch's round-to-nearest-even."""
    k, B, q_len, H_ = lse.shape
    ob = o.cpu().to(torch.bfloat16).view(torch.int16).reshape(k, B * q_len, N, H_ // N, V)
    lb = lse.cpu().contiguous().view(torch.int16).reshape(k, B * q_len, N, H_ // N, 2)
    pad = torch.zeros((k, B * q_len, N, H_ // N, 2), dtype=torch.int16)
    rec = torch.cat([ob, lb, pad], dim=-1)                        # [k, rows, N, Hl, V + 4]
    return rec.permute(2, 0, 1, 3, 4).contiguous()


@pytest.mark.parametrize("B,H_,q_len,N,I,P,lens,base,splits,parts", CASES)
def test_records_are_the_rounded_float32_result(B, H_, q_len, N, I, P, lens, base, splits, parts):
    w, lens = custom(B, H_, q_len, N, P, lens, base)
    print(f"records B={B} H={H_} q_len={q_len} N={N} I={I} lens={lens.tolist()} splits={splits} parts={parts}",
          flush=True)
    s = H.make_setup(w, I, lens=lens)
    for r in range(N):
        o, lse = dcp.dcp_stripe_attn(s.lay, r, s.q, s.sp.pools[r], s.sp.tables[r], s.sp.seq_len, workloads.SCALE,
                                     s.base_flag, num_splits=splits, status=s.status, partials=parts)
        rec, none = dcp.dcp_stripe_attn(s.lay, r, s.q, s.sp.pools[r], s.sp.tables[r], s.sp.seq_len,
                                        workloads.SCALE, s.base_flag, num_splits=splits, status=s.status,
                                        partials=parts, records=True)
        torch.cuda.synchronize()
        assert none is None and int(s.status.item()) == 0
        k = splits if parts else 1
        assert rec.shape == (N, k, B * q_len, H_ // N, V + 4) if parts else rec.shape == (N, B * q_len, H_ // N, V + 4)
        if not parts:
            o, lse = o.unsqueeze(0), lse.unsqueeze(0)
        want = expected_records(o, lse, N)
        got = rec.cpu().reshape(want.shape)
        bad = (got != want).nonzero()
        assert bad.numel() == 0, f"rank {r}: {bad.shape[0]} record slots differ, first at {bad[0].tolist()}"


@pytest.mark.parametrize("B,H_,q_len,N,I,P,lens,base,splits,parts", CASES)
def test_records_head_return_equals_full_attention(B, H_, q_len, N, I, P, lens, base, splits, parts):
    w, lens = custom(B, H_, q_len, N, P, lens, base)
    print(f"head return B={B} H={H_} q_len={q_len} N={N} I={I} lens={lens.tolist()} splits={splits} "
          f"parts={parts}", flush=True)
    s = H.make_setup(w, I, lens=lens)
    recs = [dcp.dcp_stripe_attn(s.lay, r, s.q, s.sp.pools[r], s.sp.tables[r], s.sp.seq_len, workloads.SCALE,
                                s.base_flag, num_splits=splits, status=s.status, partials=parts, records=True)[0]
            for r in range(N)]
    Hl = H_ // N
    k = splits if parts else 1
    outs = []
    for d in range(N):
        # what owner d receives: block d of every rank's send buffer (k parts each)
        recv = torch.stack([recs[r][d] for r in range(N)]).reshape(N * k, B * q_len, Hl, V + 4)
        outs.append(dcp.dcp_merge_heads(recv, s.base_flag))
    torch.cuda.synchronize()
    assert int(s.status.item()) == 0
    o = torch.cat([x[0] for x in outs], dim=1).view(B, q_len, H_, V).cpu().numpy()
    lse = torch.cat([x[1] for x in outs], dim=1).view(B, q_len, H_).cpu().numpy()
    for b in range(B):
        q64, kv64, S = H.request_inputs(s, b)
        ref_o, ref_l = OA.full_attention(q64, kv64, S, workloads.SCALE)
        H.assert_o_close(o[b], ref_o, f"record head return o, request {b}")
        H.assert_lse_close(lse[b], OA.to_base(ref_l, base), f"record head return lse, request {b}")
        if parts:
            continue
        # the oracle's reading of bf16 partials: stripe results rounded to bf16
        # (o) and float32 (lse), merged exactly
        lists = OL.stripe_positions(S, N, I)
        po, pl = zip(*[OA.stripe_attention(q64, kv64, S, lists[r], workloads.SCALE) for r in range(N)])
        mo, ml = OA.merge_bf16_parts(np.stack(po), np.stack(pl), "e")
        H.assert_o_close(o[b], mo, f"record head return vs bf16-part merge, request {b}")
        H.assert_lse_close(lse[b], OA.to_base(ml, base), f"record head return lse vs bf16-part merge, request {b}")


def test_multi_rank_records_are_the_rounded_float32_result():
    w, lens = custom(3, 32, 1, 4, 64, [7000, 64, 1500], "2")
    print("multi records", flush=True)
    s = H.make_setup(w, 1, lens=lens)
    N = s.lay.n_stripes
    # the same launch plan with float32 outputs (a per-rank call may chunk differently)
    mo, ml = dcp.dcp_stripe_attn_multi(s.lay, list(range(N)), s.q, s.sp.pools, s.sp.tables, s.sp.seq_len,
                                       workloads.SCALE, s.base_flag, status=s.status)
    rec_m, none = dcp.dcp_stripe_attn_multi(s.lay, list(range(N)), s.q, s.sp.pools, s.sp.tables, s.sp.seq_len,
                                            workloads.SCALE, s.base_flag, status=s.status, records=True)
    torch.cuda.synchronize()
    assert none is None and int(s.status.item()) == 0
    for r in range(N):
        want = expected_records(mo[r].unsqueeze(0), ml[r].unsqueeze(0), N)
        assert torch.equal(rec_m[r].cpu().reshape(want.shape), want), f"rank {r}"
    # one merge over all owners at once: rank r's records are part r of every
    # owner's rows, in owner order
    o, lse = dcp.dcp_merge_heads(rec_m.reshape(N, -1, V + 4), s.base_flag)
    torch.cuda.synchronize()
    o = o.view(N, w.B, w.H // N, V).permute(1, 0, 2, 3).reshape(w.B, 1, w.H, V).cpu().numpy()
    for b in range(w.B):
        q64, kv64, S = H.request_inputs(s, b)
        ref_o, _ = OA.full_attention(q64, kv64, S, workloads.SCALE)
        H.assert_o_close(o[b], ref_o, f"all-owner merge, request {b}")


def test_records_need_whole_head_slices():
    w, lens = custom(1, 12, 1, 8, 64, [100], "e")
    s = H.make_setup(w, 1, lens=lens)
    with pytest.raises(ValueError):
        dcp.dcp_stripe_attn(s.lay, 0, s.q, s.sp.pools[0], s.sp.tables[0], s.sp.seq_len, workloads.SCALE,
                            records=True)
