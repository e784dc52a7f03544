"""GPU parity of the bf16 outputs of dcp_stripe_attn (o_bf16 = 1) and of
dcp_lse_merge_bf16, the merge of such parts.

Page "MLA 的 DCP", section 5, sizes the partial a rank hands to the merge as
(512 + 4) x 2 bytes per (row, head): the output in bf16 beside its LSE.  With
o_bf16 the stripe writes o_r in bf16 in the plain request layout and lse_r in
float32.  Three checks:
  * o_r is exactly the float32 result rounded once to nearest even (torch's
    rounding) and lse_r is the float32 lse, bit for bit -- for a request
    written by the kernel itself, by the chunk combine, as unmerged parts and
    from one launch of all ranks;
  * the merge of the bf16 parts agrees with the oracle's full attention and
    with the oracle's merge of bf16-rounded stripe partials (merge_bf16_parts);
  * the bf16 merge of zero-weight parts holding NaN ignores them, and 3 to 70
    parts (several groups of loads in flight, more parts than lanes) and
    value widths of 256 to 1024 merge like the oracle."""

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
                            page_size=P, S=max(lens), lse_base=base, seed=13)
    return w, np.asarray(lens, dtype=np.int64)


@pytest.mark.parametrize("B,H_,q_len,N,I,P,lens,base,splits,parts", CASES)
def test_bf16_outputs_are_the_rounded_float32_result(B, H_, q_len, N, I, P, lens, base, splits, parts):
    w, lens = custom(B, H_, q_len, N, P, lens, base)
    print(f"bf16 outputs B={B} H={H_} q_len={q_len} N={N} I={I} lens={lens.tolist()} splits={splits} "
          f"parts={parts}", flush=True)
    s = H.make_setup(w, I, lens=lens)
    for r in range(N):
        o, lse = dcp.dcp_stripe_attn(s.lay, r, s.q, s.sp.pools[r], s.sp.tables[r], s.sp.seq_len, workloads.SCALE,
                                     s.base_flag, num_splits=splits, status=s.status, partials=parts)
        o16, lse16 = dcp.dcp_stripe_attn(s.lay, r, s.q, s.sp.pools[r], s.sp.tables[r], s.sp.seq_len,
                                         workloads.SCALE, s.base_flag, num_splits=splits, status=s.status,
                                         partials=parts, o_bf16=True)
        torch.cuda.synchronize()
        assert int(s.status.item()) == 0
        assert o16.dtype == torch.bfloat16 and o16.shape == o.shape and lse16.dtype == torch.float32
        want = o.cpu().to(torch.bfloat16).view(torch.int16)
        got = o16.cpu().view(torch.int16)
        bad = (got != want).nonzero()
        assert bad.numel() == 0, f"rank {r}: {bad.shape[0]} bf16 values differ, first at {bad[0].tolist()}"
        assert torch.equal(lse16.cpu().view(torch.int32), lse.cpu().view(torch.int32)), f"rank {r}: lse differs"


@pytest.mark.parametrize("B,H_,q_len,N,I,P,lens,base,splits,parts", CASES)
def test_bf16_parts_merge_to_full_attention(B, H_, q_len, N, I, P, lens, base, splits, parts):
    w, lens = custom(B, H_, q_len, N, P, lens, base)
    print(f"bf16 merge B={B} H={H_} q_len={q_len} N={N} I={I} lens={lens.tolist()} splits={splits} "
          f"parts={parts}", flush=True)
    s = H.make_setup(w, I, lens=lens)
    outs = [dcp.dcp_stripe_attn(s.lay, r, s.q, s.sp.pools[r], s.sp.tables[r], s.sp.seq_len, workloads.SCALE,
                                s.base_flag, num_splits=splits, status=s.status, partials=parts, o_bf16=True)
            for r in range(N)]
    k = splits if parts else 1
    o_parts = torch.stack([x[0] for x in outs]).reshape(N * k, B, q_len, H_, V)
    l_parts = torch.stack([x[1] for x in outs]).reshape(N * k, B, q_len, H_)
    o, lse = dcp.dcp_lse_merge(o_parts, l_parts, s.base_flag)
    torch.cuda.synchronize()
    assert int(s.status.item()) == 0
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    for b in range(B):
        q64, kv64, S = H.request_inputs(s, b)
        ref_o, ref_l = OA.full_attention(q64, kv64, S, workloads.SCALE)
        H.assert_o_close(o[b], ref_o, f"bf16-part merge o, request {b}")
        H.assert_lse_close(lse[b], OA.to_base(ref_l, base), f"bf16-part merge lse, request {b}")
        if parts:
            continue
        # the oracle's reading of bf16 partials: each stripe's result rounded to
        # bf16 (o) and float32 (lse), merged exactly
        lists = OL.stripe_positions(S, N, I)
        po, pl = zip(*[OA.stripe_attention(q64, kv64, S, lists[r], workloads.SCALE) for r in range(N)])
        mo, ml = OA.merge_bf16_parts(np.stack(po), np.stack(pl), "e")
        H.assert_o_close(o[b], mo, f"bf16-part merge vs the oracle's bf16 merge, request {b}")
        H.assert_lse_close(lse[b], OA.to_base(ml, base), f"bf16-part merge lse vs the oracle's, request {b}")


def test_multi_rank_bf16_outputs_are_the_rounded_float32_result():
    w, lens = custom(3, 32, 1, 4, 64, [7000, 64, 1500], "2")
    print("multi bf16 outputs", flush=True)
    s = H.make_setup(w, 1, lens=lens)
    N = s.lay.n_stripes
    mo, ml = dcp.dcp_stripe_attn_multi(s.lay, list(range(N)), s.q, s.sp.pools, s.sp.tables, s.sp.seq_len,
                                       workloads.SCALE, s.base_flag, status=s.status)
    mo16, ml16 = dcp.dcp_stripe_attn_multi(s.lay, list(range(N)), s.q, s.sp.pools, s.sp.tables, s.sp.seq_len,
                                           workloads.SCALE, s.base_flag, status=s.status, o_bf16=True)
    torch.cuda.synchronize()
    assert int(s.status.item()) == 0 and mo16.dtype == torch.bfloat16
    assert torch.equal(mo16.cpu().view(torch.int16), mo.cpu().to(torch.bfloat16).view(torch.int16))
    assert torch.equal(ml16.cpu().view(torch.int32), ml.cpu().view(torch.int32))
    o, lse = dcp.dcp_lse_merge(mo16, ml16, s.base_flag)
    torch.cuda.synchronize()
    o = o.cpu().numpy()
    for b in range(w.B):
        q64, kv64, S = H.request_inputs(s, b)
        ref_o, _ = OA.full_attention(q64, kv64, S, workloads.SCALE)
        H.assert_o_close(o[b], ref_o, f"one-launch bf16-part merge, request {b}")


@pytest.mark.parametrize("n_parts,v_dim,base", [(3, 512, "e"), (9, 512, "2"), (20, 256, "e"), (70, 512, "2"),
                                                 (5, 1024, "e")])
def test_bf16_merge_against_the_oracle(n_parts, v_dim, base):
    # synthetic parts: bf16 values, float32 lse spread over a few units, some
    # parts empty (lse = -inf) with NaN values that must not reach the result,
    # and one row whose parts are all empty
    print(f"bf16 merge parts={n_parts} v_dim={v_dim} base={base}", flush=True)
    dev = H.device()
    g = torch.Generator().manual_seed(n_parts * 7 + v_dim)
    rows = 37
    o16 = torch.randn((n_parts, rows, v_dim), generator=g).to(torch.bfloat16)
    lse = (torch.randn((n_parts, rows), generator=g) * 3.0).float()
    empty = torch.rand((n_parts, rows), generator=g) < 0.3
    lse[empty] = -float("inf")
    lse[:, 5] = -float("inf")                                    # an all-empty row
    o16[empty] = float("nan")
    o, l = dcp.dcp_lse_merge(o16.to(dev), lse.to(dev), 1 if base == "2" else 0)
    torch.cuda.synchronize()
    o, l = o.cpu().numpy(), l.cpu().numpy()
    # the oracle's merge of the same parts (bf16 widened exactly to float64,
    # the lse in the same base); the empty parts' NaN values are left out
    x64 = o16.float().double().numpy()
    l64 = lse.double().numpy()
    for i in range(rows):
        keep = np.isfinite(l64[:, i])
        if not keep.any():
            assert np.all(o[i] == 0.0) and l[i] == -np.inf, f"all-empty row {i}"
            continue
        ref_o, ref_l = OA.lse_merge(x64[keep, i], l64[keep, i], base)
        assert np.all(np.isfinite(o[i]))
        H.assert_o_close(o[i], ref_o, f"bf16 merge row {i}")
        H.assert_lse_close(np.asarray(l[i]), np.asarray(ref_l), f"bf16 merge lse row {i}")


def test_bf16_outputs_do_not_combine_with_records():
    w, lens = custom(1, 16, 1, 4, 64, [100], "e")
    s = H.make_setup(w, 1, lens=lens)
    with pytest.raises(ValueError):
        dcp.dcp_stripe_attn(s.lay, 0, s.q, s.sp.pools[0], s.sp.tables[0], s.sp.seq_len, workloads.SCALE,
                            records=True, o_bf16=True)
