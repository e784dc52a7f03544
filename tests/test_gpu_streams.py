"""Concurrent calls: the library keeps no state between calls outside the
caller's buffers, so per-rank stripe attentions issued on two streams at once,
each stream with its own workspace, give exactly the serial results.  A
ragged batch makes the launches uneven, so one rank's launch overlaps the
tail of the other stream's launch and its chunk combine."""

import dataclasses

import numpy as np
import pytest
import torch

from mla_context_kv_amd import dcp, workloads

import gpu_helpers as H

pytestmark = pytest.mark.gpu


def test_two_streams_equal_serial_calls_bitwise():
    lens = np.array([9000, 33, 1, 4100, 700, 12000, 7, 2500], dtype=np.int64)
    w = dataclasses.replace(workloads.WORKLOADS["tiny"], name="custom", B=len(lens), H=96, q_len=1, N=4,
                            page_size=64, S=int(lens.max()), lse_base="e", table="random", q_std=1.0, kv_std=0.5,
                            seed=11)
    print(f"two streams: lens={list(lens)} N={w.N}", flush=True)
    s = H.make_setup(w, 1, lens=lens)
    dev = s.q.device
    N = s.lay.n_stripes
    shape_o = (N, w.B, w.q_len, w.H, workloads.V_DIM)
    shape_l = (N, w.B, w.q_len, w.H)

    def call(r, o, lse, ws):
        dcp.dcp_stripe_attn(s.lay, r, s.q, s.sp.pools[r], s.sp.tables[r], s.sp.seq_len, workloads.SCALE,
                            s.base_flag, workspace=ws, o=o[r], lse=lse[r], status=s.status)

    need = max(dcp.dcp_stripe_attn_workspace(s.lay, r, s.q, s.sp.pools[r], s.sp.tables[r]) for r in range(N))
    ws = [torch.empty(max(need, 16), dtype=torch.uint8, device=dev) for _ in range(2)]

    o_ser = torch.full(shape_o, float("nan"), device=dev)
    l_ser = torch.full(shape_l, float("nan"), device=dev)
    for r in range(N):
        call(r, o_ser, l_ser, ws[0])
    torch.cuda.synchronize()
    assert int(s.status.item()) == 0

    side = torch.cuda.Stream(dev)                     # default priority
    main = torch.cuda.current_stream(dev)
    for rep in range(3):
        o_two = torch.full(shape_o, float("nan"), device=dev)
        l_two = torch.full(shape_l, float("nan"), device=dev)
        side.wait_stream(main)                        # the output buffers are filled first
        for r in range(N):
            if r % 2 == 0:
                call(r, o_two, l_two, ws[0])
            else:
                with torch.cuda.stream(side):
                    call(r, o_two, l_two, ws[1])
        main.wait_stream(side)
        torch.cuda.synchronize()
        assert int(s.status.item()) == 0
        assert torch.equal(o_two, o_ser), f"o differs on pass {rep}"
        assert torch.equal(l_two, l_ser), f"lse differs on pass {rep}"
    # and the serial results are the oracle's (every request, every stripe)
    o, lse = dcp.dcp_lse_merge(o_ser, l_ser, s.base_flag)
    for b in range(w.B):
        H.check_request(s, o_ser, l_ser, o, lse, b)
