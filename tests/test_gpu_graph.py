"""HIP graph capture: the library's calls allocate, clear and synchronise
nothing, so one decode step (every rank's stripe attention, chunk combines
included, then the merge) captures into one graph.  Every replay, with eager
work and synchronisations between replays, must give exactly the eager
step's results; the outputs are overwritten with NaN before each replay so a
replay that wrote nothing cannot pass."""

import dataclasses

import numpy as np
import pytest
import torch

from mla_context_kv_amd import dcp, workloads

import gpu_helpers as H

pytestmark = pytest.mark.gpu


def test_graph_replays_equal_the_eager_step():
    lens = np.array([5000, 64, 1, 2100, 333, 9000], dtype=np.int64)
    w = dataclasses.replace(workloads.WORKLOADS["tiny"], name="custom", B=len(lens), H=96, q_len=1, N=4,
                            page_size=64, S=int(lens.max()), lse_base="2", table="random", q_std=1.0, kv_std=0.5,
                            seed=21)
    print(f"graph: lens={list(lens)} N={w.N}", flush=True)
    s = H.make_setup(w, 1, lens=lens)
    dev = s.q.device
    N = s.lay.n_stripes
    o_parts = torch.empty((N, w.B, w.q_len, w.H, workloads.V_DIM), dtype=torch.float32, device=dev)
    lse_parts = torch.empty((N, w.B, w.q_len, w.H), dtype=torch.float32, device=dev)
    o = torch.empty((w.B, w.q_len, w.H, workloads.V_DIM), dtype=torch.float32, device=dev)
    lse = torch.empty((w.B, w.q_len, w.H), dtype=torch.float32, device=dev)
    need = max(dcp.dcp_stripe_attn_workspace(s.lay, r, s.q, s.sp.pools[r], s.sp.tables[r], lse_base=s.base_flag)
               for r in range(N))
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)

    def step():
        for r in range(N):
            dcp.dcp_stripe_attn(s.lay, r, s.q, s.sp.pools[r], s.sp.tables[r], s.sp.seq_len, workloads.SCALE,
                                s.base_flag, workspace=ws, o=o_parts[r], lse=lse_parts[r], status=s.status)
        dcp.dcp_lse_merge(o_parts, lse_parts, s.base_flag, o=o, lse=lse)

    step()
    torch.cuda.synchronize()
    assert int(s.status.item()) == 0
    ref = [t.clone() for t in (o_parts, lse_parts, o, lse)]

    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream(dev)
    cap.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.graph(g, stream=cap):
        step()
    torch.cuda.current_stream(dev).wait_stream(cap)
    torch.cuda.synchronize()

    junk = torch.randn(1 << 20, device=dev)
    for rep in range(4):
        for t in (o_parts, lse_parts, o, lse):
            t.fill_(float("nan"))
        junk.mul_(1.0001)                                   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(s.status.item()) == 0
        for got, want, name in zip((o_parts, lse_parts, o, lse), ref, ("o_r", "lse_r", "o", "lse")):
            assert torch.equal(got, want), f"replay {rep}: {name} differs from the eager step"
    # the eager step itself against the oracle, every request
    for b in range(w.B):
        H.check_request(s, ref[0], ref[1], ref[2], ref[3], b)
