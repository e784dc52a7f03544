"""The allocation-free stripe attention (dcp_stripe_attn_noalloc): its fixed
per-GPU scratch buffer replaces the caller's workspace, and its results equal
dcp_stripe_attn's bit for bit -- on two calls in a row, the second with a
smaller input, so the second call runs over what the first left in the
buffer -- and the oracle's at the parity bar.  The size limit is checked on
the host (CPU test)."""

import ctypes

import numpy as np
import pytest
import torch

from mla_context_kv_amd import dcp, workloads

import gpu_helpers as H


def test_noalloc_rejects_shapes_beyond_its_buffer():
    L = dcp.lib()
    limit = int(L.dcp_stripe_attn_noalloc_max_bytes())
    assert limit == 64 << 20
    a = dcp.dcp_attn_args()
    a.layout = dcp.layout(8, 1, 64)
    a.rank, a.batch, a.q_len, a.n_heads, a.head_dim, a.v_dim = 0, 64, 1, 96, 576, 512
    a.num_pages, a.bt_cols, a.num_splits, a.scale = 1 << 14, 256, 16, 0.07
    need = ctypes.c_size_t(0)
    assert L.dcp_stripe_attn_workspace(ctypes.byref(a), ctypes.byref(need)) == 0
    assert need.value > limit                         # 16 chunks per request of K3's shape
    # refused before any HIP call (so also without a GPU), nothing enqueued
    assert L.dcp_stripe_attn_noalloc(ctypes.byref(a), None) == dcp.DCP_ESCRATCH
    assert "scratch" in dcp.strerror(dcp.DCP_ESCRATCH)


def _both(s, r, num_splits=0):
    """rank r's stripe through dcp_stripe_attn and dcp_stripe_attn_noalloc"""
    w = s.w
    dev = s.q.device
    shape = (w.B, w.q_len, w.H)
    o_ref = torch.empty(shape + (workloads.V_DIM,), dtype=torch.float32, device=dev)
    l_ref = torch.empty(shape, dtype=torch.float32, device=dev)
    o_na = torch.full_like(o_ref, float("nan"))
    l_na = torch.full_like(l_ref, float("nan"))
    dcp.dcp_stripe_attn(s.lay, r, s.q, s.sp.pools[r], s.sp.tables[r], s.sp.seq_len, workloads.SCALE,
                        s.base_flag, num_splits=num_splits, o=o_ref, lse=l_ref, status=s.status)
    dcp.dcp_stripe_attn_noalloc(s.lay, r, s.q, s.sp.pools[r], s.sp.tables[r], s.sp.seq_len, workloads.SCALE,
                                s.base_flag, num_splits=num_splits, o=o_na, lse=l_na, status=s.status)
    torch.cuda.synchronize()
    assert int(s.status.item()) == 0
    return o_ref, l_ref, o_na, l_na


@pytest.mark.gpu
def test_noalloc_equals_workspace_call_twice_in_a_row():
    big = H.make_setup(workloads.WORKLOADS["dsv3"])        # 33.6 MB of chunk partials
    print("noalloc: dsv3 rank 3, then tiny rank 1", flush=True)
    o_ref, l_ref, o_na, l_na = _both(big, 3)
    assert torch.equal(o_na, o_ref) and torch.equal(l_na, l_ref)
    del big
    small = H.make_setup(workloads.WORKLOADS["tiny"])      # smaller: the buffer holds the first call's data
    o_ref, l_ref, o_na, l_na = _both(small, 1, num_splits=4)
    assert torch.equal(o_na, o_ref) and torch.equal(l_na, l_ref)
    # and the oracle's stripe at the parity bar
    from oracle import attention as OA
    from oracle import layout as OL
    for b in range(small.w.B):
        q64, kv64, S = H.request_inputs(small, b)
        lists = OL.stripe_positions(S, small.lay.n_stripes, small.lay.interleave)
        ro, rl = OA.stripe_attention(q64, kv64, S, lists[1], workloads.SCALE)
        H.assert_o_close(o_na[b].cpu().numpy(), ro, f"noalloc o_r, request {b}")
        H.assert_lse_close(l_na[b].cpu().numpy(), OA.to_base(rl, small.w.lse_base), f"noalloc lse_r, request {b}")


@pytest.mark.gpu
def test_noalloc_single_chunk_needs_no_scratch():
    s = H.make_setup(workloads.WORKLOADS["tiny"])
    o_ref, l_ref, o_na, l_na = _both(s, 0, num_splits=1)
    assert torch.equal(o_na, o_ref) and torch.equal(l_na, l_ref)
