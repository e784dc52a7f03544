"""GPU parity of dcp_lse_merge against the float64 oracle merge, on partial
results the oracle itself produced (random rows, empty stripes, both bases)."""

import math

import numpy as np
import pytest
import torch

from mla_context_kv_amd import dcp
from oracle import attention as OA

import gpu_helpers as H

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("base", ["e", "2"])
# part counts cover both merge bodies: up to 8 parts with every load at once, above that the generic body
# (partial groups of 8, narrow rows, more parts than lanes)
@pytest.mark.parametrize("N,rows,V", [(8, 6144, 512), (4, 37, 512), (1, 100, 512), (3, 5, 16), (16, 257, 512),
                                      (9, 130, 512), (24, 64, 512), (32, 257, 512), (64, 64, 512), (20, 50, 16),
                                      (65, 40, 512), (100, 33, 512)])
def test_merge_matches_oracle(base, N, rows, V):
    dev = H.device()
    rng = np.random.default_rng(N * 1000 + rows)
    o_parts = rng.standard_normal((N, rows, V)).astype(np.float32)
    lse_parts = (rng.standard_normal((N, rows)) * 6).astype(np.float32)
    empty = rng.random((N, rows)) < 0.2
    lse_parts[empty] = -np.inf
    o_parts[empty] = np.nan                       # never read
    lse_parts[:, :2] = -np.inf                    # rows with every stripe empty
    flag = 1 if base == "2" else 0
    o, lse = dcp.dcp_lse_merge(torch.from_numpy(o_parts).to(dev), torch.from_numpy(lse_parts).to(dev), flag)
    torch.cuda.synchronize()
    ref_o, ref_l = OA.lse_merge(np.where(empty[..., None], 0.0, o_parts.astype(np.float64)),
                                lse_parts.astype(np.float64), base)
    got_o, got_l = o.cpu().numpy(), lse.cpu().numpy()
    H.assert_lse_close(got_l, ref_l, "merge lse")
    assert np.isfinite(got_o).all()
    assert np.abs(got_o - ref_o).max() <= 1e-5 * max(1.0, np.abs(ref_o).max())
    assert (got_o[:2] == 0).all() and np.isneginf(got_l[:2]).all()


def test_merge_of_one_part_is_identity():
    dev = H.device()
    o = torch.randn(1, 50, 512, device=dev)
    l = torch.randn(1, 50, device=dev) * 3
    mo, ml = dcp.dcp_lse_merge(o, l, 0)
    torch.cuda.synchronize()
    assert torch.allclose(mo, o[0], rtol=1e-6, atol=1e-6) and torch.allclose(ml, l[0], rtol=1e-6, atol=1e-6)


def test_merge_large_lse_no_overflow():
    dev = H.device()
    o = torch.tensor([[[1.0] * 4], [[3.0] * 4]], device=dev)
    l = torch.tensor([[1000.0], [1000.0 + math.log(3)]], device=dev)
    mo, ml = dcp.dcp_lse_merge(o, l, 0)
    torch.cuda.synchronize()
    # fp32 holds lse near 1000 to ~6e-5, which bounds the weight accuracy
    assert torch.allclose(mo, torch.full_like(mo, 2.5), rtol=1e-4) and abs(ml.item() - (1000 + math.log(4))) < 1e-3


# ---- head-return exchange: pack by head owner, merge at the owner ------------

@pytest.mark.parametrize("N,rows,H_,V", [(8, 64, 96, 512), (4, 7, 16, 512), (2, 33, 6, 16), (1, 5, 4, 512)])
def test_pack_heads_bit_exact(N, rows, H_, V):
    dev = H.device()
    rng = np.random.default_rng(N * 100 + rows)
    o = (rng.standard_normal((rows, H_, V)) * np.float32(10.0) ** rng.integers(-3, 3, (rows, H_, 1))).astype(np.float32)
    o[0, 0, :4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -0.0, 1e-40]            # ties and a subnormal
    lse = (rng.standard_normal((rows, H_)) * 20).astype(np.float32)
    lse[1 % rows, 0] = -np.inf
    send = dcp.dcp_pack_heads(torch.from_numpy(o).to(dev), torch.from_numpy(lse).to(dev), N)
    torch.cuda.synchronize()
    want = OA.pack_heads(o, lse, N)
    assert np.array_equal(send.cpu().numpy().view(np.uint16), want)


@pytest.mark.parametrize("base", ["e", "2"])
@pytest.mark.parametrize("N,rows,V", [(8, 768, 512), (4, 37, 512), (3, 5, 16), (16, 100, 512), (32, 40, 512),
                                      (12, 9, 16), (72, 6, 512)])
def test_merge_heads_matches_oracle(base, N, rows, V):
    dev = H.device()
    rng = np.random.default_rng(N + rows)
    o = rng.standard_normal((N, rows, 1, V)).astype(np.float32)
    lse = (rng.standard_normal((N, rows, 1)) * 6).astype(np.float32)
    lse[rng.random((N, rows, 1)) < 0.2] = -np.inf
    lse[:, :2] = -np.inf                                                    # rows with every part empty
    recv = np.stack([OA.pack_heads(o[r], lse[r], 1)[0] for r in range(N)])  # [N, rows, 1, V + 4]
    flag = 1 if base == "2" else 0
    got_o, got_l = dcp.dcp_merge_heads(torch.from_numpy(recv.view(np.int16)).to(dev), flag)
    torch.cuda.synchronize()
    ref_o, ref_l = OA.unpack_merge(recv, base)
    got_o, got_l = got_o.cpu().numpy(), got_l.cpu().numpy()
    H.assert_lse_close(got_l, ref_l, "merge_heads lse")
    assert np.abs(got_o - ref_o).max() <= 1e-5 * max(1.0, np.abs(ref_o).max())
    assert (got_o[:2] == 0).all() and np.isneginf(got_l[:2]).all()


def test_head_return_step_equals_full_attention():
    # stripe attention on every rank -> pack by head owner -> all-to-all (on one
    # GPU: block d of rank r's buffer becomes block r of rank d's) -> merge at
    # the owner; the owners' heads together are the full attention
    from mla_context_kv_amd import workloads
    w = workloads.WORKLOADS["tiny"]
    s = H.make_setup(w)
    o_parts, lse_parts, _, _ = H.run_step(s)
    N = s.lay.n_stripes
    sends = [dcp.dcp_pack_heads(o_parts[r], lse_parts[r], N) for r in range(N)]
    Hl = w.H // N
    outs = []
    for d in range(N):
        recv = torch.stack([sends[r][d] for r in range(N)])                # [N, B*q_len, Hl, V + 4]
        outs.append(dcp.dcp_merge_heads(recv, s.base_flag))
    torch.cuda.synchronize()
    o = torch.cat([x[0] for x in outs], dim=1).view(w.B, w.q_len, w.H, -1)
    lse = torch.cat([x[1] for x in outs], dim=1).view(w.B, w.q_len, w.H)
    for b in range(w.B):
        q64, kv64, S = H.request_inputs(s, b)
        ref_o, ref_l = OA.full_attention(q64, kv64, S, workloads.SCALE)
        H.assert_o_close(o[b].cpu().numpy(), ref_o, f"head-return o, request {b}")
        H.assert_lse_close(lse[b].cpu().numpy(), OA.to_base(ref_l, w.lse_base), f"head-return lse, request {b}")
