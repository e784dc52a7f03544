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
@pytest.mark.parametrize("N,rows,V", [(8, 6144, 512), (4, 37, 512), (1, 100, 512), (3, 5, 16), (16, 257, 512)])
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
