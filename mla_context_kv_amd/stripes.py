"""Set-up of the N per-rank paged latent pools on one GPU, through libdcp.

All N ranks' pools live in one allocation [N, pool_pages, P, 576] (rank r's
pool is pools[r]); the logical KV of every request is written into them with
dcp_kv_write, one call per rank, so each pool receives exactly the rows its
rank owns.  The per-rank page tables are inputs (see workloads.make_block_tables).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import dcp
from .workloads import ROW_DIM, bf16_nan_fill


@dataclass
class StripePools:
    layout: dcp.dcp_layout
    pools: torch.Tensor          # [N, pool_pages, P, 576] bf16
    tables: list                 # N int32 device tensors [B, cols]
    seq_len: torch.Tensor        # [B] int32 device (global lengths)

    @property
    def N(self) -> int:
        return self.layout.n_stripes


def positions_and_requests(lens: np.ndarray, device) -> tuple[torch.Tensor, torch.Tensor]:
    """Global position and request index of every token, in request order."""
    lens_t = torch.as_tensor(np.asarray(lens, dtype=np.int64), device=device)
    total = int(lens_t.sum().item())
    req = torch.repeat_interleave(torch.arange(len(lens), device=device, dtype=torch.int32), lens_t)
    starts = torch.cumsum(lens_t, 0) - lens_t
    pos = torch.arange(total, device=device, dtype=torch.int64) - torch.repeat_interleave(starts, lens_t)
    return pos, req


def build_pools(lay: dcp.dcp_layout, lens: np.ndarray, kv_all: torch.Tensor, tables: list,
                pool_pages: int, nan_fill: bool = False, status: torch.Tensor | None = None) -> StripePools:
    """Allocate the pools and write all requests' rows with one dcp_kv_write per rank."""
    device = kv_all.device
    N, P = lay.n_stripes, lay.page_size
    pools = torch.empty((N, pool_pages, P, ROW_DIM), dtype=torch.bfloat16, device=device)
    if nan_fill:
        bf16_nan_fill(pools)
    tabs = [torch.as_tensor(t, dtype=torch.int32).to(device).contiguous() for t in tables]
    pos, req = positions_and_requests(lens, device)
    for r in range(N):
        dcp.dcp_kv_write(lay, r, kv_all, pos, req, tabs[r], pools[r], status)
    seq = torch.as_tensor(np.asarray(lens, dtype=np.int32)).to(device)
    return StripePools(lay, pools, tabs, seq)


def pages_from_counts(counts: np.ndarray, page_size: int) -> np.ndarray:
    """Pages each (rank, request) needs for its local rows: counts [B, N] -> [N, B]."""
    counts = np.asarray(counts, dtype=np.int64)
    return (-(-counts // page_size)).T.copy()
