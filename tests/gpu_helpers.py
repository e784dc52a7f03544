"""Shared set-up for the GPU parity tests.

Inputs come from the seeded generators (mla_context_kv_amd.workloads); the
page tables are sized from the ORACLE's token counts, so no oracle input ever
comes from the GPU library.  Pools are pre-filled with bfloat16 NaN: any read
of a row that was never written (stale, unowned, past the end) shows up as NaN.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch

from mla_context_kv_amd import dcp, stripes, workloads
from oracle import attention as OA
from oracle import layout as OL

O_ATOL = 4e-3
O_RTOL = 1e-2
LSE_ATOL = 2e-3


def device():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU test run without a visible GPU")
    return torch.device("cuda:0")


def oracle_counts(lens, N, I) -> np.ndarray:
    """count_r(S_b) for every request (rows) and rank (cols), by the oracle's simulation."""
    cache = {}
    out = np.zeros((len(lens), N), dtype=np.int64)
    for b, s in enumerate(lens):
        s = int(s)
        if s not in cache:
            cache[s] = OL.local_counts(s, N, I)
        out[b] = cache[s]
    return out


@dataclass
class Setup:
    w: workloads.Workload
    lay: dcp.dcp_layout
    lens: np.ndarray
    q: torch.Tensor
    kv: torch.Tensor            # logical rows of all requests, request order
    offsets: np.ndarray
    tables: list
    pool_pages: int
    sp: stripes.StripePools
    status: torch.Tensor

    @property
    def base_flag(self) -> int:
        return 1 if self.w.lse_base == "2" else 0


def make_setup(w: workloads.Workload, interleave: int = 1, lens=None, nan_fill: bool = True,
               spare_pages: int = 0) -> Setup:
    dev = device()
    lens = workloads.seq_lens(w) if lens is None else np.asarray(lens, dtype=np.int64)
    N, P = w.N, w.page_size
    lay = dcp.layout(N, interleave, P)
    counts = oracle_counts(lens, N, interleave)
    tables, pool_pages = workloads.make_block_tables(w, stripes.pages_from_counts(counts, P), spare_pages)
    q = workloads.make_q(w, dev)
    kv = workloads.make_all_kv(w, lens, dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    sp = stripes.build_pools(lay, lens, kv, tables, pool_pages, nan_fill=nan_fill, status=status)
    offsets = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    return Setup(w, lay, lens, q, kv, offsets, tables, pool_pages, sp, status)


def run_step(s: Setup, num_splits: int = 0, window: int = 0, softcap: float = 0.0, sinks=None,
             sink_rank: int = 0, slopes=None):
    """All N stripe attentions + merge, as one decode step (sinks, fp64 [H],
    go to rank sink_rank only; position-bias slopes [H] to every rank)."""
    w = s.w
    dev = s.q.device
    N = s.lay.n_stripes
    o_parts = torch.empty((N, w.B, w.q_len, w.H, workloads.V_DIM), dtype=torch.float32, device=dev)
    lse_parts = torch.empty((N, w.B, w.q_len, w.H), dtype=torch.float32, device=dev)
    sk = None if sinks is None else torch.tensor(np.asarray(sinks), dtype=torch.float32, device=dev)
    sl = None if slopes is None else torch.tensor(np.asarray(slopes), dtype=torch.float32, device=dev)
    for r in range(N):
        dcp.dcp_stripe_attn(s.lay, r, s.q, s.sp.pools[r], s.sp.tables[r], s.sp.seq_len, workloads.SCALE,
                            s.base_flag, num_splits=num_splits, o=o_parts[r], lse=lse_parts[r], status=s.status,
                            window=window, softcap=softcap, sinks=sk if r == sink_rank else None,
                            bias_slopes=sl)
    o, lse = dcp.dcp_lse_merge(o_parts, lse_parts, s.base_flag)
    torch.cuda.synchronize()
    return o_parts, lse_parts, o, lse


def request_inputs(s: Setup, b: int, heads=None):
    """float64 host copies of request b's queries (optionally a head subset) and latent rows."""
    S = int(s.lens[b])
    q = s.q[b]
    if heads is not None:
        q = q[:, heads]
    q64 = q.double().cpu().numpy()
    kv64 = s.kv[int(s.offsets[b]):int(s.offsets[b]) + S].double().cpu().numpy()
    return q64, kv64, S


def assert_o_close(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    excess = np.abs(got - ref) - (O_ATOL + O_RTOL * np.abs(ref))
    i = int(np.argmax(excess))
    assert excess.flat[i] <= 0, (f"{what}: |o - ref| = {abs(got.flat[i] - ref.flat[i]):.3e} at flat {i} "
                                  f"(ref {ref.flat[i]:.4e}) exceeds {O_ATOL} + {O_RTOL}|ref|")


def assert_lse_close(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape
    empty = np.isneginf(ref)
    assert (np.isneginf(got) == empty).all(), f"{what}: empty-stripe lse mismatch"
    if (~empty).any():
        d = np.abs(got[~empty] - ref[~empty])
        assert d.max() <= LSE_ATOL, f"{what}: |lse - ref| = {d.max():.3e} > {LSE_ATOL}"


def check_request(s: Setup, o_parts, lse_parts, o, lse, b: int, heads=None, chunk=None, window=0, softcap=0.0,
                  sinks=None, sink_rank=0, slopes=None):
    """Compare request b's merged output and every stripe's partial with the oracle."""
    q64, kv64, S = request_inputs(s, b, heads)
    hsel = slice(None) if heads is None else heads
    sinks = None if sinks is None else np.asarray(sinks, dtype=np.float32).astype(np.float64)
    if sinks is not None and heads is not None:
        sinks = sinks[heads]
    if slopes is not None:
        slopes = np.asarray(slopes, dtype=np.float32).astype(np.float64)
        if heads is not None:
            slopes = slopes[heads]
    var = dict(window=window, softcap=softcap, slopes=slopes)
    ref_o, ref_l = OA.full_attention(q64, kv64, S, workloads.SCALE, chunk=chunk, sinks=sinks, **var)
    assert_o_close(o[b][:, hsel].cpu().numpy(), ref_o, f"merged o, request {b}")
    assert_lse_close(lse[b][:, hsel].cpu().numpy(), OA.to_base(ref_l, s.w.lse_base), f"merged lse, request {b}")
    lists = OL.stripe_positions(S, s.lay.n_stripes, s.lay.interleave)
    for r in range(s.lay.n_stripes):
        ro, rl = OA.stripe_attention(q64, kv64, S, lists[r], workloads.SCALE, chunk=chunk,
                                     sinks=sinks if r == sink_rank else None, **var)
        got_o = o_parts[r][b][:, hsel].cpu().numpy()
        got_l = lse_parts[r][b][:, hsel].cpu().numpy()
        assert_lse_close(got_l, OA.to_base(rl, s.w.lse_base), f"lse_r, request {b}, stripe {r}")
        assert_o_close(got_o, ro, f"o_r, request {b}, stripe {r}")
        empty = np.isneginf(rl)
        assert (got_o[empty] == 0).all(), "empty stripe must give o_r = 0"
