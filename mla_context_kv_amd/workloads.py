"""Seeded synthetic inputs for the five decode workloads.

This module only draws random numbers and permutations; it holds none of the
striping, attention or merge arithmetic, so both the GPU library's callers and
the CPU oracle's callers can use it without sharing any of the method.

Recipe (the same on every device, seed 0 unless stated):

* Context lengths: fixed S, or for the ragged batch S_b = clamp(round(exp(u)),
  1, 65536) with u ~ U(0, ln 65536) from ``numpy.random.default_rng([seed, 11])``,
  then S_0..S_6 overwritten with 1..7 so that some stripes are empty.
* Queries q [B, q_len, H, 576]: float32 normal(0, q_std) from a
  ``torch.Generator`` on the target device seeded ``1000003*seed``, rounded to
  bfloat16 (round to nearest even).
* Latent rows of request b [S_b, 576]: float32 normal(0, kv_std) from a
  generator seeded ``1000003*seed + b + 1``, rounded to bfloat16; one
  generator per request so a single request can be regenerated alone.
* Page tables: for rank r a permutation of that rank's pool pages from
  ``numpy.random.default_rng([seed, 23, r])`` handed out in (request, page)
  order ("random"), or request b owning pages b*cols .. b*cols+cols-1
  ("identity"); unused entries are -1.  How many pages each (rank, request)
  needs is an input: the caller derives it from the token counts.

"kv ~ N(0, 0.5)" is read as standard deviation 0.5.  Values drawn on a GPU and
on the CPU differ (different generators); within one run every consumer reads
the same tensors.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

ROW_DIM = 576          # latent row: 512 compressed dims + 64 rope dims
V_DIM = 512            # value = first 512 dims of the latent row
SCALE = 1.0 / math.sqrt(192.0)   # 1/sqrt(d_nope + d_rope) = 1/sqrt(128 + 64)


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    q_len: int
    N: int
    page_size: int
    S: int                       # fixed context length, or the maximum for "ragged"
    lengths: str = "fixed"       # "fixed" | "ragged"
    interleaves: tuple = (1,)
    q_std: float = 1.0
    kv_std: float = 0.5
    lse_base: str = "e"          # "e" | "2"
    table: str = "random"        # "random" | "identity"
    seed: int = 0
    note: str = field(default="", compare=False)


WORKLOADS = {
    "tiny": Workload("tiny", B=2, H=16, q_len=1, N=4, page_size=16, S=1024,
                     q_std=1.0, kv_std=1.0, lse_base="e", table="identity",
                     note="B=2, S=1024, H=16, N=4, page 16, identity table"),
    "dsv3": Workload("dsv3", B=32, H=128, q_len=1, N=8, page_size=64, S=8192,
                     lse_base="e", note="DeepSeek-V3-shaped: B=32, S=8192, H=128, N=8"),
    "k3": Workload("k3", B=64, H=96, q_len=1, N=8, page_size=64, S=131072,
                   lse_base="2", note="Kimi-K3-shaped: B=64, S=131072, H=96, N=8, base-2 LSE"),
    "ragged": Workload("ragged", B=128, H=96, q_len=1, N=8, page_size=64, S=65536,
                       lengths="ragged", lse_base="e",
                       note="B=128, S log-uniform in [1, 65536] incl. 1..7, H=96, N=8"),
    "long": Workload("long", B=8, H=96, q_len=4, N=8, page_size=64, S=1048576,
                     interleaves=(1, 64), lse_base="2",
                     note="B=8, S=2^20, H=96, q_len=4 causal drafts, N=8, I in {1, 64}"),
}


def seq_lens(w: Workload) -> np.ndarray:
    """Global context length of every request (int64 [B])."""
    if w.lengths == "fixed":
        return np.full(w.B, w.S, dtype=np.int64)
    if w.lengths == "ragged":
        rng = np.random.default_rng([w.seed, 11])
        u = rng.uniform(0.0, math.log(float(w.S)), size=w.B)
        s = np.clip(np.rint(np.exp(u)), 1, w.S).astype(np.int64)
        k = min(7, w.B)
        s[:k] = np.arange(1, k + 1)
        return s
    raise ValueError(f"unknown length kind {w.lengths!r}")


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def make_q(w: Workload, device="cpu") -> torch.Tensor:
    """Query rows q [B, q_len, H, 576] in bfloat16."""
    g = _gen(device, 1000003 * w.seed)
    x = torch.randn((w.B, w.q_len, w.H, ROW_DIM), generator=g, device=device, dtype=torch.float32)
    return (x * w.q_std).to(torch.bfloat16)


def make_request_kv(w: Workload, b: int, S_b: int, device="cpu") -> torch.Tensor:
    """Latent rows of request b in logical order, [S_b, 576] bfloat16."""
    g = _gen(device, 1000003 * w.seed + b + 1)
    x = torch.randn((int(S_b), ROW_DIM), generator=g, device=device, dtype=torch.float32)
    return (x * w.kv_std).to(torch.bfloat16)


def make_all_kv(w: Workload, lens: np.ndarray, device="cpu") -> torch.Tensor:
    """All requests' latent rows concatenated in request order, [sum S_b, 576]."""
    total = int(np.sum(lens))
    out = torch.empty((total, ROW_DIM), dtype=torch.bfloat16, device=device)
    off = 0
    for b, s in enumerate(lens):
        s = int(s)
        if s:
            out[off:off + s] = make_request_kv(w, b, s, device)
        off += s
    return out


def make_block_tables(w: Workload, pages_needed: np.ndarray, spare_pages: int = 0):
    """Per-rank page tables.

    pages_needed [N, B]: pages rank r must give request b.
    Returns (tables, pool_pages): tables is a list of N int32 arrays
    [B, cols] (cols = max pages of any (rank, request), at least 1; unused
    entries -1), pool_pages the number of pages each rank's pool must hold.
    """
    pages_needed = np.asarray(pages_needed, dtype=np.int64)
    N, B = pages_needed.shape
    cols = max(1, int(pages_needed.max()) if pages_needed.size else 1)
    tables = []
    if w.table == "identity":
        pool_pages = B * cols + spare_pages
        for r in range(N):
            t = np.full((B, cols), -1, dtype=np.int32)
            for b in range(B):
                k = int(pages_needed[r, b])
                t[b, :k] = b * cols + np.arange(k)
            tables.append(t)
        return tables, pool_pages
    if w.table == "random":
        pool_pages = int(pages_needed.sum(axis=1).max()) + spare_pages
        pool_pages = max(pool_pages, 1)
        for r in range(N):
            rng = np.random.default_rng([w.seed, 23, r])
            perm = rng.permutation(pool_pages).astype(np.int32)
            t = np.full((B, cols), -1, dtype=np.int32)
            k = 0
            for b in range(B):
                n = int(pages_needed[r, b])
                t[b, :n] = perm[k:k + n]
                k += n
            tables.append(t)
        return tables, pool_pages
    raise ValueError(f"unknown table kind {w.table!r}")


def bf16_nan_fill(t: torch.Tensor) -> torch.Tensor:
    """Fill a bfloat16 tensor with quiet NaN so that any read of a row that was
    never written shows up in the output."""
    return t.view(torch.int16).fill_(0x7FC0).view(torch.bfloat16)
