"""Thin ctypes binding of libdcp (include/dcp.h) with the same entry-point names.

Only argument marshalling happens here: shapes, dtypes, devices and
contiguity are checked, tensors are passed as raw device pointers together
with torch's current HIP stream, and every step of the computation runs in the
library's kernels.  There is no fallback: if libdcp.so is missing or fails to
load, every call raises.
"""

from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdcp.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "dcp.h")

DCP_OK = 0
DCP_EINVAL = -1
DCP_EUNSUPPORTED = -2
DCP_EHIP = -3
DCP_ERANGE = -4
DCP_ESCRATCH = -5

HEAD_DIM = 576
V_DIM = 512


class DcpError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {strerror(code)} ({code})")


class dcp_layout(ctypes.Structure):
    _fields_ = [("n_stripes", ctypes.c_int32), ("interleave", ctypes.c_int32),
                ("page_size", ctypes.c_int32)]


class dcp_attn_args(ctypes.Structure):
    _fields_ = [
        ("layout", dcp_layout),
        ("rank", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("q_len", ctypes.c_int32),
        ("n_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("v_dim", ctypes.c_int32),
        ("q", ctypes.c_void_p),
        ("pool", ctypes.c_void_p),
        ("num_pages", ctypes.c_int64),
        ("block_table", ctypes.c_void_p),
        ("bt_cols", ctypes.c_int32),
        ("seq_len", ctypes.c_void_p),
        ("scale", ctypes.c_float),
        ("lse_base", ctypes.c_int32),
        ("num_splits", ctypes.c_int32),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("o", ctypes.c_void_p),
        ("lse", ctypes.c_void_p),
        ("status", ctypes.c_void_p),
        ("window", ctypes.c_int32),
        ("softcap", ctypes.c_float),
        ("sinks", ctypes.c_void_p),
        ("partials", ctypes.c_int32),
        ("bias_slopes", ctypes.c_void_p),
        ("sparse_rows", ctypes.c_void_p),
        ("sparse_bits", ctypes.c_void_p),
        ("sparse_count", ctypes.c_void_p),
        ("sparse_stride", ctypes.c_int32),
        ("out_records", ctypes.c_int32),
        ("o_bf16", ctypes.c_int32),
    ]


_lib_handle: Optional[ctypes.CDLL] = None

_VP = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SIGNATURES = {
    "dcp_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "dcp_abi_version": (ctypes.c_int, []),
    "dcp_slot_map": (ctypes.c_int, [dcp_layout, _I32, _VP, _VP, _I64, _VP, _I32, _I32, _VP, _VP, _VP, _VP, _VP]),
    "dcp_local_count": (ctypes.c_int, [dcp_layout, _VP, _VP, _I64, _VP, _VP]),
    "dcp_kv_write": (ctypes.c_int, [dcp_layout, _I32, _VP, _I32, _I64, _VP, _VP, _VP, _I32, _I32, _VP, _I64, _VP, _VP]),
    "dcp_stripe_attn_workspace": (ctypes.c_int, [ctypes.POINTER(dcp_attn_args), ctypes.POINTER(ctypes.c_size_t)]),
    "dcp_stripe_attn": (ctypes.c_int, [ctypes.POINTER(dcp_attn_args), _VP]),
    "dcp_stripe_attn_noalloc": (ctypes.c_int, [ctypes.POINTER(dcp_attn_args), _VP]),
    "dcp_stripe_attn_noalloc_max_bytes": (ctypes.c_size_t, []),
    "dcp_stripe_attn_multi_workspace": (ctypes.c_int, [ctypes.POINTER(dcp_attn_args), _I32,
                                                       ctypes.POINTER(ctypes.c_size_t)]),
    "dcp_stripe_attn_multi": (ctypes.c_int, [ctypes.POINTER(dcp_attn_args), _I32, _VP]),
    "dcp_lse_merge": (ctypes.c_int, [_I32, _I64, _I32, _VP, _VP, _I32, _VP, _VP, _VP]),
    "dcp_lse_merge_bf16": (ctypes.c_int, [_I32, _I64, _I32, _VP, _VP, _I32, _VP, _VP, _VP]),
    "dcp_pack_heads": (ctypes.c_int, [_I32, _I64, _I32, _I32, _VP, _VP, _VP, _VP]),
    "dcp_sparse_plan": (ctypes.c_int, [dcp_layout, _I32, _I32, _I32, _I32, _VP, _VP, _VP, _VP, _VP, _I32, _VP]),
    "dcp_merge_heads": (ctypes.c_int, [_I32, _I64, _I32, _VP, _I32, _VP, _VP, _VP]),
    "dcp_relayout": (ctypes.c_int, [dcp_layout, _I32, _I32, _VP, _I64, _I32, _VP, _I32, _VP, _VP, _I32, _I64,
                                    _VP, _I32, _VP, _I64, _VP, _VP]),
}


def lib() -> ctypes.CDLL:
    """The loaded libdcp (raises if it is not built or cannot be loaded)."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, argt) in _SIGNATURES.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = argt
        _lib_handle = h
    return _lib_handle


def header_functions() -> list[str]:
    """Names of the functions include/dcp.h declares."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dcp_[a-z0-9_]+)\s*\(", text)))


def strerror(code: int) -> str:
    return lib().dcp_strerror(int(code)).decode()


def layout(n_stripes: int, interleave: int = 1, page_size: int = 64) -> dcp_layout:
    return dcp_layout(int(n_stripes), int(interleave), int(page_size))


def _check(code: int, where: str):
    if code != DCP_OK:
        raise DcpError(code, where)


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t: Optional[torch.Tensor], dtype=None, name: str = "", device=None) -> Optional[int]:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def dcp_slot_map(lay: dcp_layout, rank: int, pos: torch.Tensor, req: Optional[torch.Tensor] = None,
                 block_table: Optional[torch.Tensor] = None, status: Optional[torch.Tensor] = None):
    """owner (int32), local row (int64) and slot (int64) of every position."""
    dev = pos.device
    n = pos.numel()
    owner = torch.empty(n, dtype=torch.int32, device=dev)
    row = torch.empty(n, dtype=torch.int64, device=dev)
    slot = torch.empty(n, dtype=torch.int64, device=dev)
    bt_rows, bt_cols = (block_table.shape if block_table is not None else (0, 0))
    rc = lib().dcp_slot_map(lay, int(rank), _ptr(pos, torch.int64, "pos", dev),
                            _ptr(req, torch.int32, "req", dev), n,
                            _ptr(block_table, torch.int32, "block_table", dev), int(bt_rows), int(bt_cols),
                            owner.data_ptr(), row.data_ptr(), slot.data_ptr(),
                            _ptr(status, torch.int32, "status", dev), _stream(dev))
    _check(rc, "dcp_slot_map")
    return owner, row, slot


def dcp_local_count(lay: dcp_layout, length: torch.Tensor, start: Optional[torch.Tensor] = None):
    """Every rank's share of [start, start+length): int64 [n, N]."""
    dev = length.device
    n = length.numel()
    count = torch.empty((n, lay.n_stripes), dtype=torch.int64, device=dev)
    rc = lib().dcp_local_count(lay, _ptr(start, torch.int64, "start", dev),
                               _ptr(length, torch.int64, "length", dev), n, count.data_ptr(), _stream(dev))
    _check(rc, "dcp_local_count")
    return count


def dcp_kv_write(lay: dcp_layout, rank: int, kv_new: torch.Tensor, pos: torch.Tensor,
                 req: Optional[torch.Tensor], block_table: torch.Tensor, pool: torch.Tensor,
                 status: Optional[torch.Tensor] = None) -> None:
    """Store the rows of kv_new that rank `rank` owns into its paged pool."""
    dev = pool.device
    if kv_new.dim() != 2 or pool.dim() != 3 or pool.shape[2] != kv_new.shape[1]:
        raise ValueError("kv_new must be [T, D] and pool [pages, P, D]")
    if pool.shape[1] != lay.page_size:
        raise ValueError("pool page size does not match the layout")
    rc = lib().dcp_kv_write(lay, int(rank), _ptr(kv_new, torch.bfloat16, "kv_new", dev), int(kv_new.shape[1]),
                            int(kv_new.shape[0]), _ptr(pos, torch.int64, "pos", dev),
                            _ptr(req, torch.int32, "req", dev), _ptr(block_table, torch.int32, "block_table", dev),
                            int(block_table.shape[0]), int(block_table.shape[1]),
                            _ptr(pool, torch.bfloat16, "pool", dev), int(pool.shape[0]),
                            _ptr(status, torch.int32, "status", dev), _stream(dev))
    _check(rc, "dcp_kv_write")


def dcp_relayout(lay: dcp_layout, rank: int, src_pool: torch.Tensor, src_block_table: torch.Tensor,
                 start: torch.Tensor, length: torch.Tensor, block_table: torch.Tensor, pool: torch.Tensor,
                 max_len: Optional[int] = None, status: Optional[torch.Tensor] = None) -> None:
    """Copy the positions [start[b], start[b] + length[b]) that rank `rank` owns from
    request b's dense prefill pages (src_pool [pages, Ps, D], src_block_table [B, cols])
    into the rank's compact pool (pool [pages, P, D], block_table [B, cols])."""
    dev = pool.device
    if src_pool.dim() != 3 or pool.dim() != 3 or src_pool.shape[2] != pool.shape[2]:
        raise ValueError("src_pool and pool must be [pages, page_size, D] with the same D")
    if pool.shape[1] != lay.page_size:
        raise ValueError("pool page size does not match the layout")
    B = int(start.numel())
    if length.numel() != B or src_block_table.shape[0] != B or block_table.shape[0] != B:
        raise ValueError("start, length and both block tables need one row per request")
    if max_len is None:
        max_len = int(length.max().item()) if B else 0
    rc = lib().dcp_relayout(lay, int(rank), int(pool.shape[2]), _ptr(src_pool, torch.bfloat16, "src_pool", dev),
                            int(src_pool.shape[0]), int(src_pool.shape[1]),
                            _ptr(src_block_table, torch.int32, "src_block_table", dev), int(src_block_table.shape[1]),
                            _ptr(start, torch.int64, "start", dev), _ptr(length, torch.int64, "length", dev), B,
                            int(max_len), _ptr(block_table, torch.int32, "block_table", dev),
                            int(block_table.shape[1]), _ptr(pool, torch.bfloat16, "pool", dev), int(pool.shape[0]),
                            _ptr(status, torch.int32, "status", dev), _stream(dev))
    _check(rc, "dcp_relayout")


def _attn_args(lay, rank, q, pool, block_table, seq_len, scale, lse_base, num_splits,
               workspace, o, lse, status, window=0, softcap=0.0, partials=0) -> dcp_attn_args:
    B, q_len, H, D = q.shape
    a = dcp_attn_args()
    a.layout = lay
    a.rank = int(rank)
    a.batch, a.q_len, a.n_heads, a.head_dim, a.v_dim = int(B), int(q_len), int(H), int(D), V_DIM
    a.num_pages = int(pool.shape[0])
    a.bt_cols = int(block_table.shape[1])
    a.scale = float(scale)
    a.lse_base = int(lse_base)
    a.num_splits = int(num_splits)
    a.window = int(window)
    a.softcap = float(softcap)
    a.partials = int(partials)
    return a


def dcp_stripe_attn_workspace(lay: dcp_layout, rank: int, q: torch.Tensor, pool: torch.Tensor,
                              block_table: torch.Tensor, num_splits: int = 0, lse_base: int = 0) -> int:
    """Workspace bytes dcp_stripe_attn needs for these shapes."""
    a = _attn_args(lay, rank, q, pool, block_table, None, 1.0, lse_base, num_splits, None, None, None, None)
    nbytes = ctypes.c_size_t(0)
    _check(lib().dcp_stripe_attn_workspace(ctypes.byref(a), ctypes.byref(nbytes)), "dcp_stripe_attn_workspace")
    return int(nbytes.value)


def dcp_stripe_attn(lay: dcp_layout, rank: int, q: torch.Tensor, pool: torch.Tensor,
                    block_table: torch.Tensor, seq_len: torch.Tensor, scale: float, lse_base: int = 0,
                    num_splits: int = 0, workspace: Optional[torch.Tensor] = None,
                    o: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                    status: Optional[torch.Tensor] = None, window: int = 0, softcap: float = 0.0,
                    sinks: Optional[torch.Tensor] = None, partials: bool = False,
                    bias_slopes: Optional[torch.Tensor] = None, sparse=None, records: bool = False,
                    o_bf16: bool = False):
    """One rank's stripe attention: returns (o_r fp32 [B,q_len,H,512], lse_r fp32 [B,q_len,H]);
    with o_bf16=True o_r is bf16 (the float32 result rounded to nearest even) and lse_r float32.

    window / softcap / sinks / bias_slopes select the mergeable variants (sinks: fp32 [H], on one
    rank only; bias_slopes: fp32 [H], on every rank).  sparse = (rows, bits, count) from
    dcp_sparse_plan restricts the stripe to the rank's selected tokens.
    partials=True (with num_splits = k >= 1) returns the k unmerged parts instead:
    o [k,B,q_len,H,512], lse [k,B,q_len,H].
    records=True writes packed records in place of (o, lse), already in the head-return send
    layout: returns (rec, None), rec int16 [N, (k,) B*q_len, H/N, 516] (N = lay.n_stripes) --
    the bf16 output then the fp32 lse and two zero slots per (row, head), the record of
    dcp_pack_heads; rec[d] goes to head owner d, whose dcp_merge_heads folds what it receives."""
    dev = q.device
    if q.dim() != 4 or pool.dim() != 3 or block_table.dim() != 2:
        raise ValueError("q must be [B, q_len, H, 576], pool [pages, P, 576], block_table [B, cols]")
    B, q_len, H, D = q.shape
    if pool.shape[1] != lay.page_size or pool.shape[2] != D:
        raise ValueError("pool must be [pages, page_size, head_dim]")
    if block_table.shape[0] != B or seq_len.numel() != B:
        raise ValueError("block_table and seq_len need one row per request")
    k = int(num_splits) if partials else 1
    if partials and k < 1:
        raise ValueError("partials needs num_splits >= 1")
    lead = (k,) if partials else ()
    if records and o_bf16:
        raise ValueError("records already carry bf16 outputs: o_bf16 does not combine with them")
    if records:
        N = int(lay.n_stripes)
        if H % N:
            raise ValueError("records need n_heads to be a multiple of n_stripes")
        if o is None:
            o = torch.empty((N,) + lead + (B * q_len, H // N, V_DIM + 4), dtype=torch.int16, device=dev)
        if o.numel() != k * B * q_len * H * (V_DIM + 4):
            raise ValueError("the record tensor has the wrong size")
        lse = None
    else:
        if o is None:
            o = torch.empty(lead + (B, q_len, H, V_DIM), dtype=torch.bfloat16 if o_bf16 else torch.float32,
                            device=dev)
        if lse is None:
            lse = torch.empty(lead + (B, q_len, H), dtype=torch.float32, device=dev)
        if o.numel() != k * B * q_len * H * V_DIM or lse.numel() != k * B * q_len * H:
            raise ValueError("o / lse have the wrong size")
    a = _attn_args(lay, rank, q, pool, block_table, seq_len, scale, lse_base, num_splits, workspace, o, lse, status,
                   window, softcap, 1 if partials else 0)
    a.out_records = 1 if records else 0
    a.o_bf16 = 1 if o_bf16 else 0
    if sinks is not None and sinks.numel() != H:
        raise ValueError("sinks must hold one value per head")
    if bias_slopes is not None and bias_slopes.numel() != H:
        raise ValueError("bias_slopes must hold one value per head")
    a.q = _ptr(q, torch.bfloat16, "q", dev)
    a.pool = _ptr(pool, torch.bfloat16, "pool", dev)
    a.block_table = _ptr(block_table, torch.int32, "block_table", dev)
    a.seq_len = _ptr(seq_len, torch.int32, "seq_len", dev)
    a.o = _ptr(o, torch.int16 if records else (torch.bfloat16 if o_bf16 else torch.float32), "o", dev)
    a.lse = _ptr(lse, torch.float32, "lse", dev)
    a.status = _ptr(status, torch.int32, "status", dev)
    a.sinks = _ptr(sinks, torch.float32, "sinks", dev)
    a.bias_slopes = _ptr(bias_slopes, torch.float32, "bias_slopes", dev)
    if sparse is not None:
        rows, bits, count = sparse
        if rows.shape[0] != B or bits.shape != rows.shape or count.numel() != B:
            raise ValueError("sparse rows / bits must be [B, stride] and count [B]")
        a.sparse_rows = _ptr(rows, torch.int32, "sparse rows", dev)
        a.sparse_bits = _ptr(bits, torch.int32, "sparse bits", dev)
        a.sparse_count = _ptr(count, torch.int32, "sparse count", dev)
        a.sparse_stride = int(rows.shape[1])
    # the size query sees every field the call will see (a sparse selection
    # sizes the plan by its stride, not by the page table)
    need = ctypes.c_size_t(0)
    _check(lib().dcp_stripe_attn_workspace(ctypes.byref(a), ctypes.byref(need)), "dcp_stripe_attn_workspace")
    if need.value and (workspace is None or workspace.numel() * workspace.element_size() < need.value):
        workspace = torch.empty(need.value, dtype=torch.uint8, device=dev)
    a.workspace = _ptr(workspace, None, "workspace", dev) if workspace is not None else None
    a.workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().dcp_stripe_attn(ctypes.byref(a), _stream(dev)), "dcp_stripe_attn")
    return o, lse


def dcp_stripe_attn_noalloc(lay: dcp_layout, rank: int, q: torch.Tensor, pool: torch.Tensor,
                            block_table: torch.Tensor, seq_len: torch.Tensor, scale: float, lse_base: int = 0,
                            num_splits: int = 0, o: torch.Tensor = None, lse: torch.Tensor = None,
                            status: Optional[torch.Tensor] = None):
    """dcp_stripe_attn through the entry point that allocates nothing (the
    library's fixed per-GPU scratch buffer replaces the workspace).  o and lse
    must be given, so the call allocates nothing on this side either."""
    dev = q.device
    if q.dim() != 4 or pool.dim() != 3 or block_table.dim() != 2:
        raise ValueError("q must be [B, q_len, H, 576], pool [pages, P, 576], block_table [B, cols]")
    B, q_len, H, D = q.shape
    if o is None or lse is None:
        raise ValueError("o and lse are required")
    if o.numel() != B * q_len * H * V_DIM or lse.numel() != B * q_len * H:
        raise ValueError("o / lse have the wrong size")
    if block_table.shape[0] != B or seq_len.numel() != B or pool.shape[1] != lay.page_size:
        raise ValueError("block_table and seq_len need one row per request, pool [pages, page_size, 576]")
    a = _attn_args(lay, rank, q, pool, block_table, seq_len, scale, lse_base, num_splits, None, o, lse, status)
    a.q = _ptr(q, torch.bfloat16, "q", dev)
    a.pool = _ptr(pool, torch.bfloat16, "pool", dev)
    a.block_table = _ptr(block_table, torch.int32, "block_table", dev)
    a.seq_len = _ptr(seq_len, torch.int32, "seq_len", dev)
    a.o = _ptr(o, torch.float32, "o", dev)
    a.lse = _ptr(lse, torch.float32, "lse", dev)
    a.status = _ptr(status, torch.int32, "status", dev)
    _check(lib().dcp_stripe_attn_noalloc(ctypes.byref(a), _stream(dev)), "dcp_stripe_attn_noalloc")
    return o, lse


def dcp_lse_merge(o_parts: torch.Tensor, lse_parts: torch.Tensor, lse_base: int = 0,
                  o: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None):
    """Exact merge over the leading (stripe) axis: o_parts [N, ..., V] (float32, or bfloat16
    through dcp_lse_merge_bf16), lse_parts [N, ...] float32; o, lse float32."""
    dev = o_parts.device
    N = o_parts.shape[0]
    v_dim = o_parts.shape[-1]
    rows = lse_parts[0].numel()
    if o_parts.numel() != N * rows * v_dim or lse_parts.shape[0] != N:
        raise ValueError("o_parts must be [N, rows..., V] matching lse_parts [N, rows...]")
    if o is None:
        o = torch.empty(o_parts.shape[1:], dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty(lse_parts.shape[1:], dtype=torch.float32, device=dev)
    bf16 = o_parts.dtype == torch.bfloat16
    fn = lib().dcp_lse_merge_bf16 if bf16 else lib().dcp_lse_merge
    rc = fn(int(N), int(rows), int(v_dim), _ptr(o_parts, torch.bfloat16 if bf16 else torch.float32, "o_parts", dev),
            _ptr(lse_parts, torch.float32, "lse_parts", dev), int(lse_base),
            _ptr(o, torch.float32, "o", dev), _ptr(lse, torch.float32, "lse", dev), _stream(dev))
    _check(rc, "dcp_lse_merge_bf16" if bf16 else "dcp_lse_merge")
    return o, lse


def dcp_pack_heads(o_r: torch.Tensor, lse_r: torch.Tensor, n_stripes: int,
                   send: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Pack one rank's (o_r [B, q_len, H, V] fp32, lse_r [B, q_len, H] fp32) by head owner:
    returns send int16 [N, B*q_len, H/N, V + 4] (bf16 output, fp32 lse, padding per record)."""
    dev = o_r.device
    H, v = int(o_r.shape[-2]), int(o_r.shape[-1])
    rows = int(o_r.numel() // (H * v))
    N = int(n_stripes)
    if lse_r.numel() != rows * H or H % N:
        raise ValueError("lse_r must be [..., H] matching o_r, and H a multiple of n_stripes")
    if send is None:
        send = torch.empty((N, rows, H // N, v + 4), dtype=torch.int16, device=dev)
    if send.numel() != N * rows * (H // N) * (v + 4):
        raise ValueError("send has the wrong size")
    rc = lib().dcp_pack_heads(N, rows, H, v, _ptr(o_r, torch.float32, "o_r", dev), _ptr(lse_r, torch.float32, "lse_r", dev),
                              _ptr(send, torch.int16, "send", dev), _stream(dev))
    _check(rc, "dcp_pack_heads")
    return send


def dcp_merge_heads(recv: torch.Tensor, lse_base: int = 0, o: Optional[torch.Tensor] = None,
                    lse: Optional[torch.Tensor] = None):
    """The owner's merge of received records recv int16 [N, rows..., V + 4]:
    returns o fp32 [rows..., V] and lse fp32 [rows...]."""
    dev = recv.device
    N = int(recv.shape[0])
    v = int(recv.shape[-1]) - 4
    rows = int(recv[0].numel() // (v + 4))
    if o is None:
        o = torch.empty(tuple(recv.shape[1:-1]) + (v,), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty(tuple(recv.shape[1:-1]), dtype=torch.float32, device=dev)
    rc = lib().dcp_merge_heads(N, rows, v, _ptr(recv, torch.int16, "recv", dev), int(lse_base),
                               _ptr(o, torch.float32, "o", dev), _ptr(lse, torch.float32, "lse", dev), _stream(dev))
    _check(rc, "dcp_merge_heads")
    return o, lse


def dcp_sparse_plan(lay: dcp_layout, rank: int, topk_pos: torch.Tensor, seq_len: torch.Tensor,
                    out=None):
    """Rank `rank`'s share of a global selection topk_pos int32 [B, q_len, K] (-1 = unused):
    returns (rows int32 [B, q_len*K], bits int32 [B, q_len*K], count int32 [B])."""
    dev = topk_pos.device
    if topk_pos.dim() != 3:
        raise ValueError("topk_pos must be [B, q_len, K]")
    B, q_len, K = (int(x) for x in topk_pos.shape)
    if out is None:
        rows = torch.empty((B, q_len * K), dtype=torch.int32, device=dev)
        bits = torch.empty((B, q_len * K), dtype=torch.int32, device=dev)
        count = torch.empty(B, dtype=torch.int32, device=dev)
    else:
        rows, bits, count = out
    rc = lib().dcp_sparse_plan(lay, int(rank), B, q_len, K, _ptr(topk_pos, torch.int32, "topk_pos", dev),
                               _ptr(seq_len, torch.int32, "seq_len", dev), _ptr(rows, torch.int32, "rows", dev),
                               _ptr(bits, torch.int32, "bits", dev), _ptr(count, torch.int32, "count", dev),
                               int(rows.shape[1]), _stream(dev))
    _check(rc, "dcp_sparse_plan")
    return rows, bits, count


def dcp_stripe_attn_multi(lay: dcp_layout, ranks, q: torch.Tensor, pools, block_tables, seq_len: torch.Tensor,
                          scale: float, lse_base: int = 0, num_splits: int = 0, o: Optional[torch.Tensor] = None,
                          lse: Optional[torch.Tensor] = None, status: Optional[torch.Tensor] = None,
                          window: int = 0, softcap: float = 0.0, sinks=None, bias_slopes=None, sparse=None,
                          workspace: Optional[torch.Tensor] = None, records: bool = False,
                          o_bf16: bool = False):
    """The stripe attentions of several ranks in one launch: ranks[i] with pools[i],
    block_tables[i] (and sinks[i], sparse[i] when given per rank, else None).  Returns
    o [n, B, q_len, H, 512] and lse [n, B, q_len, H], equal to n dcp_stripe_attn calls.
    records=True: returns (rec, None), rec int16 [n, N, B*q_len, H/N, 516], each rank's
    records in head-owner order (see dcp_stripe_attn)."""
    dev = q.device
    n = len(ranks)
    B, q_len, H, D = q.shape
    if len(pools) != n or len(block_tables) != n:
        raise ValueError("one pool and one block table per rank")
    if records:
        N = int(lay.n_stripes)
        if H % N:
            raise ValueError("records need n_heads to be a multiple of n_stripes")
        if o is None:
            o = torch.empty((n, N, B * q_len, H // N, V_DIM + 4), dtype=torch.int16, device=dev)
        if o.shape[0] != n or o[0].numel() != B * q_len * H * (V_DIM + 4):
            raise ValueError("the record tensor needs one block of [N, B*q_len, H/N, 516] per rank")
        lse = None
    else:
        if o is None:
            o = torch.empty((n, B, q_len, H, V_DIM), dtype=torch.bfloat16 if o_bf16 else torch.float32, device=dev)
        if lse is None:
            lse = torch.empty((n, B, q_len, H), dtype=torch.float32, device=dev)
        if o.shape[0] != n or lse.shape[0] != n:
            raise ValueError("o / lse need one block per rank")
    arr = (dcp_attn_args * n)()
    for i in range(n):
        a = _attn_args(lay, ranks[i], q, pools[i], block_tables[i], seq_len, scale, lse_base, num_splits,
                       None, None, None, None, window, softcap, 0)
        a.q = _ptr(q, torch.bfloat16, "q", dev)
        a.pool = _ptr(pools[i], torch.bfloat16, "pool", dev)
        a.block_table = _ptr(block_tables[i], torch.int32, "block_table", dev)
        a.seq_len = _ptr(seq_len, torch.int32, "seq_len", dev)
        a.o = _ptr(o[i], torch.int16 if records else (torch.bfloat16 if o_bf16 else torch.float32), "o", dev)
        a.lse = None if records else _ptr(lse[i], torch.float32, "lse", dev)
        a.out_records = 1 if records else 0
        a.o_bf16 = 1 if o_bf16 else 0
        a.status = _ptr(status, torch.int32, "status", dev)
        a.bias_slopes = _ptr(bias_slopes, torch.float32, "bias_slopes", dev)
        if sinks is not None and sinks[i] is not None:
            a.sinks = _ptr(sinks[i], torch.float32, "sinks", dev)
        if sparse is not None:
            rows, bits, count = sparse[i]
            a.sparse_rows = _ptr(rows, torch.int32, "sparse rows", dev)
            a.sparse_bits = _ptr(bits, torch.int32, "sparse bits", dev)
            a.sparse_count = _ptr(count, torch.int32, "sparse count", dev)
            a.sparse_stride = int(rows.shape[1])
        arr[i] = a
    need = ctypes.c_size_t(0)
    _check(lib().dcp_stripe_attn_multi_workspace(arr, n, ctypes.byref(need)), "dcp_stripe_attn_multi_workspace")
    if need.value and (workspace is None or workspace.numel() * workspace.element_size() < need.value):
        workspace = torch.empty(need.value, dtype=torch.uint8, device=dev)
    if workspace is not None:
        arr[0].workspace = _ptr(workspace, None, "workspace", dev)
        arr[0].workspace_bytes = workspace.numel() * workspace.element_size()
    _check(lib().dcp_stripe_attn_multi(arr, n, _stream(dev)), "dcp_stripe_attn_multi")
    return o, lse
