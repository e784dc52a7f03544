"""ctypes binding of libdcp_probe.so: the streaming-read probe that measures
the HBM read peak with the stripe kernel's own 16-byte direct-to-LDS load, and
the MFMA probe that measures the bf16 matrix peak with its own MFMA
instruction.

A measurement tool only (bench.py uses it); the attention path never calls it.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
PROBE_LIB_PATH = os.path.join(_PKG, "libdcp_probe.so")

MODES = {"lds1": 0, "lds4": 1, "reg": 2}
MODE_NOTES = {
    "lds1": "16-byte direct-to-LDS non-temporal loads by one wave per workgroup, 4-stage ring "
            "(the stripe kernel's loader without its compute), one workgroup per CU",
    "lds4": "the same loads issued by four waves per workgroup",
    "reg": "16-byte non-temporal loads into registers, eight in flight per lane",
}

_h: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    global _h
    if _h is None:
        if not os.path.exists(PROBE_LIB_PATH):
            raise RuntimeError(f"{PROBE_LIB_PATH} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        h = ctypes.CDLL(PROBE_LIB_PATH)
        h.dcp_probe_stream.restype = ctypes.c_int
        h.dcp_probe_stream.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64), ctypes.c_void_p]
        h.dcp_probe_block_threads.restype = ctypes.c_int
        h.dcp_probe_block_threads.argtypes = [ctypes.c_int32]
        h.dcp_probe_mfma.restype = ctypes.c_int
        h.dcp_probe_mfma.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64),
                                     ctypes.c_void_p]
        h.dcp_probe_mfma_block_threads.restype = ctypes.c_int
        h.dcp_probe_mfma_block_threads.argtypes = []
        _h = h
    return _h


def grid_for(mode: str, cus: int) -> int:
    return cus if mode in ("lds1", "lds4") else 8 * cus


def make_sink(mode: str, grid: int, device) -> torch.Tensor:
    return torch.empty(grid * lib().dcp_probe_block_threads(MODES[mode]), dtype=torch.int32, device=device)


def stream(src: torch.Tensor, nbytes: int, mode: str, grid: int, sink: torch.Tensor, stream_handle: int) -> int:
    """Enqueue one streaming read of the first `nbytes` bytes of `src`; returns the bytes read."""
    if not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous GPU tensor")
    if nbytes > src.numel() * src.element_size():
        raise ValueError("nbytes exceeds the tensor")
    got = ctypes.c_int64(0)
    rc = lib().dcp_probe_stream(ctypes.c_void_p(src.data_ptr()), int(nbytes), MODES[mode], int(grid),
                                ctypes.c_void_p(sink.data_ptr()), ctypes.byref(got), ctypes.c_void_p(stream_handle))
    if rc != 0:
        raise RuntimeError(f"dcp_probe_stream returned {rc}")
    return int(got.value)


def make_mfma_sink(grid: int, device) -> torch.Tensor:
    return torch.empty(grid * lib().dcp_probe_mfma_block_threads(), dtype=torch.float32, device=device)


def mfma(grid: int, iters: int, sink: torch.Tensor, stream_handle: int) -> int:
    """Enqueue one MFMA-probe launch (8 waves per workgroup, 4 independent
    32x32x16 bf16 chains per wave); returns its matrix FLOPs."""
    flops = ctypes.c_int64(0)
    rc = lib().dcp_probe_mfma(int(grid), int(iters), ctypes.c_void_p(sink.data_ptr()), ctypes.byref(flops),
                              ctypes.c_void_p(stream_handle))
    if rc != 0:
        raise RuntimeError(f"dcp_probe_mfma returned {rc}")
    return int(flops.value)
