"""The measurement probes' library (libdcp_probe.so): it loads, exports its
entry points, and rejects bad arguments on the host before any launch."""

import ctypes

from mla_context_kv_amd import probe as PR


def test_probe_library_exports_and_argument_errors():
    L = PR.lib()
    assert L.dcp_probe_block_threads(0) == 512 and L.dcp_probe_block_threads(2) == 256
    assert L.dcp_probe_mfma_block_threads() == 512
    fake = ctypes.c_void_p(0x1000)
    got = ctypes.c_int64(-1)
    # streaming read: NULL source or sink, negative size, bad mode or grid
    assert L.dcp_probe_stream(None, 1 << 20, 0, 1, fake, ctypes.byref(got), None) == -1
    assert L.dcp_probe_stream(fake, 1 << 20, 0, 1, None, ctypes.byref(got), None) == -1
    assert L.dcp_probe_stream(fake, -1, 0, 1, fake, ctypes.byref(got), None) == -1
    assert L.dcp_probe_stream(fake, 1 << 20, 3, 1, fake, ctypes.byref(got), None) == -1
    assert L.dcp_probe_stream(fake, 1 << 20, 0, 0, fake, ctypes.byref(got), None) == -1
    # less than one 36,864-byte piece: nothing to read, nothing launched
    assert L.dcp_probe_stream(fake, 36863, 0, 1, fake, ctypes.byref(got), None) == 0 and got.value == 0
    # MFMA probe: bad grid, iterations or sink
    assert L.dcp_probe_mfma(0, 10, fake, ctypes.byref(got), None) == -1
    assert L.dcp_probe_mfma(4, 0, fake, ctypes.byref(got), None) == -1
    assert L.dcp_probe_mfma(4, 10, None, ctypes.byref(got), None) == -1
