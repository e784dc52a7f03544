"""MI355X-native decode context parallelism (DCP) for absorbed-MLA latent KV.

The compute lives in a C-ABI shared library (``libdcp.so``, HIP kernels for
gfx950) declared in ``include/dcp.h``; ``mla_context_kv_amd.dcp`` is a thin
ctypes binding with the same entry-point names.  PyTorch is used only for
device memory and streams.  The library is loaded on first use, and a missing
or unloadable library raises immediately: there is no fallback path.
"""

from .workloads import WORKLOADS, Workload, SCALE, ROW_DIM, V_DIM  # noqa: F401
