"""MI355X-native selective scan (Mamba SSM) behind a C-ABI HIP library.

The public entry points mirror the C functions of ``include/ssm_scan.h``:
``ssm_scan_fwd``, ``ssm_scan_fwd_noalloc`` (the same scan without any
allocation), ``ssm_scan_fwd_wavefront`` (the same scan as a chunked
associative scan, for comparison), ``ssm_scan_workspace_size``, ``ssm_scan_aggregate`` (the
affine aggregate of a sequence shard), ``ssm_state_update`` and the backward
pass ``ssm_scan_bwd``. They
take torch tensors only as carriers of device pointers and the current stream;
every step of the computation runs in the HIP kernels of ``libssmscan.so``.
The library is loaded on first use and a missing build raises at that point.
"""
from .binding import (  # noqa: F401
    SsmError,
    library_path,
    load_library,
    ssm_scan_aggregate,
    ssm_scan_bwd,
    ssm_scan_fwd,
    ssm_scan_fwd_noalloc,
    ssm_scan_fwd_wavefront,
    ssm_scan_workspace_size,
    ssm_state_update,
)
