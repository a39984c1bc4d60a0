"""Mamba-2 SSD forward pass for AMD Instinct MI355X (gfx950).

The computation lives in ``libssd.so`` (C ABI declared in include/ssd.h, HIP
kernels under csrc/); this package is its thin Python binding. Build the
library with ``python -m mamba_ssd_scan_fwd_amd.build``.
"""

from .binding import (  # noqa: F401
    EXPORTED_SYMBOLS,
    PATH_NAMES,
    STATUS_CHAIN_INCOMPLETE,
    STATUS_NO_RECORD,
    STATUS_WAIT_CUT_OFF_ONE_PASS,
    STATUS_WAIT_CUT_OFF_SEGMENTED,
    SSDDesc,
    SSDError,
    chunk_cumsum,
    chunk_scan,
    chunk_state,
    conv1d_split,
    cumsum_chunk_state,
    decode_step,
    effective_chunk_size,
    forward,
    forward_noalloc,
    forward_varlen,
    lib_path,
    load_library,
    make_desc,
    state_passing,
    status_string,
    workspace_bytes,
    workspace_bytes_varlen,
    workspace_status,
    workspace_status_varlen,
)
