"""gfx950 (MI355X) matrix-state affine prefix scan: gated delta rule (with
optionally split erase/write strengths), gated linear attention, and PRISM's
rank-L write expanded onto the same scan, diagonal (per-key-channel) gates and
the scan's gradient; and the large-chunk fast-weight update (LaCT-style
test-time training with linear fast weights).

The compute path is the C-ABI library ``libgdscan.so`` (``include/gdscan.h``,
sources in ``csrc/``); this package is its Python binding.  The library is
loaded on first use.
"""
from ._lib import (  # noqa: F401
    PATHS, SCAN_BF16, SCAN_F32, SCAN_GDN, SCAN_GDN_DIAG, SCAN_GDN_EW, SCAN_GLA, SCAN_GLA_DIAG,
    ScanError, decode_step,
    last_error, lact_fwd, lact_fwd_workspace_size, lib, prism_expand, prism_scan, prism_scan_fwd,
    prism_scan_workspace_size, scan_bwd,
    scan_bwd_workspace_size, scan_fwd, scan_fwd_noalloc, scan_fwd_workspace_size, version,
)
