"""MI355X (gfx950) selective state-space scan: forward, backward, impulse
sensitivity (one output row or a block of rows of the input Jacobian),
forward-mode complex gradients, complex scans with given transitions and
PD-transition scans behind the C ABI of
include/ssmscan.h.

The Python functions marshal torch tensors into the C ABI of libssmscan.so;
all computation runs in the library's HIP kernels.
"""
from .binding import (  # noqa: F401
    SSM_BF16,
    SSM_EULER,
    SSM_ZOH,
    SSM_COMPLEX_DENSE,
    SSM_COMPLEX_SHARED,
    SSM_F32,
    SSM_HEAD_SCALAR,
    SSM_REAL_DENSE,
    SSM_REAL_SELECTIVE,
    SSMError,
    complex_rtrl,
    impulse_sensitivity,
    lib,
    n_chunks,
    output_sensitivity,
    pd_scan_bwd,
    pd_scan_fwd,
    scan_bwd,
    scan_fwd,
    scan_fwd_noalloc,
    sensitivity_rows,
    set_allocator,
)
