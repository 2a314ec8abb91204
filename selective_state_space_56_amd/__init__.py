"""MI355X (gfx950) selective state-space scan (S6): fused scan forward, its
backward (gradients by state recomputation) and one-token decode, and the causal convolution + SiLU front-end of the SSM
branch, as hand-written HIP kernels behind a C ABI (``include/mamba_scan.h``,
``include/mamba_scan_bwd.h``, ``include/mamba_conv.h``), with a thin ctypes binding;
and the Mamba-2 SSD layer by the chunked algorithm on the matrix cores
(``include/mamba_ssd.h``).

``scan_fwd`` and ``state_update`` call the native library; importing this
package does not load it, but the first call does, and raises if the library
has not been built (there is no fallback path).
"""
from .binding import (bwd_workspace_size, conv1d_fwd, conv1d_update, library_path,  # noqa: F401
                      load_library, scan_bwd, scan_fwd, ssd_fwd, state_update, workspace_size)
