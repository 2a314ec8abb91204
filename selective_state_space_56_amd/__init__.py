"""MI355X (gfx950) selective state-space scan (S6): fused scan forward and
one-token decode as hand-written HIP kernels behind a C ABI
(``include/mamba_scan.h``), with a thin ctypes binding.

``scan_fwd`` and ``state_update`` call the native library; importing this
package does not load it, but the first call does, and raises if the library
has not been built (there is no fallback path).
"""
from .binding import scan_fwd, state_update, workspace_size, library_path, load_library  # noqa: F401
