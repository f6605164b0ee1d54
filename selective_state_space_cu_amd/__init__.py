"""Mamba2 SSD chunked selective scan over variable-length packed batches, for
AMD Instinct MI355X (gfx950): HIP kernels behind the C ABI of libssd.so
(include/ssd.h), with a thin ctypes binding."""
from .ssd import (SSDError, VarlenMeta, chunk_scan_varlen, export_chunk_states,  # noqa: F401
                  load_library, status_string, varlen_metadata)
