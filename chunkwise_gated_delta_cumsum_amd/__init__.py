"""Chunkwise gated delta rule forward (Gated DeltaNet / KDA) for MI355X.

The computation runs in hand-written HIP kernels for gfx950 behind the C ABI
declared in include/gdr.h (libgdr.so, built in-tree by ``build.py``); this
package is the thin Python binding over it plus the seeded input generator.
"""
from .binding import (GDR_BF16, GDR_F32, CHECK_BITS, EXPORTED, GdrError, GdrProblem,  # noqa: F401
                      LIB_PATH, NOALLOC_SCRATCH_BYTES, check, check_bit_names,
                      gdr_check_inputs, gdr_chunk_fwd, gdr_chunk_fwd_noalloc,
                      gdr_chunk_prep, gdr_chunk_scan, gdr_decode_step, load,
                      problem,
                      scan_segments, scan_slab, status_string, workspace_size)

__version__ = "0.5.0"
