"""Chunked gated delta rule (Gated DeltaNet) for AMD Instinct MI355X (gfx950).

The computation lives in libgdn.so (HIP kernels behind the C ABI of
include/gdn.h); this package is its Python binding plus the seeded synthetic
input generators.
"""
from .ops import (SeqLens, chunk_bwd, chunk_bwd_saved, chunk_fwd, chunk_fwd_noalloc,  # noqa: F401
                  chunk_fwd_save, device_copy, epilogue, forward_workspace, kda_chunk_bwd,
                  kda_chunk_bwd_saved, kda_chunk_fwd, kda_chunk_fwd_save, kda_saved_buffer, make_problem,
                  prologue, recurrent_ref, saved_buffer)
from ._native import GdnError, GdnLibraryMissing  # noqa: F401
