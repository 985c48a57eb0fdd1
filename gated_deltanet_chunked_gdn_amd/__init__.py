"""Chunked gated delta rule (Gated DeltaNet) for AMD Instinct MI355X (gfx950).

The computation lives in libgdn.so (HIP kernels behind the C ABI of
include/gdn.h); this package is its Python binding plus the seeded synthetic
input generators.
"""
from .ops import (SeqLens, chunk_bwd, chunk_fwd, chunk_fwd_noalloc, device_copy, epilogue,  # noqa: F401
                  forward_workspace, kda_chunk_fwd, make_problem, prologue, recurrent_ref)
from ._native import GdnError, GdnLibraryMissing  # noqa: F401
