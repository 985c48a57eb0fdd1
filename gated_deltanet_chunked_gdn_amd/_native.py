"""ctypes binding of libgdn.so (the C ABI declared in include/gdn.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the ABI.  Importing this module never builds anything; if the
library is missing, loading raises ``GdnLibraryMissing`` (there is no CPU
fallback).
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libgdn.so")

# gdn_status
GDN_OK = 0
GDN_ERR_NULL = 1
GDN_ERR_SHAPE = 2
GDN_ERR_DTYPE = 3
GDN_ERR_UNSUPPORTED = 4
GDN_ERR_WORKSPACE = 5
GDN_ERR_ALIAS = 6
GDN_ERR_HIP = 7
GDN_ERR_SEQLENS = 8
GDN_ERR_ALIGN = 9
GDN_ERR_SCRATCH = 10
# bytes of the device array gdn_chunk_fwd_noalloc uses as its workspace
GDN_NOALLOC_SCRATCH_BYTES = 64 << 20
# gdn_dtype
GDN_FP32 = 0
GDN_BF16 = 1
# gdn_precision
GDN_PRECISION_IO = 0
GDN_PRECISION_FP32 = 1
# gdn_gate_kind
GDN_GATE_GDN = 0
GDN_GATE_BOUNDED5 = 1
GDN_GATE_GDN_CHANNEL = 2
# gdn_pass
GDN_PASS_CHUNK_FWD = 0
GDN_PASS_CHUNK_BWD = 1
GDN_PASS_RECURRENT_FWD = 2
GDN_PASS_RECURRENT_BWD = 3
GDN_PASS_KDA_FWD = 4
GDN_PASS_CHUNK_SAVED = 5
GDN_PASS_KDA_BWD = 6
GDN_PASS_KDA_SAVED = 7

# Every symbol include/gdn.h declares.
EXPORTED = ("gdn_abi_version", "gdn_status_str", "gdn_workspace_size", "gdn_chunk_fwd",
            "gdn_chunk_bwd", "gdn_recurrent_ref", "gdn_prologue", "gdn_epilogue",
            "gdn_kda_chunk_fwd", "gdn_chunk_fwd_noalloc", "gdn_device_copy", "gdn_chunk_fwd_save",
            "gdn_chunk_bwd_saved", "gdn_kda_chunk_bwd", "gdn_kda_chunk_fwd_save", "gdn_kda_chunk_bwd_saved")


class GdnLibraryMissing(RuntimeError):
    pass


class GdnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} (status {status})")


class Problem(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
        ("Dk", ctypes.c_int32), ("Dv", ctypes.c_int32),
        ("num_seqs", ctypes.c_int32),
        ("cu_seqlens_host", ctypes.c_void_p),
        ("cu_seqlens_dev", ctypes.c_void_p),
        ("io_dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("chunk", ctypes.c_int32),
        ("num_segments", ctypes.c_int32),
        ("precision", ctypes.c_int32),
    ]


_lib = None


def load():
    """Load libgdn.so once; raise GdnLibraryMissing if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise GdnLibraryMissing(
            f"{LIB_PATH} not found: build it with `python -m gated_deltanet_chunked_gdn_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    PP = ctypes.POINTER(Problem)
    lib.gdn_abi_version.argtypes = []
    lib.gdn_abi_version.restype = ctypes.c_int32
    lib.gdn_status_str.argtypes = [ctypes.c_int32]
    lib.gdn_status_str.restype = ctypes.c_char_p
    lib.gdn_workspace_size.argtypes = [PP, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]
    lib.gdn_workspace_size.restype = ctypes.c_int
    lib.gdn_chunk_fwd.argtypes = [PP, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.gdn_chunk_fwd.restype = ctypes.c_int
    lib.gdn_chunk_bwd.argtypes = [PP, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P,
                                  ctypes.c_size_t, P]
    lib.gdn_chunk_bwd.restype = ctypes.c_int
    lib.gdn_recurrent_ref.argtypes = [PP, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P,
                                      ctypes.c_size_t, P]
    lib.gdn_recurrent_ref.restype = ctypes.c_int
    lib.gdn_prologue.argtypes = [PP, P, P, P, P, P, P, ctypes.c_int32, ctypes.c_int32, P, P, P, P, P]
    lib.gdn_prologue.restype = ctypes.c_int
    lib.gdn_epilogue.argtypes = [PP, P, P, P, ctypes.c_float, P, P]
    lib.gdn_epilogue.restype = ctypes.c_int
    lib.gdn_kda_chunk_fwd.argtypes = [PP, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.gdn_kda_chunk_fwd.restype = ctypes.c_int
    lib.gdn_chunk_fwd_noalloc.argtypes = [PP, P, P, P, P, P, P, P, P, P]
    lib.gdn_chunk_fwd_noalloc.restype = ctypes.c_int
    lib.gdn_device_copy.argtypes = [P, P, ctypes.c_size_t, P]
    lib.gdn_chunk_fwd_save.argtypes = [PP, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.gdn_chunk_fwd_save.restype = ctypes.c_int
    lib.gdn_chunk_bwd_saved.argtypes = [PP, P, P, P, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.gdn_chunk_bwd_saved.restype = ctypes.c_int
    lib.gdn_device_copy.restype = ctypes.c_int
    lib.gdn_kda_chunk_bwd.argtypes = [PP, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.gdn_kda_chunk_bwd.restype = ctypes.c_int
    lib.gdn_kda_chunk_fwd_save.argtypes = [PP, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.gdn_kda_chunk_fwd_save.restype = ctypes.c_int
    lib.gdn_kda_chunk_bwd_saved.argtypes = [PP, P, P, P, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.gdn_kda_chunk_bwd_saved.restype = ctypes.c_int
    _lib = lib
    return lib


def status_str(status: int) -> str:
    try:
        return load().gdn_status_str(int(status)).decode()
    except GdnLibraryMissing:
        return "unknown"


def workspace_size(problem: Problem, pass_: int) -> int:
    n = ctypes.c_size_t(0)
    st = load().gdn_workspace_size(ctypes.byref(problem), int(pass_), ctypes.byref(n))
    if st != GDN_OK:
        raise GdnError(st, "gdn_workspace_size")
    return int(n.value)


def check(status: int, where: str) -> None:
    if status != GDN_OK:
        raise GdnError(status, where)
