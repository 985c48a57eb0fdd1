"""Python entry points over libgdn's C ABI (include/gdn.h).

PyTorch supplies device memory and the current HIP stream; every step of the
computation runs in libgdn's HIP kernels.  There is no CPU fallback: without the
built library every call raises ``GdnLibraryMissing``.

    o, S_final = chunk_fwd(q, k, v, g, beta, S0=None, cu_seqlens=None, scale=1.0)
    grads      = chunk_bwd(q, k, v, g, beta, dO, S0=..., dS_final=None)
    out        = recurrent_ref(q, k, v, g, beta, ..., dO=None)
    q, k, g, beta = prologue(q_raw, k_raw, a, b, A_log=..., dt_bias=..., gate="gdn")
    y          = epilogue(o, z, weight=None, eps=1e-6)
    o, S_final = kda_chunk_fwd(q, k, v, g, beta, ...)   # g (B, T, H, Dk): per-channel decay
    grads      = kda_chunk_bwd(q, k, v, g, beta, dO, ...)
    o, S_final, saved = kda_chunk_fwd_save(...); grads = kda_chunk_bwd_saved(..., saved)

Shapes: q, k (B, T, H, Dk); v (B, T, H, Dv); g, beta (B, T, H) fp32;
S0 / S_final (N, H, Dk, Dv) fp32.  q, k, v share the io dtype (bf16 or fp32).
Packed sequences: B == 1 and ``cu_seqlens`` the N + 1 offsets.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import numpy as np
import torch

from . import _native as nat

_IO = {torch.bfloat16: nat.GDN_BF16, torch.float32: nat.GDN_FP32}


class SeqLens:
    """Packed-sequence offsets held twice: host int32 (validated by the library
    before launching) and a device copy (read by the kernels)."""

    def __init__(self, offsets, device):
        host = np.ascontiguousarray(np.asarray(
            offsets.cpu().numpy() if isinstance(offsets, torch.Tensor) else offsets,
            dtype=np.int32))
        if host.ndim != 1 or host.size < 1:
            raise ValueError("cu_seqlens must be a 1-D sequence of N + 1 offsets")
        self.host = host
        self.dev = torch.from_numpy(host.copy()).to(device)
        self.num_seqs = host.size - 1

    @property
    def max_len(self) -> int:
        return int(np.max(np.diff(self.host))) if self.num_seqs else 0


def _seqlens(cu_seqlens, device) -> Optional[SeqLens]:
    if cu_seqlens is None or isinstance(cu_seqlens, SeqLens):
        return cu_seqlens
    return SeqLens(cu_seqlens, device)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _on_device(t, device, name):
    """Every pointer handed to the library must be device memory of the call's GPU:
    a host pointer reaching a kernel is a memory fault, which the C ABI (it sees
    plain addresses) cannot detect."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be on {device} (got {t.device})")


def _check_inputs(q, k, v, g, beta):
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if not t.is_cuda:
            raise ValueError(f"{name} must be on a GPU device")
        _on_device(t, q.device, name)
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if q.dtype not in _IO or k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one io dtype: bfloat16 or float32")
    if g.dtype != torch.float32 or beta.dtype != torch.float32:
        raise TypeError("g and beta must be float32")
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError("q, k must be (B, T, H, Dk) and v (B, T, H, Dv)")
    if g.shape != q.shape[:3] or beta.shape != q.shape[:3]:
        raise ValueError("g and beta must be (B, T, H)")


def _fp32_state(t, N, H, Dk, Dv, name, device):
    if t is None:
        return None
    _on_device(t, device, name)
    if t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != (N, H, Dk, Dv):
        raise ValueError(f"{name} must be a contiguous float32 tensor of shape {(N, H, Dk, Dv)}")
    return t


_PRECISION = {"io": nat.GDN_PRECISION_IO, "fp32": nat.GDN_PRECISION_FP32}


def make_problem(q, v, seqs: Optional[SeqLens], scale: float, num_segments: int = 1,
                 precision: str = "io") -> nat.Problem:
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    p = nat.Problem()
    p.B, p.T, p.H, p.Dk, p.Dv = B, T, H, Dk, Dv
    if seqs is None:
        p.num_seqs = B
        p.cu_seqlens_host = None
        p.cu_seqlens_dev = None
    else:
        p.num_seqs = seqs.num_seqs
        p.cu_seqlens_host = seqs.host.ctypes.data
        p.cu_seqlens_dev = seqs.dev.data_ptr()
    p.io_dtype = _IO[q.dtype]
    p.scale = float(scale)
    p.chunk = 64
    p.num_segments = int(num_segments)
    if precision not in _PRECISION:
        raise ValueError(f"precision must be one of {sorted(_PRECISION)}")
    p.precision = _PRECISION[precision]
    return p


def _workspace(problem, pass_, device):
    n = nat.workspace_size(problem, pass_)
    if n == 0:
        return None, 0
    return torch.empty(n, dtype=torch.uint8, device=device), n


def forward_workspace(q, v, cu_seqlens=None, num_segments: int = 1, precision: str = "io"):
    """A uint8 device tensor of the size gdn_chunk_fwd asks for (None if 0 bytes)."""
    seqs = _seqlens(cu_seqlens, q.device)
    return _workspace(make_problem(q, v, seqs, 1.0, num_segments, precision), nat.GDN_PASS_CHUNK_FWD,
                      q.device)[0]


def chunk_fwd(q, k, v, g, beta, S0=None, cu_seqlens=None, scale: float = 1.0,
              num_segments: int = 1, output_final_state: bool = True, out=None,
              final_state_out=None, workspace=None, precision: str = "io"):
    """Chunked forward pass.  Returns (o, S_final or None).

    ``out`` / ``final_state_out`` / ``workspace`` may supply preallocated
    buffers (o shaped like v; S_final (N, H, Dk, Dv) fp32; a uint8 device
    tensor of at least the size the library asks for).  ``precision``: "io"
    (bf16 io: bf16 MFMA operands, fp32 accumulation) or "fp32" (every product in
    IEEE fp32, also for bf16 inputs and output)."""
    lib = nat.load()
    _check_inputs(q, k, v, g, beta)
    seqs = _seqlens(cu_seqlens, q.device)
    prob = make_problem(q, v, seqs, scale, num_segments, precision)
    N, H, Dk, Dv = prob.num_seqs, prob.H, prob.Dk, prob.Dv
    S0 = _fp32_state(S0, N, H, Dk, Dv, "S0", q.device)
    if out is None:
        o = torch.empty_like(v)
    else:
        _on_device(out, q.device, "out")
        if out.dtype != v.dtype or out.shape != v.shape or not out.is_contiguous():
            raise ValueError("out must be contiguous, shaped and typed like v")
        o = out
    if final_state_out is not None:
        Sf = _fp32_state(final_state_out, N, H, Dk, Dv, "final_state_out", q.device)
    elif output_final_state:
        Sf = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=q.device)
    else:
        Sf = None
    if workspace is not None:
        _on_device(workspace, q.device, "workspace")
        if not workspace.is_contiguous():
            raise ValueError("workspace must be contiguous")
        ws, nws = workspace, workspace.numel() * workspace.element_size()
    else:
        ws, nws = _workspace(prob, nat.GDN_PASS_CHUNK_FWD, q.device)
    st = lib.gdn_chunk_fwd(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                           _ptr(S0), _ptr(o), _ptr(Sf), _ptr(ws), nws, _stream(q.device))
    nat.check(st, "gdn_chunk_fwd")
    return o, Sf


def chunk_fwd_noalloc(q, k, v, g, beta, out, final_state_out=None, S0=None, cu_seqlens=None,
                      scale: float = 1.0, num_segments: int = 1):
    """gdn_chunk_fwd_noalloc: chunk_fwd with the library's fixed device workspace.

    The caller passes every output (``out`` shaped like v; ``final_state_out``
    (N, H, Dk, Dv) fp32 or None) and the call allocates nothing, so it can run
    where allocation is not allowed (e.g. under HIP graph capture).  Calls on one
    device share the workspace: do not let two of them run concurrently.  With
    ``cu_seqlens``, pass a SeqLens built beforehand (building one allocates)."""
    lib = nat.load()
    _check_inputs(q, k, v, g, beta)
    if cu_seqlens is not None and not isinstance(cu_seqlens, SeqLens):
        raise TypeError("chunk_fwd_noalloc takes cu_seqlens as a prebuilt SeqLens")
    prob = make_problem(q, v, cu_seqlens, scale, num_segments)
    N, H, Dk, Dv = prob.num_seqs, prob.H, prob.Dk, prob.Dv
    S0 = _fp32_state(S0, N, H, Dk, Dv, "S0", q.device)
    _on_device(out, q.device, "out")
    if out is None or out.dtype != v.dtype or out.shape != v.shape or not out.is_contiguous():
        raise ValueError("out must be contiguous, shaped and typed like v")
    Sf = _fp32_state(final_state_out, N, H, Dk, Dv, "final_state_out", q.device)
    st = lib.gdn_chunk_fwd_noalloc(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                   _ptr(S0), _ptr(out), _ptr(Sf), _stream(q.device))
    nat.check(st, "gdn_chunk_fwd_noalloc")
    return out, Sf


def kda_chunk_fwd(q, k, v, g, beta, S0=None, cu_seqlens=None, scale: float = 1.0,
                  output_final_state: bool = True, out=None, final_state_out=None, workspace=None,
                  num_segments: int = 1):
    """Chunked forward pass with one log-decay per key channel: g is fp32 and
    shaped like q.  Returns (o, S_final or None); buffers as for chunk_fwd;
    num_segments > 1 runs the segment split."""
    lib = nat.load()
    _check_inputs(q, k, v, beta, beta)
    if not isinstance(g, torch.Tensor) or g.dtype != torch.float32 or g.shape != q.shape:
        raise ValueError("g must be a float32 tensor shaped like q (one log-decay per key channel)")
    _on_device(g, q.device, "g")
    if not g.is_contiguous():
        raise ValueError("g must be a contiguous GPU tensor")
    seqs = _seqlens(cu_seqlens, q.device)
    prob = make_problem(q, v, seqs, scale, num_segments)
    N, H, Dk, Dv = prob.num_seqs, prob.H, prob.Dk, prob.Dv
    S0 = _fp32_state(S0, N, H, Dk, Dv, "S0", q.device)
    if out is None:
        o = torch.empty_like(v)
    else:
        _on_device(out, q.device, "out")
        if out.dtype != v.dtype or out.shape != v.shape or not out.is_contiguous():
            raise ValueError("out must be contiguous, shaped and typed like v")
        o = out
    if final_state_out is not None:
        Sf = _fp32_state(final_state_out, N, H, Dk, Dv, "final_state_out", q.device)
    elif output_final_state:
        Sf = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=q.device)
    else:
        Sf = None
    if workspace is not None:
        _on_device(workspace, q.device, "workspace")
        if not workspace.is_contiguous():
            raise ValueError("workspace must be contiguous")
        ws, nws = workspace, workspace.numel() * workspace.element_size()
    else:
        ws, nws = _workspace(prob, nat.GDN_PASS_KDA_FWD, q.device)
    st = lib.gdn_kda_chunk_fwd(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                               _ptr(S0), _ptr(o), _ptr(Sf), _ptr(ws), nws, _stream(q.device))
    nat.check(st, "gdn_kda_chunk_fwd")
    return o, Sf


def kda_chunk_bwd(q, k, v, g, beta, dO, S0=None, dS_final=None, cu_seqlens=None,
                  scale: float = 1.0, want_dS0: bool = True):
    """Backward of kda_chunk_fwd (g fp32, shaped like q).  Returns dict dq, dk,
    dv, dg (shaped like g), dbeta, dS0."""
    lib = nat.load()
    _kda_check(q, k, v, g, beta)
    _on_device(dO, q.device, "dO")
    if dO.dtype != v.dtype or dO.shape != v.shape or not dO.is_contiguous():
        raise ValueError("dO must be contiguous, shaped and typed like v")
    seqs = _seqlens(cu_seqlens, q.device)
    prob = make_problem(q, v, seqs, scale, 1)
    N, H, Dk, Dv = prob.num_seqs, prob.H, prob.Dk, prob.Dv
    S0 = _fp32_state(S0, N, H, Dk, Dv, "S0", q.device)
    dS_final = _fp32_state(dS_final, N, H, Dk, Dv, "dS_final", q.device)
    out = {
        "dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v),
        "dg": torch.empty_like(g), "dbeta": torch.empty_like(beta),
        "dS0": torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=q.device) if want_dS0 else None,
    }
    ws, nws = _workspace(prob, nat.GDN_PASS_KDA_BWD, q.device)
    st = lib.gdn_kda_chunk_bwd(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                               _ptr(S0), _ptr(dO), _ptr(dS_final), _ptr(out["dq"]), _ptr(out["dk"]),
                               _ptr(out["dv"]), _ptr(out["dg"]), _ptr(out["dbeta"]), _ptr(out["dS0"]),
                               _ptr(ws), nws, _stream(q.device))
    nat.check(st, "gdn_kda_chunk_bwd")
    return out


def _kda_check(q, k, v, g, beta):
    _check_inputs(q, k, v, beta, beta)
    if not isinstance(g, torch.Tensor) or g.dtype != torch.float32 or g.shape != q.shape:
        raise ValueError("g must be a float32 tensor shaped like q (one log-decay per key channel)")
    _on_device(g, q.device, "g")
    if not g.is_contiguous():
        raise ValueError("g must be a contiguous GPU tensor")


def kda_saved_buffer(q, v, cu_seqlens=None):
    """A uint8 device tensor of the size kda_chunk_fwd_save / kda_chunk_bwd_saved
    need (gdn_workspace_size with GDN_PASS_KDA_SAVED; None if 0 bytes)."""
    seqs = _seqlens(cu_seqlens, q.device)
    return _workspace(make_problem(q, v, seqs, 1.0, 1), nat.GDN_PASS_KDA_SAVED, q.device)[0]


def _kda_saved_arg(saved, q, v, seqs, device):
    if saved is None:
        return _workspace(make_problem(q, v, seqs, 1.0, 1), nat.GDN_PASS_KDA_SAVED, device)
    _on_device(saved, device, "saved")
    if not saved.is_contiguous():
        raise ValueError("saved must be contiguous")
    return saved, saved.numel() * saved.element_size()


def kda_chunk_fwd_save(q, k, v, g, beta, S0=None, cu_seqlens=None, scale: float = 1.0, saved=None):
    """gdn_kda_chunk_fwd_save: the per-channel-decay forward that also keeps what
    the backward needs.  Returns (o, S_final, saved); pass ``saved`` to
    kda_chunk_bwd_saved with the same inputs."""
    lib = nat.load()
    _kda_check(q, k, v, g, beta)
    seqs = _seqlens(cu_seqlens, q.device)
    prob = make_problem(q, v, seqs, scale, 1)
    N, H, Dk, Dv = prob.num_seqs, prob.H, prob.Dk, prob.Dv
    S0 = _fp32_state(S0, N, H, Dk, Dv, "S0", q.device)
    o = torch.empty_like(v)
    Sf = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=q.device)
    sv, nsv = _kda_saved_arg(saved, q, v, seqs, q.device)
    st = lib.gdn_kda_chunk_fwd_save(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                    _ptr(S0), _ptr(o), _ptr(Sf), _ptr(sv), nsv, _stream(q.device))
    nat.check(st, "gdn_kda_chunk_fwd_save")
    return o, Sf, sv


def kda_chunk_bwd_saved(q, k, v, g, beta, dO, saved, dS_final=None, cu_seqlens=None,
                        scale: float = 1.0, want_dS0: bool = True):
    """gdn_kda_chunk_bwd_saved: the per-channel-decay backward from a buffer
    filled by kda_chunk_fwd_save with the same q, k, v, g, beta, S0 and
    cu_seqlens.  Returns dict dq, dk, dv, dg, dbeta, dS0."""
    lib = nat.load()
    _kda_check(q, k, v, g, beta)
    _on_device(dO, q.device, "dO")
    if dO.dtype != v.dtype or dO.shape != v.shape or not dO.is_contiguous():
        raise ValueError("dO must be contiguous, shaped and typed like v")
    if saved is None:
        raise ValueError("saved must be the buffer kda_chunk_fwd_save filled")
    seqs = _seqlens(cu_seqlens, q.device)
    prob = make_problem(q, v, seqs, scale, 1)
    N, H, Dk, Dv = prob.num_seqs, prob.H, prob.Dk, prob.Dv
    dS_final = _fp32_state(dS_final, N, H, Dk, Dv, "dS_final", q.device)
    sv, nsv = _kda_saved_arg(saved, q, v, seqs, q.device)
    out = {
        "dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v),
        "dg": torch.empty_like(g), "dbeta": torch.empty_like(beta),
        "dS0": torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=q.device) if want_dS0 else None,
    }
    st = lib.gdn_kda_chunk_bwd_saved(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                     _ptr(dO), _ptr(dS_final), _ptr(out["dq"]), _ptr(out["dk"]),
                                     _ptr(out["dv"]), _ptr(out["dg"]), _ptr(out["dbeta"]), _ptr(out["dS0"]),
                                     _ptr(sv), nsv, _stream(q.device))
    nat.check(st, "gdn_kda_chunk_bwd_saved")
    return out


def chunk_bwd(q, k, v, g, beta, dO, S0=None, dS_final=None, cu_seqlens=None,
              scale: float = 1.0, want_dS0: bool = True):
    """Chunked backward pass.  Returns dict dq, dk, dv, dg, dbeta, dS0."""
    lib = nat.load()
    _check_inputs(q, k, v, g, beta)
    _on_device(dO, q.device, "dO")
    if dO.dtype != v.dtype or dO.shape != v.shape or not dO.is_contiguous():
        raise ValueError("dO must be contiguous, shaped and typed like v")
    seqs = _seqlens(cu_seqlens, q.device)
    prob = make_problem(q, v, seqs, scale, 1)
    N, H, Dk, Dv = prob.num_seqs, prob.H, prob.Dk, prob.Dv
    S0 = _fp32_state(S0, N, H, Dk, Dv, "S0", q.device)
    dS_final = _fp32_state(dS_final, N, H, Dk, Dv, "dS_final", q.device)
    out = {
        "dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v),
        "dg": torch.empty_like(g), "dbeta": torch.empty_like(beta),
        "dS0": torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=q.device) if want_dS0 else None,
    }
    ws, nws = _workspace(prob, nat.GDN_PASS_CHUNK_BWD, q.device)
    st = lib.gdn_chunk_bwd(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                           _ptr(S0), _ptr(dO), _ptr(dS_final), _ptr(out["dq"]), _ptr(out["dk"]),
                           _ptr(out["dv"]), _ptr(out["dg"]), _ptr(out["dbeta"]), _ptr(out["dS0"]),
                           _ptr(ws), nws, _stream(q.device))
    nat.check(st, "gdn_chunk_bwd")
    return out


def saved_buffer(q, v, cu_seqlens=None):
    """A uint8 device tensor of the size chunk_fwd_save / chunk_bwd_saved need
    (gdn_workspace_size with GDN_PASS_CHUNK_SAVED; None if 0 bytes)."""
    seqs = _seqlens(cu_seqlens, q.device)
    return _workspace(make_problem(q, v, seqs, 1.0, 1), nat.GDN_PASS_CHUNK_SAVED, q.device)[0]


def _saved_arg(saved, q, v, seqs, device):
    if saved is None:
        return _workspace(make_problem(q, v, seqs, 1.0, 1), nat.GDN_PASS_CHUNK_SAVED, device)
    _on_device(saved, device, "saved")
    if not saved.is_contiguous():
        raise ValueError("saved must be contiguous")
    return saved, saved.numel() * saved.element_size()


def chunk_fwd_save(q, k, v, g, beta, S0=None, cu_seqlens=None, scale: float = 1.0, saved=None):
    """gdn_chunk_fwd_save: the chunked forward that also keeps what the backward
    needs.  Returns (o, S_final, saved); pass ``saved`` to chunk_bwd_saved with
    the same inputs."""
    lib = nat.load()
    _check_inputs(q, k, v, g, beta)
    seqs = _seqlens(cu_seqlens, q.device)
    prob = make_problem(q, v, seqs, scale, 1)
    N, H, Dk, Dv = prob.num_seqs, prob.H, prob.Dk, prob.Dv
    S0 = _fp32_state(S0, N, H, Dk, Dv, "S0", q.device)
    o = torch.empty_like(v)
    Sf = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=q.device)
    sv, nsv = _saved_arg(saved, q, v, seqs, q.device)
    st = lib.gdn_chunk_fwd_save(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                _ptr(S0), _ptr(o), _ptr(Sf), _ptr(sv), nsv, _stream(q.device))
    nat.check(st, "gdn_chunk_fwd_save")
    return o, Sf, sv


def chunk_bwd_saved(q, k, v, g, beta, dO, saved, dS_final=None, cu_seqlens=None,
                    scale: float = 1.0, want_dS0: bool = True):
    """gdn_chunk_bwd_saved: the backward from a buffer filled by chunk_fwd_save
    with the same q, k, v, g, beta, S0 and cu_seqlens.  Returns dict dq, dk, dv,
    dg, dbeta, dS0."""
    lib = nat.load()
    _check_inputs(q, k, v, g, beta)
    _on_device(dO, q.device, "dO")
    if dO.dtype != v.dtype or dO.shape != v.shape or not dO.is_contiguous():
        raise ValueError("dO must be contiguous, shaped and typed like v")
    if saved is None:
        raise ValueError("saved must be the buffer chunk_fwd_save filled")
    seqs = _seqlens(cu_seqlens, q.device)
    prob = make_problem(q, v, seqs, scale, 1)
    N, H, Dk, Dv = prob.num_seqs, prob.H, prob.Dk, prob.Dv
    dS_final = _fp32_state(dS_final, N, H, Dk, Dv, "dS_final", q.device)
    sv, nsv = _saved_arg(saved, q, v, seqs, q.device)
    out = {
        "dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v),
        "dg": torch.empty_like(g), "dbeta": torch.empty_like(beta),
        "dS0": torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=q.device) if want_dS0 else None,
    }
    st = lib.gdn_chunk_bwd_saved(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                 _ptr(dO), _ptr(dS_final), _ptr(out["dq"]), _ptr(out["dk"]),
                                 _ptr(out["dv"]), _ptr(out["dg"]), _ptr(out["dbeta"]), _ptr(out["dS0"]),
                                 _ptr(sv), nsv, _stream(q.device))
    nat.check(st, "gdn_chunk_bwd_saved")
    return out


def recurrent_ref(q, k, v, g, beta, S0=None, cu_seqlens=None, scale: float = 1.0, dO=None,
                  dS_final=None, want_dS0: bool = True):
    """fp32 token-loop reference on the GPU.  Returns dict o, S_final (+ gradients if dO)."""
    lib = nat.load()
    _check_inputs(q, k, v, g, beta)
    seqs = _seqlens(cu_seqlens, q.device)
    prob = make_problem(q, v, seqs, scale, 1)
    N, H, Dk, Dv = prob.num_seqs, prob.H, prob.Dk, prob.Dv
    S0 = _fp32_state(S0, N, H, Dk, Dv, "S0", q.device)
    out = {"o": torch.empty_like(v),
           "S_final": torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=q.device)}
    grads = dict.fromkeys(("dq", "dk", "dv", "dg", "dbeta", "dS0"))
    pass_ = nat.GDN_PASS_RECURRENT_FWD
    if dO is not None:
        _on_device(dO, q.device, "dO")
        if dO.dtype != v.dtype or dO.shape != v.shape or not dO.is_contiguous():
            raise ValueError("dO must be contiguous, shaped and typed like v")
        dS_final = _fp32_state(dS_final, N, H, Dk, Dv, "dS_final", q.device)
        grads = {"dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v),
                 "dg": torch.empty_like(g), "dbeta": torch.empty_like(beta),
                 "dS0": torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=q.device)
                 if want_dS0 else None}
        pass_ = nat.GDN_PASS_RECURRENT_BWD
    ws, nws = _workspace(prob, pass_, q.device)
    st = lib.gdn_recurrent_ref(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                               _ptr(S0), _ptr(out["o"]), _ptr(out["S_final"]), _ptr(dO),
                               _ptr(dS_final), _ptr(grads["dq"]), _ptr(grads["dk"]),
                               _ptr(grads["dv"]), _ptr(grads["dg"]), _ptr(grads["dbeta"]),
                               _ptr(grads["dS0"]), _ptr(ws), nws, _stream(q.device))
    nat.check(st, "gdn_recurrent_ref")
    if dO is not None:
        out.update(grads)
    return out


def prologue(q_raw, k_raw, a, b, A_log=None, dt_bias=None, gate: str = "gdn",
             allow_neg_eigval: bool = False, Dv: Optional[int] = None):
    """Fused input prologue (gdn_prologue): L2-normalised q and k (fp32 norms, one
    rounding to the io dtype), g and beta from the raw projections.  Returns
    (q, k, g, beta).  gate: "gdn" (g = -exp(A_log) softplus(a + dt_bias); A_log and
    dt_bias of shape (H,)), "bounded5" (g = -5 sigmoid(a)), or "gdn_channel" (the
    first form per key channel, for kda_chunk_fwd: a and g shaped like q, dt_bias
    (H, Dk))."""
    lib = nat.load()
    if not isinstance(q_raw, torch.Tensor) or not q_raw.is_cuda:
        raise ValueError("q_raw must be a GPU tensor")
    dev = q_raw.device
    for name, t in (("k_raw", k_raw), ("a", a), ("b", b), ("A_log", A_log), ("dt_bias", dt_bias)):
        _on_device(t, dev, name)
    if q_raw.dtype not in _IO or k_raw.dtype != q_raw.dtype:
        raise TypeError("q_raw and k_raw must share the io dtype (bfloat16 or float32)")
    if q_raw.dim() != 4 or k_raw.shape != q_raw.shape or not q_raw.is_contiguous() or not k_raw.is_contiguous():
        raise ValueError("q_raw and k_raw must be contiguous (B, T, H, Dk) tensors of one shape")
    B, T, H, Dk = q_raw.shape
    kind = {"gdn": nat.GDN_GATE_GDN, "bounded5": nat.GDN_GATE_BOUNDED5,
            "gdn_channel": nat.GDN_GATE_GDN_CHANNEL}[gate]
    chan = kind == nat.GDN_GATE_GDN_CHANNEL
    a_shape = (B, T, H, Dk) if chan else (B, T, H)
    for name, t, shape in (("a", a, a_shape), ("b", b, (B, T, H))):
        if t.dtype != torch.float32 or tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 {shape} tensor")
    if kind != nat.GDN_GATE_BOUNDED5:
        for name, t, shape in (("A_log", A_log, (H,)), ("dt_bias", dt_bias, (H, Dk) if chan else (H,))):
            if t is None or t.dtype != torch.float32 or tuple(t.shape) != shape or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous float32 {shape} tensor for gate='{gate}'")
    prob = nat.Problem(B=B, T=T, H=H, Dk=Dk, Dv=Dv if Dv is not None else 16, num_seqs=B,
                       cu_seqlens_host=None, cu_seqlens_dev=None, io_dtype=_IO[q_raw.dtype],
                       scale=1.0, chunk=64, num_segments=1)
    q = torch.empty_like(q_raw)
    k = torch.empty_like(k_raw)
    g = torch.empty(a_shape, dtype=torch.float32, device=q_raw.device)
    beta = torch.empty((B, T, H), dtype=torch.float32, device=q_raw.device)
    st = lib.gdn_prologue(ctypes.byref(prob), _ptr(q_raw), _ptr(k_raw), _ptr(a), _ptr(b), _ptr(A_log),
                          _ptr(dt_bias), kind, int(bool(allow_neg_eigval)), _ptr(q), _ptr(k), _ptr(g),
                          _ptr(beta), _stream(q_raw.device))
    nat.check(st, "gdn_prologue")
    return q, k, g, beta


def epilogue(o, z, weight=None, eps: float = 1e-6):
    """Output epilogue (gdn_epilogue): y = o / sqrt(mean(o^2) + eps) * weight * silu(z)
    per (token, head) over the last dimension.  o, z: (B, T, H, Dv) of the io dtype;
    weight: float32 (Dv,) or None (ones)."""
    lib = nat.load()
    if not isinstance(o, torch.Tensor) or not o.is_cuda:
        raise ValueError("o must be a GPU tensor")
    for name, t in (("z", z), ("weight", weight)):
        _on_device(t, o.device, name)
    if o.dtype not in _IO or z.dtype != o.dtype:
        raise TypeError("o and z must share the io dtype (bfloat16 or float32)")
    if o.dim() != 4 or z.shape != o.shape or not o.is_contiguous() or not z.is_contiguous():
        raise ValueError("o and z must be contiguous (B, T, H, Dv) tensors of one shape")
    B, T, H, Dv = o.shape
    if weight is not None and (weight.dtype != torch.float32 or tuple(weight.shape) != (Dv,)
                               or not weight.is_contiguous()):
        raise ValueError("weight must be a contiguous float32 (Dv,) tensor")
    prob = nat.Problem(B=B, T=T, H=H, Dk=64, Dv=Dv, num_seqs=B, cu_seqlens_host=None, cu_seqlens_dev=None,
                       io_dtype=_IO[o.dtype], scale=1.0, chunk=64, num_segments=1)
    y = torch.empty_like(o)
    st = lib.gdn_epilogue(ctypes.byref(prob), _ptr(o), _ptr(z), _ptr(weight), float(eps), _ptr(y),
                          _stream(o.device))
    nat.check(st, "gdn_epilogue")
    return y


def device_copy(dst, src):
    """gdn_device_copy: copy src into dst (same byte size, device tensors) with the
    library's copy kernel, the HBM roofline calibration."""
    lib = nat.load()
    for name, t in (("dst", dst), ("src", src)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    _on_device(dst, src.device, "dst")
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n:
        raise ValueError("dst and src must have the same size in bytes")
    nat.check(lib.gdn_device_copy(_ptr(dst), _ptr(src), n, _stream(src.device)), "gdn_device_copy")
    return dst
