"""Shared helpers of the GPU tests: moving generated inputs to the device and
comparing GPU results with the oracle."""
import numpy as np
import torch

import oracle
from oracle.compare import max_rel, rel_rms, worst_head_rel_rms


def io_torch(io: str):
    return torch.bfloat16 if io == "bf16" else torch.float32


def to_device(d: dict, device="cuda") -> dict:
    """Generated float32 arrays -> device tensors in the io dtype (exact casts)."""
    io = io_torch(d["io"])
    out = {}
    for key in ("q", "k", "v", "dO"):
        if d.get(key) is not None:
            out[key] = torch.from_numpy(d[key]).to(device).to(io).contiguous()
    for key in ("g", "beta", "S0"):
        if d.get(key) is not None:
            out[key] = torch.from_numpy(np.ascontiguousarray(d[key])).to(device)
    return out


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def oracle_fwd(d: dict, scale=None):
    o, Sf = oracle.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu_seqlens"],
                       S0=d["S0"], scale=d["scale"] if scale is None else scale)
    return o.reshape(d["v"].shape), Sf


def truncate(d: dict, T: int) -> dict:
    """The first T tokens of every sequence of a dense workload."""
    if d["cu_seqlens"] is not None:
        raise ValueError("truncate() is for dense workloads")
    out = dict(d)
    for key in ("q", "k", "v", "g", "beta", "dO"):
        if d.get(key) is not None:
            out[key] = np.ascontiguousarray(d[key][:, :T])
    return out


def report(name, **vals):
    print(name, " ".join(f"{k}={v:.3e}" for k, v in vals.items()), flush=True)


__all__ = ["io_torch", "to_device", "to_np", "oracle_fwd", "truncate", "max_rel", "rel_rms", "report",
           "worst_head_rel_rms"]
