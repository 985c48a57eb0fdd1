"""The Python binding refuses host tensors in every pointer slot.

The C ABI sees plain addresses and cannot tell host memory from device memory; a
host pointer that reached a kernel would be a GPU memory fault.  So ops.py checks
the device of every tensor it hands over, and must raise ValueError before any
library call.  The library object is replaced by one whose entry points fail the
test if they are reached.
"""
import pytest
import torch

import gated_deltanet_chunked_gdn_amd.ops as ops
from gated_deltanet_chunked_gdn_amd import _native as nat


class _NoCalls:
    def __getattr__(self, name):
        if name.startswith("gdn_"):
            raise AssertionError(f"library entry point {name} reached before the device checks")
        raise AttributeError(name)


@pytest.fixture()
def no_calls(monkeypatch):
    monkeypatch.setattr(nat, "load", lambda: _NoCalls())


def _inputs(device, B=1, T=64, H=2, D=64):
    q = torch.zeros(B, T, H, D, dtype=torch.bfloat16, device=device)
    g = torch.zeros(B, T, H, dtype=torch.float32, device=device)
    return q, q.clone(), q.clone(), g, g.clone()


def test_host_inputs_rejected(no_calls):
    q, k, v, g, beta = _inputs("cpu")
    with pytest.raises(ValueError):
        ops.chunk_fwd(q, k, v, g, beta)
    with pytest.raises(ValueError):
        ops.chunk_bwd(q, k, v, g, beta, v.clone())
    with pytest.raises(ValueError):
        ops.recurrent_ref(q, k, v, g, beta)
    with pytest.raises(ValueError):
        ops.prologue(q, k, g, beta, A_log=torch.zeros(2), dt_bias=torch.zeros(2))
    with pytest.raises(ValueError):
        ops.epilogue(v, v.clone())
    with pytest.raises(ValueError):
        ops.kda_chunk_fwd(q, k, v, torch.zeros(q.shape), beta)
    with pytest.raises(ValueError):
        ops.kda_chunk_bwd(q, k, v, torch.zeros(q.shape), beta, v.clone())


@pytest.mark.gpu
def test_host_tensor_in_any_slot_rejected(no_calls):
    dev = torch.device("cuda", torch.cuda.current_device())
    q, k, v, g, beta = _inputs(dev)
    S0_host = torch.zeros(1, 2, 64, 64)
    with pytest.raises(ValueError, match="S0"):
        ops.chunk_fwd(q, k, v, g, beta, S0=S0_host)
    with pytest.raises(ValueError, match="S0"):
        ops.kda_chunk_fwd(q, k, v, torch.zeros(q.shape, device=dev), beta, S0=S0_host)
    with pytest.raises(ValueError, match="out"):
        ops.chunk_fwd(q, k, v, g, beta, out=torch.empty(v.shape, dtype=v.dtype))
    with pytest.raises(ValueError, match="final_state_out"):
        ops.chunk_fwd(q, k, v, g, beta, final_state_out=S0_host)
    with pytest.raises(ValueError, match="workspace"):
        ops.chunk_fwd(q, k, v, g, beta, workspace=torch.empty(1 << 20, dtype=torch.uint8))
    with pytest.raises(ValueError, match="dS_final"):
        ops.chunk_bwd(q, k, v, g, beta, v.clone(), dS_final=S0_host)
    with pytest.raises(ValueError, match="dO"):
        ops.chunk_bwd(q, k, v, g, beta, v.cpu())
    with pytest.raises(ValueError, match="beta"):
        ops.chunk_fwd(q, k, v, g, beta.cpu())
    with pytest.raises(ValueError, match="dt_bias"):
        ops.prologue(q, k, g, beta, A_log=torch.zeros(2, device=dev), dt_bias=torch.zeros(2))
    with pytest.raises(ValueError, match="A_log"):
        ops.prologue(q, k, g, beta, A_log=torch.zeros(2), dt_bias=torch.zeros(2, device=dev))
    with pytest.raises(ValueError, match="weight"):
        ops.epilogue(v, v.clone(), weight=torch.ones(64))
    with pytest.raises(ValueError, match="z"):
        ops.epilogue(v, v.cpu())
    gk = torch.zeros(q.shape, device=dev)
    with pytest.raises(ValueError, match="g"):
        ops.kda_chunk_bwd(q, k, v, gk.cpu(), beta, v.clone())
    with pytest.raises(ValueError, match="dO"):
        ops.kda_chunk_bwd(q, k, v, gk, beta, v.cpu())
    with pytest.raises(ValueError, match="S0"):
        ops.kda_chunk_bwd(q, k, v, gk, beta, v.clone(), S0=S0_host)
    with pytest.raises(ValueError, match="dS_final"):
        ops.kda_chunk_bwd(q, k, v, gk, beta, v.clone(), dS_final=S0_host)
