"""GPU parity of the output epilogue (gdn_epilogue) against the oracle's float64
epilogue, through the C ABI (marked gpu).  y is one rounding of an fp32 result:
each element within 2^-8 (bf16) or 2e-6 (fp32) of the float64 value relative to
the row's largest |y| (an elementwise relative bound is unbounded where silu(z)
crosses zero).
"""
import numpy as np
import pytest
import torch

import gated_deltanet_chunked_gdn_amd as gdn
import oracle
from gated_deltanet_chunked_gdn_amd.workloads import round_bf16
from _helpers import report

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B,T,H,Dv,io,weighted,eps", [
    (1, 1, 1, 16, "bf16", False, 1e-6),
    (2, 77, 3, 128, "bf16", True, 1e-6),
    (1, 300, 5, 256, "bf16", True, 1e-5),
    (3, 65, 2, 64, "fp32", True, 1e-6),
    (1, 129, 4, 32, "fp32", False, 0.0),
    (4, 4096, 8, 128, "bf16", True, 1e-6),
])
def test_epilogue_matches_oracle(B, T, H, Dv, io, weighted, eps):
    rng = np.random.default_rng(B * 100 + T)
    o = rng.standard_normal((B, T, H, Dv), dtype=np.float32) * np.float32(0.3)
    z = rng.standard_normal((B, T, H, Dv), dtype=np.float32) * np.float32(2.0)
    if io == "bf16":
        o, z = round_bf16(o), round_bf16(z)
    w = rng.uniform(0.5, 1.5, size=Dv).astype(np.float32) if weighted else None
    dt = torch.bfloat16 if io == "bf16" else torch.float32
    y = gdn.epilogue(torch.from_numpy(o).cuda().to(dt), torch.from_numpy(z).cuda().to(dt),
                     None if w is None else torch.from_numpy(w).cuda(), eps=eps)
    torch.cuda.synchronize()
    ref = oracle.epilogue(o, z, w, eps=eps)
    x = y.float().cpu().numpy().astype(np.float64)
    rowmax = np.max(np.abs(ref), axis=-1, keepdims=True)
    err = np.max(np.abs(x - ref) / np.maximum(rowmax, 1e-30))
    report(f"epilogue {io} Dv={Dv}", max_err_rel_row=err)
    assert err <= (2.0 ** -8 if io == "bf16" else 2e-6)
