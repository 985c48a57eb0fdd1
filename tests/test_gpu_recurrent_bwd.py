"""GPU parity of the fp32 recurrent reference's reverse mode against the oracle's
fp64 reverse mode (marked gpu)."""
import numpy as np
import pytest
import torch

import gated_deltanet_chunked_gdn_amd as gdn
import oracle
from gated_deltanet_chunked_gdn_amd.workloads import WORKLOADS, Workload, generate
from _helpers import max_rel, rel_rms, report, to_device, to_np, truncate

pytestmark = pytest.mark.gpu

GRADS = ("dq", "dk", "dv", "dg", "dbeta", "dS0")


def run_both(d, dS_final=None):
    t = to_device(d)
    dSf_t = None if dS_final is None else torch.from_numpy(dS_final).cuda()
    out = gdn.recurrent_ref(t["q"], t["k"], t["v"], t["g"], t["beta"], S0=t.get("S0"),
                            cu_seqlens=d["cu_seqlens"], scale=d["scale"], dO=t["dO"],
                            dS_final=dSf_t)
    torch.cuda.synchronize()
    ref = oracle.bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["dO"], cu_seqlens=d["cu_seqlens"],
                     S0=d["S0"], dS_final=dS_final, scale=d["scale"])
    return out, ref


@pytest.mark.parametrize("packed", [False, True])
def test_recurrent_backward_fp32(packed):
    cu = (0, 40, 40, 100) if packed else None
    w = Workload("rb", 1 if packed else 2, 100, 2, 64, 48, io="fp32", qk="norm_both", gate="gdn",
                 cu_seqlens=cu, s0_std=0.3, with_dO=True, scale=0.4, seed=9)
    d = generate(w)
    N = w.num_seqs
    dSf = np.random.default_rng(1).standard_normal((N, 2, 64, 48)).astype(np.float32)
    out, ref = run_both(d, dSf)
    for name in GRADS:
        e = max_rel(to_np(out[name]), ref[name].reshape(out[name].shape))
        report(f"recurrent bwd fp32 {name}", max_rel=e)
        assert e <= 3e-4, name


def test_recurrent_backward_bf16_training_slice():
    """The value-expansion-2 training shape (B=32, T=1024, H=16, d_k=64, d_v=128)
    on its first 256 tokens."""
    d = truncate(generate(WORKLOADS["fwdbwd_bf16"]), 256)
    out, ref = run_both(d)
    for name in GRADS:
        e = rel_rms(to_np(out[name]), ref[name].reshape(out[name].shape))
        report(f"recurrent bwd bf16 {name}", rel_rms=e)
        assert e <= 8e-3, name
