"""Host-side checks of the seeded input generators (CPU only)."""
import numpy as np
import pytest
import torch

from gated_deltanet_chunked_gdn_amd.workloads import WORKLOADS, generate, round_bf16


def test_round_bf16_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-20, 20, 100000),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0, -0.0], np.float32)])
    x = x.astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(round_bf16(x), ref)


@pytest.mark.parametrize("name", ["tiny_fp32", "packed_bf16"])
def test_generators_are_seeded_and_exact_in_io_dtype(name):
    w = WORKLOADS[name]
    if w.T > 20000:
        w = w.with_(T=4096)
    a, b = generate(w), generate(w)
    for key in ("q", "k", "v", "g", "beta"):
        np.testing.assert_array_equal(a[key], b[key])
    if w.io == "bf16":
        for key in ("q", "k", "v"):
            np.testing.assert_array_equal(round_bf16(a[key]), a[key])
    assert np.all(a["g"] <= 0) and np.all(a["beta"] > 0) and np.all(a["beta"] < 2)
    kn = np.linalg.norm(a["k"].astype(np.float64), axis=-1)
    assert np.allclose(kn, 1.0, atol=1e-2 if w.io == "bf16" else 1e-6)


def test_workload_shapes_follow_the_pages():
    w = WORKLOADS
    assert (w["train_bf16"].B, w["train_bf16"].T, w["train_bf16"].H, w["train_bf16"].Dk) == (4, 4096, 8, 128)
    assert tuple(w["packed_bf16"].cu_seqlens) == (0, 5120, 10240) and w["packed_bf16"].H == 12
    assert (w["long_bf16"].T, w["long_bf16"].H) == (65536, 1)
    assert (w["fwdbwd_bf16"].B, w["fwdbwd_bf16"].T, w["fwdbwd_bf16"].H, w["fwdbwd_bf16"].Dk,
            w["fwdbwd_bf16"].Dv) == (32, 1024, 16, 64, 128)
    small = generate(w["packed_bf16"].with_(T=256, cu_seqlens=(0, 100, 256)))
    assert small["S0"].shape == (2, 12, 128, 128)
    assert abs(float(np.std(small["S0"])) - 0.1) < 0.01
    assert np.all(small["g"] > -5) and np.all(small["g"] < 0)


def test_channel_gate_generator():
    w = WORKLOADS["kda_bf16"]
    assert (w.B, w.T, w.H, w.Dk, w.Dv) == (4, 4096, 8, 128, 128)
    d = generate(w.with_(B=1, T=128))
    assert d["g"].shape == d["q"].shape
    assert np.all(d["g"] < 0) and np.all(np.isfinite(d["g"]))
    # channels of one head differ (dt_bias per channel), heads differ (A_log per head)
    assert np.std(d["g"][0, :, 0, :].mean(axis=0)) > 0.05
