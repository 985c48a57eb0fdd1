#!/usr/bin/env python3
"""Throughput of the chunked gated-delta-rule forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload train_bf16]

A step is one gdn_chunk_fwd call (every stage of the forward hot path: cumsum of
g, K K^T and the triangular solve, the WY errors, the state pass, the causal
output and the final state) over one batch of seeded synthetic input already
resident in HBM.  Four independent input/output sets are rotated so that the
256 MB on-package cache cannot hold the working set between steps.  Prints one
JSON line.

Roofline (the forward pass is HBM-bound at this shape: ~134 algorithmic FLOP per
byte, below MI355X's bf16-MFMA/HBM ridge):
  algorithmic bytes per launch = token-heads * ((2 Dk + Dv) + Dv) * s_io + 8
                                 + N H Dk Dv 4 (final state) [+ the same for S0]
  achieved = those bytes / mean kernel duration (HIP events on the launch stream).
The CPU baseline times the fp64 oracle on the host cores (bench-only use).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "chunked GDN fwd tokens/s + % MFMA/HBM roofline (B4 H8 T4096 d128 bf16)"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
CHUNK = 64


def alg_bytes(w, s_io: int) -> int:
    th = w.B * w.T * w.H
    per_th = (2 * w.Dk + w.Dv) * s_io + w.Dv * s_io + 8
    state = w.num_seqs * w.H * w.Dk * w.Dv * 4
    return th * per_th + state * (2 if w.s0_std is not None else 1)


def alg_flops(w) -> float:
    th = w.B * w.T * w.H
    per_th = 6 * w.Dk * w.Dv + 3 * CHUNK * w.Dk + 2 * CHUNK * w.Dv + CHUNK * CHUNK / 3
    return th * per_th


def bwd_alg_bytes(w, s_io: int) -> int:
    """Reads q, k, v, dO, g, beta; writes dq, dk, dv, dg, dbeta; reads S0 and writes dS0."""
    th = w.B * w.T * w.H
    per_th = (2 * w.Dk + 2 * w.Dv) * s_io + 8 + (2 * w.Dk + w.Dv) * s_io + 8
    return th * per_th + 2 * w.num_seqs * w.H * w.Dk * w.Dv * 4


def event_times(call, n_calls, warmup, stream):
    """Per-call durations (s) of `call(i)` from HIP events on `stream`."""
    import torch

    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n_calls)]
    for i in range(n_calls):
        ev[i][0].record(stream)
        call(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in ev]) * 1e-3


EXTRAS = ("bwd", "segment_split", "prologue", "epilogue", "kda", "kda_bwd", "kda_segment_split", "policy")


def extra_measurements(gdn, generate, WORKLOADS, dev, steps, warmup, which=EXTRAS):
    """The other passes, reported beside the headline forward number (not in it):
    backward of the training shape, the segment split of the long sequence, the
    input prologue and output epilogue, and the per-key-channel-decay forward
    (serial and with the segment split)."""
    import torch

    from gated_deltanet_chunked_gdn_amd import _native as nat

    out = {}
    stream = torch.cuda.current_stream(dev)
    if "bwd" in which:
        # backward, B=32 T=1024 H=16 d_k=64 d_v=128
        w = WORKLOADS["fwdbwd_bf16"]
        d = generate(w)
        sets = []
        for _ in range(2):
            t = {key: torch.from_numpy(d[key]).to(dev).to(torch.bfloat16) for key in ("q", "k", "v", "dO")}
            t.update({key: torch.from_numpy(d[key]).to(dev) for key in ("g", "beta", "S0")})
            sets.append(t)

        def bwd(i):
            t = sets[i % len(sets)]
            gdn.chunk_bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["dO"], S0=t["S0"], scale=d["scale"])

        kt = event_times(bwd, steps, warmup, stream)
        nb = bwd_alg_bytes(w, 2)
        out["bwd"] = {"workload": w.name, "ms_mean": float(kt.mean()) * 1e3,
                      "tokens_per_s": w.B * w.T / float(kt.mean()),
                      "alg_bytes_per_launch": nb, "alg_GBps": nb / float(kt.mean()) / 1e9,
                      "kernels": "prep + state (with per-chunk states) + chunk_dstate + chunk_grad"}

        # retained states (the fla issue #1550 page's retain-or-recompute choice): a
        # training step as forward + recomputing backward, against the forward that
        # keeps the backward's records + the backward from them
        def fwd(i):
            t = sets[i % len(sets)]
            gdn.chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], S0=t["S0"], scale=d["scale"])

        saved = [gdn.saved_buffer(t["q"], t["v"]) for t in sets]

        def fsave(i):
            t = sets[i % len(sets)]
            gdn.chunk_fwd_save(t["q"], t["k"], t["v"], t["g"], t["beta"], S0=t["S0"], scale=d["scale"],
                               saved=saved[i % len(sets)])

        def bsaved(i):
            t = sets[i % len(sets)]
            gdn.chunk_bwd_saved(t["q"], t["k"], t["v"], t["g"], t["beta"], t["dO"], saved[i % len(sets)],
                                scale=d["scale"])

        tf = event_times(fwd, steps, warmup, stream)
        ts = event_times(fsave, steps, warmup, stream)  # leaves both buffers filled
        tb = event_times(bsaved, steps, warmup, stream)
        f_ms, s_ms, b_ms = (float(x.mean()) * 1e3 for x in (tf, ts, tb))
        out["bwd"]["recompute"] = {"fwd_ms": f_ms, "bwd_ms": out["bwd"]["ms_mean"],
                                   "step_ms": f_ms + out["bwd"]["ms_mean"]}
        out["bwd"]["retain"] = {"fwd_save_ms": s_ms, "bwd_saved_ms": b_ms, "step_ms": s_ms + b_ms,
                                "saved_bytes": int(saved[0].numel())}
        del sets, saved
    if "segment_split" in which:
        # segment split, B=1 T=65536 H=1 d=128
        w = WORKLOADS["long_bf16"]
        d = generate(w)
        t = {key: torch.from_numpy(d[key]).to(dev).to(torch.bfloat16) for key in ("q", "k", "v")}
        t.update({key: torch.from_numpy(d[key]).to(dev) for key in ("g", "beta")})
        seg = {}
        for G in (1, 2, 4, 8, 16):
            ws = gdn.forward_workspace(t["q"], t["v"], None, G)
            o = torch.empty_like(t["v"])
            Sf = torch.empty((1, 1, w.Dk, w.Dv), dtype=torch.float32, device=dev)

            def fwd(i, G=G, ws=ws, o=o, Sf=Sf):
                gdn.chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], scale=d["scale"], num_segments=G,
                              out=o, final_state_out=Sf, workspace=ws)

            kt = event_times(fwd, max(5, steps // 4), 2, stream)
            seg[str(G)] = {"ms_mean": float(kt.mean()) * 1e3, "tokens_per_s": w.T / float(kt.mean())}
        out["segment_split"] = {"workload": w.name, "by_num_segments": seg}
    if "kda_segment_split" in which:
        # per-key-channel decay, segment split, B=1 T=65536 H=1 d=128 (slow per-channel decay)
        w = WORKLOADS["kda_long_bf16"]
        d = generate(w)
        t = {key: torch.from_numpy(d[key]).to(dev).to(torch.bfloat16) for key in ("q", "k", "v")}
        t.update({key: torch.from_numpy(d[key]).to(dev) for key in ("g", "beta")})
        seg = {}
        for G in (1, 2, 4, 8, 16):
            prob = gdn.make_problem(t["q"], t["v"], None, 1.0, G)
            ws = torch.empty(nat.workspace_size(prob, nat.GDN_PASS_KDA_FWD), dtype=torch.uint8, device=dev)
            o = torch.empty_like(t["v"])
            Sf = torch.empty((1, 1, w.Dk, w.Dv), dtype=torch.float32, device=dev)

            def fwd(i, G=G, ws=ws, o=o, Sf=Sf):
                gdn.kda_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], scale=d["scale"], num_segments=G,
                                  out=o, final_state_out=Sf, workspace=ws)

            kt = event_times(fwd, max(5, steps // 4), 2, stream)
            seg[str(G)] = {"ms_mean": float(kt.mean()) * 1e3, "tokens_per_s": w.T / float(kt.mean())}
        out["kda_segment_split"] = {"workload": w.name, "by_num_segments": seg}
    if "prologue" in which:
        # fused input prologue (normalised q, k; g; beta) on the training shape
        w = WORKLOADS["train_bf16"]
        rng = np.random.default_rng(11)
        shape = (w.B, w.T, w.H, w.Dk)
        qr = torch.from_numpy(rng.standard_normal(shape, dtype=np.float32)).to(dev).to(torch.bfloat16)
        kr = torch.from_numpy(rng.standard_normal(shape, dtype=np.float32)).to(dev).to(torch.bfloat16)
        a = torch.from_numpy(rng.standard_normal(shape[:3], dtype=np.float32)).to(dev)
        b = torch.from_numpy(rng.standard_normal(shape[:3], dtype=np.float32)).to(dev)
        A_log = torch.from_numpy(rng.uniform(0.0, 1.5, size=(w.H,)).astype(np.float32)).to(dev)
        dt = torch.from_numpy((0.5 * rng.standard_normal(w.H)).astype(np.float32)).to(dev)
        kt = event_times(lambda i: gdn.prologue(qr, kr, a, b, A_log, dt), steps, warmup, stream)
        th = w.B * w.T * w.H
        nb = th * (2 * w.Dk * 2 * 2 + 4 * 4)  # q, k read and written (bf16); a, b read, g, beta written
        out["prologue"] = {"workload": w.name, "ms_mean": float(kt.mean()) * 1e3, "bytes_per_launch": nb,
                           "GBps": nb / float(kt.mean()) / 1e9, "frac_of_8TBps": nb / float(kt.mean()) / 8e12}
        del qr, kr
    if "epilogue" in which:
        # output epilogue (RMSNorm(o) * weight * silu(z)) on the training shape
        w = WORKLOADS["train_bf16"]
        rng = np.random.default_rng(12)
        th = w.B * w.T * w.H
        shape = (w.B, w.T, w.H, w.Dv)
        o = torch.from_numpy(rng.standard_normal(shape, dtype=np.float32)).to(dev).to(torch.bfloat16)
        z = torch.from_numpy(rng.standard_normal(shape, dtype=np.float32)).to(dev).to(torch.bfloat16)
        wt = torch.ones(w.Dv, dtype=torch.float32, device=dev)
        kt = event_times(lambda i: gdn.epilogue(o, z, wt), steps, warmup, stream)
        nb = th * w.Dv * 2 * 3  # o, z read, y written (bf16)
        out["epilogue"] = {"workload": w.name, "ms_mean": float(kt.mean()) * 1e3, "bytes_per_launch": nb,
                           "GBps": nb / float(kt.mean()) / 1e9, "frac_of_8TBps": nb / float(kt.mean()) / 8e12}
        del o, z
    if "kda" in which:
        # per-key-channel decay (gdn_kda_chunk_fwd) on the training shape
        w = WORKLOADS["kda_bf16"]
        d = generate(w)
        t = {key: torch.from_numpy(d[key]).to(dev).to(torch.bfloat16) for key in ("q", "k", "v")}
        t.update({key: torch.from_numpy(d[key]).to(dev) for key in ("g", "beta")})
        del d
        o = torch.empty_like(t["v"])
        Sf = torch.empty((w.B, w.H, w.Dk, w.Dv), dtype=torch.float32, device=dev)
        kws = torch.empty(gdn_workspace_bytes(gdn, t["q"], t["v"]), dtype=torch.uint8, device=dev)
        kt = event_times(lambda i: gdn.kda_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], scale=w.scale,
                                                     out=o, final_state_out=Sf, workspace=kws),
                         steps, warmup, stream)
        th = w.B * w.T * w.H
        # q, k, v read and o written (bf16), g (Dk fp32 per token-head) and beta read, S_final written
        nb = th * ((2 * w.Dk + 2 * w.Dv) * 2 + w.Dk * 4 + 4) + w.B * w.H * w.Dk * w.Dv * 4
        out["kda"] = {"workload": w.name, "ms_mean": float(kt.mean()) * 1e3, "tokens_per_s": w.B * w.T / float(kt.mean()),
                      "alg_bytes_per_launch": nb, "alg_GBps": nb / float(kt.mean()) / 1e9,
                      "kernels": "kda_prep_kernel + kda_state_kernel"}
    if "kda_bwd" in which:
        # backward of the per-key-channel-decay pass (gdn_kda_chunk_bwd) on the same shape
        w = WORKLOADS["kda_bf16"]
        d = generate(w)
        t = {key: torch.from_numpy(d[key]).to(dev).to(torch.bfloat16) for key in ("q", "k", "v")}
        t.update({key: torch.from_numpy(d[key]).to(dev) for key in ("g", "beta")})
        del d
        rng = np.random.default_rng(11)
        t["dO"] = torch.from_numpy(rng.standard_normal((w.B, w.T, w.H, w.Dv), dtype=np.float32)).to(dev).to(
            torch.bfloat16)
        kt = event_times(lambda i: gdn.kda_chunk_bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["dO"],
                                                     scale=w.scale, want_dS0=False), steps, warmup, stream)
        th = w.B * w.T * w.H
        # q, k, v, dO read and dq, dk, dv written (bf16); g read and dg written (Dk fp32 per
        # token-head); beta read and dbeta written
        nb = th * ((2 * w.Dk + 2 * w.Dv) * 2 + (2 * w.Dk + w.Dv) * 2 + 2 * (w.Dk * 4 + 4))
        out["kda_bwd"] = {"workload": w.name, "ms_mean": float(kt.mean()) * 1e3,
                          "tokens_per_s": w.B * w.T / float(kt.mean()), "alg_bytes_per_launch": nb,
                          "alg_GBps": nb / float(kt.mean()) / 1e9,
                          "kernels": "kda_prep_kernel + kda_state_kernel (states) + kda_dstate_kernel + kda_grad_kernel"}
        # a training step recomputing the forward's records and states in the
        # backward, against one that keeps them (gdn_kda_chunk_fwd_save /
        # gdn_kda_chunk_bwd_saved)
        f_ms = float(event_times(lambda i: gdn.kda_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"],
                                                             scale=w.scale), steps, warmup, stream).mean()) * 1e3
        saved = gdn.kda_saved_buffer(t["q"], t["v"])
        s_ms = float(event_times(lambda i: gdn.kda_chunk_fwd_save(t["q"], t["k"], t["v"], t["g"], t["beta"],
                                                                  scale=w.scale, saved=saved),
                                 steps, warmup, stream).mean()) * 1e3
        b_ms = float(event_times(lambda i: gdn.kda_chunk_bwd_saved(t["q"], t["k"], t["v"], t["g"], t["beta"], t["dO"],
                                                                   saved, scale=w.scale, want_dS0=False),
                                 steps, warmup, stream).mean()) * 1e3
        out["kda_bwd"]["recompute"] = {"fwd_ms": f_ms, "bwd_ms": out["kda_bwd"]["ms_mean"],
                                       "step_ms": f_ms + out["kda_bwd"]["ms_mean"]}
        out["kda_bwd"]["retain"] = {"fwd_save_ms": s_ms, "bwd_saved_ms": b_ms, "step_ms": s_ms + b_ms,
                                    "saved_bytes": saved.numel()}
        del t, saved
    if "policy" in which:
        # latency, workspace and peak device memory of one forward call per precision
        # policy on the same bf16 inputs (the metric shape, B=4 T=4096 H=8 d=128):
        # "io" (bf16 MFMA operands, fp32 accumulation and state) and "fp32" (every
        # product in IEEE fp32, o rounded to bf16 once); and fp32 io for reference
        w = WORKLOADS["train_bf16"]
        d = generate(w)
        pol = {}
        for name, io, precision in (("bf16_io", torch.bfloat16, "io"), ("bf16_io_fp32_products", torch.bfloat16, "fp32"),
                                    ("fp32_io", torch.float32, "io")):
            t = {key: torch.from_numpy(d[key]).to(dev).to(io) for key in ("q", "k", "v")}
            t.update({key: torch.from_numpy(d[key]).to(dev) for key in ("g", "beta")})
            kt = event_times(lambda i: gdn.chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], scale=w.scale,
                                                     precision=precision),
                             max(5, steps // 2), 2, stream)
            torch.cuda.synchronize()
            torch.cuda.reset_peak_memory_stats(dev)
            base = torch.cuda.memory_allocated(dev)
            o, Sf = gdn.chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], scale=w.scale, precision=precision)
            torch.cuda.synchronize()
            peak = torch.cuda.max_memory_allocated(dev) - base
            ws = gdn.forward_workspace(t["q"], t["v"], precision=precision)
            pol[name] = {"precision": precision, "ms_mean": float(kt.mean()) * 1e3,
                         "tokens_per_s": w.B * w.T / float(kt.mean()),
                         "workspace_bytes": 0 if ws is None else ws.numel(),
                         "peak_call_bytes": int(peak),
                         "input_bytes": int(sum(x.numel() * x.element_size() for x in t.values()))}
            del t, o, Sf, ws
        out["policy"] = {"workload": "train_bf16 (B4 T4096 H8 d128), forward", "by_policy": pol}
    return out


def gdn_workspace_bytes(gdn, q, v):
    """Workspace bytes gdn_kda_chunk_fwd asks for (dense inputs)."""
    from gated_deltanet_chunked_gdn_amd import _native as nat

    return nat.workspace_size(gdn.make_problem(q, v, None, 1.0, 1), nat.GDN_PASS_KDA_FWD)


FWD_KERNEL_SOURCES = ("gated_deltanet_chunked_gdn_amd/csrc/gdn_chunk_fwd.hip",
                      "gated_deltanet_chunked_gdn_amd/csrc/gdn_chunk_chain.hip")


def _source_hashes():
    import hashlib

    return {src: hashlib.sha256(open(os.path.join(ROOT, src), "rb").read()).hexdigest()
            for src in FWD_KERNEL_SOURCES}


def measured_traffic(workload: str):
    """HBM bytes per forward call from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    record, or None when a kernel source has changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"chunk_fwd_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_sources_sha256") != _source_hashes():
        return None
    return rec["traffic_bytes_per_launch"]


def write_traffic_record(fwd_fetch, fwd_write, copy_fetch, copy_write, workload="train_bf16"):
    """Write profiles/chunk_fwd_<workload>_traffic.json from four rocprofv3 --pmc
    counter_collection CSV files: FETCH_SIZE and WRITE_SIZE of a bench.py run, and
    of a `bench.py --micro copy` run (2 GiB read + 2 GiB written, which calibrates
    each counter to bytes).  Counters are in KiB per dispatch."""
    import csv

    def per_kernel(path, counter):
        acc = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in acc.items()}

    copy_bytes = 2 * 1024 ** 3
    cf = [v for k, v in per_kernel(copy_fetch, "FETCH_SIZE").items() if "copy" in k.lower()]
    cw = [v for k, v in per_kernel(copy_write, "WRITE_SIZE").items() if "copy" in k.lower()]
    f_scale = copy_bytes / (max(cf) * 1024)
    w_scale = copy_bytes / (max(cw) * 1024)
    ff = per_kernel(fwd_fetch, "FETCH_SIZE")
    fw = per_kernel(fwd_write, "WRITE_SIZE")
    kernels = sorted(k for k in ff if "gdn::" in k and ("prep" in k or "chain" in k))
    rows = {k.split("(anonymous namespace)::")[-1][:60]: {
        "fetch_KiB": ff[k], "write_KiB": fw.get(k, 0.0),
        "read_bytes": ff[k] * 1024 * f_scale, "written_bytes": fw.get(k, 0.0) * 1024 * w_scale}
        for k in kernels}
    total = sum(r["read_bytes"] + r["written_bytes"] for r in rows.values())
    rec = {"workload": workload, "kernels": rows, "kernel_sources_sha256": _source_hashes(),
           "traffic_bytes_per_launch": int(total), "fetch_size_scale": f_scale,
           "write_size_scale": w_scale, "summary": f"chunk_fwd_{workload}_hbm_traffic.md"}
    out = os.path.join(ROOT, "profiles", f"chunk_fwd_{workload}_traffic.json")
    json.dump(rec, open(out, "w"), indent=1)
    print(json.dumps(rec, indent=1))


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="train_bf16")
    ap.add_argument("--sets", type=int, default=4, help="rotated input/output sets")
    ap.add_argument("--num-segments", type=int, default=1,
                    help="segments per sequence (1: serial over chunks; 2..16: segment split)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the measurements of the other passes")
    ap.add_argument("--extra", choices=EXTRAS, default=None,
                    help="time only this other pass (HIP events) and print its JSON object")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="approximate CPU time budget of the oracle baseline")
    ap.add_argument("--traffic-from", nargs=4, metavar=("FWD_FETCH", "FWD_WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="write the HBM-traffic record from four rocprofv3 --pmc CSV files and exit")
    ap.add_argument("--micro", choices=("copy", "gemm"), default=None,
                    help="run a roofline microbenchmark instead: a 2 GiB device copy "
                         "(bytes counted as read + write) or 8192^3 bf16/fp32 GEMMs")
    return ap.parse_args()


def measure_copy(dev, steps: int, warmup: int, gib: int = 2):
    """A `gib` GiB device copy, timed with HIP events, bytes counted as read plus
    written: torch's copy_ and the library's own copy kernel (gdn_device_copy)."""
    import torch

    import gated_deltanet_chunked_gdn_amd as gdn

    n = gib * 1024 ** 3 // 4
    a = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    res = {"bytes_per_copy": 2 * a.numel() * 4}
    for name, fn in (("torch_copy", lambda: b.copy_(a)), ("hip_copy_kernel", lambda: gdn.device_copy(b, a))):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3 / steps
        res[name] = {"GBps": 2 * a.numel() * 4 / t / 1e9, "frac_of_8TBps": 2 * a.numel() * 4 / t / 8e12,
                     "ms": t * 1e3}
    assert bool((b == 1.0).all()), "copy check"
    res["copy_GBps"] = max(res["torch_copy"]["GBps"], res["hip_copy_kernel"]["GBps"])
    del a, b
    torch.cuda.empty_cache()
    return res


def micro(kind: str, steps: int, warmup: int):
    """Measured peaks, as the Day-2 page measures its GB10 ("Rooflines": a copy of a
    2 GB tensor and (8192, 8192) x (8192, 8192) matmuls).  The library is only run."""
    import torch

    dev = torch.device("cuda:0")
    out = {"micro": kind}
    if kind == "copy":
        out.update(measure_copy(dev, steps, warmup))
    else:
        for dt, peak in ((torch.bfloat16, 2.5e15), (torch.float32, 157.3e12)):
            x = torch.randn(8192, 8192, device=dev).to(dt)
            y = torch.randn(8192, 8192, device=dev).to(dt)
            for _ in range(warmup):
                torch.matmul(x, y)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                torch.matmul(x, y)
            e1.record()
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) * 1e-3 / steps
            fl = 2 * 8192 ** 3 / t
            out[str(dt).split(".")[-1]] = {"TFLOPs": fl / 1e12, "frac_of_peak": fl / peak, "ms": t * 1e3}
    print(json.dumps(out), flush=True)


def cpu_baseline(d, w, budget_s: float):
    """Time the fp64 oracle on the host on the same workload (whole passes,
    repeated until about `budget_s` seconds have passed, at most 500)."""
    import oracle

    threads = oracle.default_threads()
    reps, t_total = 0, 0.0
    while reps < 500 and (reps == 0 or t_total < budget_s):
        t0 = time.perf_counter()
        oracle.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu_seqlens"],
                   S0=d["S0"], scale=d["scale"], nthreads=threads)
        t_total += time.perf_counter() - t0
        reps += 1
    tokens = w.B * w.T * reps
    # one pass on a single thread as well (the oracle's parallel speed-up is printed beside it)
    t0 = time.perf_counter()
    oracle.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu_seqlens"],
               S0=d["S0"], scale=d["scale"], nthreads=1)
    t1 = time.perf_counter() - t0
    return {"value": tokens / t_total, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} full forward pass(es) of workload {w.name} "
                      f"({w.B * w.T} tokens x {w.H} heads each), fp64 C oracle, "
                      f"{t_total:.2f} s total",
            "single_thread_value": w.B * w.T / t1,
            "host_cpu": _host_cpu()}


def _host_cpu() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return f"{line.split(':', 1)[1].strip()}, {os.cpu_count()} logical CPUs visible"
    except OSError:
        pass
    return f"{os.cpu_count()} logical CPUs visible"


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); "
              "this build has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    if args.traffic_from:
        write_traffic_record(*args.traffic_from, workload=args.workload)
        return
    if args.micro:
        micro(args.micro, args.steps, args.warmup)
        return

    import torch

    import gated_deltanet_chunked_gdn_amd as gdn
    from gated_deltanet_chunked_gdn_amd.workloads import WORKLOADS, generate

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.extra:
        dev = torch.device("cuda:0")
        res = extra_measurements(gdn, generate, WORKLOADS, dev, args.steps, args.warmup, (args.extra,))
        print(json.dumps({"extra": args.extra, **res[args.extra]}), flush=True)
        return
    w = WORKLOADS[args.workload]
    d = generate(w)
    io = torch.bfloat16 if w.io == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    print(f"[bench] workload {w.name} generated", file=sys.stderr, flush=True)

    sets = []
    for s in range(args.sets):
        # independent copies (identical values) at distinct addresses
        t = {key: torch.from_numpy(d[key]).to(dev).to(io) for key in ("q", "k", "v")}
        t.update({key: torch.from_numpy(d[key]).to(dev) for key in ("g", "beta")})
        t["S0"] = None if d["S0"] is None else torch.from_numpy(d["S0"]).to(dev)
        t["o"] = torch.empty_like(t["v"])
        t["Sf"] = torch.empty((w.num_seqs, w.H, w.Dk, w.Dv), dtype=torch.float32, device=dev)
        sets.append(t)
    seqs = None if d["cu_seqlens"] is None else gdn.SeqLens(d["cu_seqlens"], dev)
    for t in sets:  # workspaces allocated before the timed region
        t["ws"] = gdn.forward_workspace(t["q"], t["v"], seqs, args.num_segments)

    def step(i):
        t = sets[i % len(sets)]
        gdn.chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], S0=t["S0"], cu_seqlens=seqs,
                      scale=d["scale"], num_segments=args.num_segments, out=t["o"],
                      final_state_out=t["Sf"], workspace=t["ws"])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    print(f"[bench] warmup {args.warmup} done", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kt = np.array([a.elapsed_time(b) for a, b in ev]) * 1e-3  # seconds per launch
    print(f"[bench] timed {args.steps} steps", file=sys.stderr, flush=True)

    s_io = 2 if w.io == "bf16" else 4
    nbytes = alg_bytes(w, s_io)
    flops = alg_flops(w)
    k_mean = float(kt.mean())
    achieved_gbs = nbytes / k_mean / 1e9
    tokens = w.B * w.T
    result = {
        "metric": METRIC,
        "value": tokens * args.steps / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.io,
        "data": "synthetic (seeded numpy generator; random inputs of the named shape)",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "H": w.H, "Dk": w.Dk, "Dv": w.Dv,
                   "chunk": CHUNK, "io": w.io, "state": "fp32", "num_segments": args.num_segments,
                   "packed": d["cu_seqlens"] is not None},
        "roofline": {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved_gbs / HBM_PEAK_GBS,
                     "traffic": measured_traffic(w.name),
                     "kernel": "gdn_chunk_fwd = chunk_prep_kernel + chunk_chain_kernel",
                     "alg_bytes_per_launch": nbytes,
                     "kernel_ms_mean": k_mean * 1e3,
                     "kernel_ms_p10": float(np.percentile(kt, 10)) * 1e3,
                     "kernel_ms_p90": float(np.percentile(kt, 90)) * 1e3},
        "extras": {"alg_tflops": flops / k_mean / 1e12,
                   "alg_flops_per_launch": flops,
                   "mfma_bf16_frac_of_peak": flops / k_mean / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                   "recurrence_tflops_6DkDv": w.B * w.T * w.H * 6 * w.Dk * w.Dv / k_mean / 1e12,
                   "token_heads_per_s": w.B * w.T * w.H / k_mean},
    }
    if not args.no_extras:
        # the attainable copy bandwidth on this machine (2 GiB, read + write counted):
        # the forward's fraction of it is reported beside the fraction of 8 TB/s
        print("[bench] copy ceiling ...", file=sys.stderr, flush=True)
        cp = measure_copy(dev, 10, 3)
        result["roofline"]["measured_copy_GBps"] = cp["copy_GBps"]
        result["roofline"]["frac_of_measured_copy"] = achieved_gbs / cp["copy_GBps"]
        result["extras"]["copy"] = cp
    if not args.no_extras and args.workload == "train_bf16":
        print("[bench] extras: backward, segment split ...", file=sys.stderr, flush=True)
        result["extras"].update(extra_measurements(gdn, generate, WORKLOADS, dev, args.steps,
                                                   args.warmup))
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline ...", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(d, w, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
