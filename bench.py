#!/usr/bin/env python3
"""Benchmark of the selective-scan hot path on one MI355X.

A step is one forward + backward pass (every hot-path kernel) over one batch
of seeded synthetic inputs.  The headline workload is the Mamba-layer-shaped
selective scan B=8 D=2048 N=16 L=4096 with bf16 streams, fp32 state and
accumulation, chunk length 256; value = B*D*N*L / (time of forward+backward).

Inputs are resident in HBM before timing.  The timed region is K steps
bracketed by torch.cuda.synchronize(); per-kernel durations come from HIP
events the library records around each of its launches on the same stream
(ssm_profile_begin / ssm_profile_end), in a separate pass after the timed one.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-others]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # MI355X HBM3E, bytes/s
METRIC = "scan elements/s (B·D·N·L) fwd+bwd at 1 GPU; % of HBM peak BW"
# Vector ALU peak with packed fp32 disabled: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz
VALU_PEAK_OPS = 256 * 4 * 16 * 2.4e9


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-others", action="store_true", help="skip the secondary workloads")
    ap.add_argument("--cpu-batches", type=int, default=8, help="batch rows of the headline workload in the CPU sample")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# per-kernel timing through the library's event hook
# ---------------------------------------------------------------------------
def profile_kernels(fn, reps=5, cap=4096):
    import torch
    from selective_state_space_chunked_amd import lib
    L = lib()
    L.ssm_profile_begin.argtypes = [ctypes.c_int]
    L.ssm_profile_end.argtypes = [ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_float),
                                  ctypes.POINTER(ctypes.c_char_p), ctypes.c_int]
    torch.cuda.synchronize()
    assert L.ssm_profile_begin(cap) == 0
    for _ in range(reps):
        fn()
    n = ctypes.c_int(0)
    ms = (ctypes.c_float * cap)()
    names = (ctypes.c_char_p * cap)()
    assert L.ssm_profile_end(ctypes.byref(n), ms, names, cap) == 0
    agg = {}
    for i in range(n.value):
        k = names[i].decode()
        agg.setdefault(k, []).append(ms[i])
    return {k: (sum(v) / len(v), len(v) // reps) for k, v in agg.items()}


def time_steps(step, steps, warmup):
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps * 1e3


def to_dev(arr, bf16=False):
    import torch
    if bf16:
        return torch.from_numpy(arr.astype(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------
def real_workload(name, shape, dtype, steps, warmup):
    """Selective real scan, forward + backward (gradients w.r.t. delta, x, B, C)."""
    import synth
    import selective_state_space_chunked_amd as ssm
    B, D, N, L = shape["B"], shape["D"], shape["N"], shape["L"]
    cfg = synth.make_real(B=B, D=D, N=N, L=L, dtype=dtype, seed=0)
    bf = dtype == "bf16"
    t = {k: to_dev(cfg[k], bf) for k in ("delta", "x", "Bm", "C")}
    t["A"] = to_dev(cfg["A"])
    gy = to_dev(cfg["gy"], bf)
    es = 2 if bf else 4
    fwd_out = ssm.scan_fwd(ssm.SSM_REAL_SELECTIVE, want_ckpt=True, **t)
    grads = ssm.scan_bwd(ssm.SSM_REAL_SELECTIVE, gy=gy, ckpt=fwd_out["ckpt"], want=("gdelta", "gx", "gBm", "gC"), **t)

    def step():
        ssm.scan_fwd(ssm.SSM_REAL_SELECTIVE, want_ckpt=True, out=fwd_out, **t)
        ssm.scan_bwd(ssm.SSM_REAL_SELECTIVE, gy=gy, ckpt=fwd_out["ckpt"], want=("gdelta", "gx", "gBm", "gC"),
                     out=grads, **t)

    ms = time_steps(step, steps, warmup)
    kern = profile_kernels(step)
    nc = -(-L // 256)
    BDL, BLN = B * D * L, B * L * N
    ck = B * D * nc * N * 4
    fwd_bytes = 2 * BDL * es + 2 * BLN * es + D * N * 4 + BDL * es + ck
    bwd_kernel_bytes = 3 * BDL * es + 2 * BLN * es + D * N * 4 + ck + 2 * BDL * es
    bwd_bytes = bwd_kernel_bytes + 2 * BLN * es
    return dict(name=name, elements=B * D * N * L, ms=ms, kernels=kern,
                bytes=dict(total=fwd_bytes + bwd_bytes, fwd=fwd_bytes, bwd=bwd_bytes,
                           per_kernel={"selective forward": fwd_bytes, "selective backward": bwd_kernel_bytes}),
                config=dict(B=B, D=D, N=N, L=L, streams=dtype, chunk_len=256), inputs=cfg)


def impulse_workload(steps, warmup):
    """Impulse response + full sensitivity, B=1 D=1024 N=16 L=128000 fp32."""
    import synth
    import selective_state_space_chunked_amd as ssm
    cfg = synth.make_impulse(B=1, D=1024, N=16, L=128000, seed=0)
    t = {k: to_dev(cfg[k]) for k in ("delta", "x", "Bm", "C", "A")}
    out = ssm.impulse_sensitivity(**t)

    def step():
        ssm.impulse_sensitivity(out=out, **t)

    ms = time_steps(step, max(3, steps // 4), max(1, warmup // 2))
    BDL, BLN = 1024 * 128000, 128000 * 16
    byts = 2 * BDL * 4 + 2 * BLN * 4 + BDL * 4 + (BDL * 4 + BLN * 4 + BDL * 4)
    return dict(name="impulse", elements=BDL * 16, ms=ms, kernels=profile_kernels(step, reps=2),
                bytes=dict(total=byts), config=dict(B=1, D=1024, N=16, L=128000, streams="f32"))


def summarize(w):
    ms = w["ms"]
    r = dict(el_per_s=w["elements"] / (ms * 1e-3), ms_per_step=ms,
             hbm_frac=w["bytes"]["total"] / (ms * 1e-3) / HBM_PEAK, config=w["config"],
             kernels_ms={k: round(v[0], 4) for k, v in w["kernels"].items()})
    return r


def cpu_baseline(inputs, batches):
    """fp64 oracle (forward + backward) on the first `batches` batch rows of the headline inputs."""
    import oracle
    D, L, N = inputs["D"], inputs["L"], inputs["N"]
    nb = max(1, min(batches, inputs["B"]))
    kw = dict(delta=inputs["delta"][:nb], x=inputs["x"][:nb], A=inputs["A"], Bm=inputs["Bm"][:nb],
              C=inputs["C"][:nb], B=nb, D=D, L=L, N=N)
    t0 = time.perf_counter()
    oracle.real_fwd(**kw)
    oracle.real_bwd(**kw, gy=inputs["gy"][:nb])
    dt = time.perf_counter() - t0
    el = nb * D * L * N
    return {"value": el / dt, "unit": "elements/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": f"batch rows 0..{nb - 1} of the headline workload (B={nb} D={D} N={N} L={L}), "
                      f"forward + backward in fp64, {dt:.1f} s wall"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: the scan is "
              "independent per sequence and no multi-GPU path is built", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    head = real_workload("real-mamba", dict(B=8, D=2048, N=16, L=4096), "bf16", args.steps, args.warmup)
    s = summarize(head)
    kern = head["kernels"]
    # dominant kernel by time
    dom = max(kern, key=lambda k: kern[k][0] * kern[k][1])
    dur = kern[dom][0] * 1e-3
    byts = head["bytes"]["per_kernel"].get(dom)
    roof = {"kernel": dom, "bound": "hbm", "achieved": byts / dur / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
            "frac": byts / dur / HBM_PEAK, "traffic": None, "duration_ms": kern[dom][0]}
    others = {}
    if not args.no_others:
        others["impulse"] = summarize(impulse_workload(args.steps, args.warmup))
        small = real_workload("real-small", dict(B=1, D=16, N=16, L=1024), "f32", args.steps, args.warmup)
        others["real-small"] = summarize(small)
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(head["inputs"], args.cpu_batches)
    line = {
        "metric": METRIC, "value": s["el_per_s"], "unit": "elements/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": s["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "real-mamba: selective scan fwd+bwd, B=8 D=2048 N=16 L=4096, bf16 streams, "
                               "fp32 state, chunk 256", **head["config"]},
        "hbm_frac": s["hbm_frac"], "algorithmic_bytes_per_step": head["bytes"]["total"],
        "kernels_ms": s["kernels_ms"], "roofline": roof, "cpu_baseline": cpu, "others": others,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
