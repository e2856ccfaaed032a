#!/usr/bin/env python3
"""Benchmark of the selective-scan hot path on one MI355X.

A step is one forward + backward pass (every hot-path kernel) over one batch
of seeded synthetic inputs.  The headline workload is the Mamba-layer-shaped
selective scan B=8 D=2048 N=16 L=4096 with bf16 streams, fp32 state and
accumulation, chunk length 256; value = B*D*N*L / (time of forward+backward).
The other workloads (impulse sensitivity at L=128000, with and without the
step-size sensitivity, 16 rows of the input Jacobian at that length, complex
shared-control scan and its forward-mode gradients, complex scan with given
transitions, PD scan with and without
the straight-through selection gradient, dense-a/b scan at the Mamba-layer
shape, the small fp32 case) are reported under "others" with the same fields.

Inputs are resident in HBM before timing.  The timed region is K steps
bracketed by torch.cuda.synchronize(); per-kernel durations come from HIP
events the library records around each of its launches on the same stream
(ssm_profile_begin / ssm_profile_end), in a separate pass after the timed one.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
                       [--no-others | --workloads a,b,...] [--calib-copy]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12  # MI355X HBM3E, bytes/s
# fp32 vector peak: 256 CUs x 4 SIMDs x 32 lanes per cycle x 2 flops (FMA) x 2.4 GHz = 157.3 TFLOP/s.
# Non-packed v_fma_f32 / v_mul_f32 issue a wave64 in two cycles on gfx950 (measured), so this peak
# holds with packed fp32 disabled; v_exp_f32 issues at a quarter of that rate.
VALU_F32_PEAK = 256 * 4 * 32 * 2 * 2.4e9
METRIC = "scan elements/s (B·D·N·L) fwd+bwd at 1 GPU; % of HBM peak BW"
HEADLINE = "real-mamba"

# Algorithmic flops per scan element (the recurrence's arithmetic, exp counted
# as one operation, fused multiply-add as two):
#   forward:  delta*A, exp, (delta x)*B, a*h + b, y += C*h                      = 7
#   backward: recompute (delta*A, exp, (delta x)*B, a*h + b)                   = 5
#             lambda = C*gy + nu, nu = a*lambda                                 = 3
#             gdelta += A*lambda*(a*h_prev), gx term += lambda*B                = 5
#             gB += lambda*(delta x), gC += gy*h (products + channel sums)      = 4   -> 17
FLOPS_PER_ELEMENT = {"selective forward": 7, "selective backward": 17}

# HBM bytes per launch of the dominant kernel, measured with rocprofv3 --pmc
# FETCH_SIZE and --pmc WRITE_SIZE and scaled by what the same counters read for
# a 1 GiB device copy (reads x2.0, writes x1.0), and its VALU occupancy.  Kept with the SHA-256 of the
# kernel sources they were measured on and reported only while those are
# unchanged (profiles/selective_mamba_layer_fwd_bwd.md holds the run).
MEASURED_TRAFFIC = {
    "selective backward": {"read_bytes": 465.8e6, "written_bytes": 540.6e6,
                           # SQ_ACTIVE_INST_VALU x 4 cycles over 1024 SIMD x kernel cycles, and cycles per
                           # VALU instruction (profiles/selective_headline_counters.md)
                           "valu_busy": 0.82, "cycles_per_valu_instr": 4.45,
                           # per-class instruction counts x the issue-rate probes' cycles per class, over the
                           # kernel's cycles; and the fraction of wave cycles waiting at barriers
                           # (SQ_WAIT_ANY - SQ_WAIT_INST_ANY over SQ_WAVE_CYCLES)
                           "issue_model_frac": 0.59, "barrier_wait_frac": 0.13,
                           "sources_sha256": "7aa15ddc9a2c187eaec9312f3f124733b42098951f21341c6748b94e9487cf73"},
}
# (file, hashed spans as (start marker, end marker); None = start / end of the file)
TRAFFIC_SOURCES = (("selective.hpp", ((None, "// forward (SUMMARY"), ("// backward.  Reverse over the tiles", None))),
                   ("real_selective.hip", ((None, "// segment combines"),)), ("common.hpp", ((None, None),)))


def kernel_sources_sha256():
    """SHA-256 of what the selective backward is built from: the kernel header's helpers and backward kernel
    (not its forward kernel), the part of its translation unit before the segment combines, the shared device
    helpers and its parameter struct (later kernels in that file and the other modes' structs in kernels.hpp do
    not change it)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "selective_state_space_chunked_amd", "csrc")
    for f, spans in TRAFFIC_SOURCES:
        text = open(os.path.join(csrc, f)).read()
        for start, end in spans:
            a = text.index(start) if start else 0
            h.update(text[a:text.index(end, a) if end else len(text)].encode())
    hdr = open(os.path.join(csrc, "kernels.hpp")).read()
    for struct in ("struct StepXform {", "struct SelBwdParams {"):
        i = hdr.index(struct)
        h.update(hdr[i:hdr.index("};", i)].encode())
    return h.hexdigest()


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-others", action="store_true", help="only the headline workload")
    ap.add_argument("--workloads", default="", help="comma list of secondary workloads to run")
    ap.add_argument("--cpu-batches", type=int, default=8, help="batch rows of the headline in the CPU sample")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one 1 GiB device copy (calibrates HBM byte counters)")
    ap.add_argument("--no-roof", action="store_true",
                    help="skip the issue-rate probes of each VALU instruction class (ssm_roof_probe) at 1, 2, 4 "
                         "and 8 waves per SIMD, whose measured fp32 FMA ceiling the line reports by default")
    ap.add_argument("--roof", action="store_true", help=argparse.SUPPRESS)   # the default; kept for old commands
    return ap.parse_args()


# ---------------------------------------------------------------------------
# timing helpers
# ---------------------------------------------------------------------------
def profile_kernels(fn, reps=5, cap=8192):
    """Average duration (ms) and launches per call of every kernel fn enqueues."""
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
        agg.setdefault(names[i].decode(), []).append(ms[i])
    return {k: (sum(v) / len(v), len(v) / reps) for k, v in agg.items()}


def time_steps(step, steps, warmup):
    import gc
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # no garbage-collection pause of the interpreter inside the timed region
    gc.collect()
    gc.disable()
    try:
        t0 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    finally:
        gc.enable()
    return (t1 - t0) / steps * 1e3


def to_dev(arr, bf16=False):
    import torch
    if bf16:
        return torch.from_numpy(arr.astype(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


# ---------------------------------------------------------------------------
# workloads: each returns elements, ms per step, kernel times, algorithmic bytes
# ---------------------------------------------------------------------------
def w_real(name, B, D, N, L, dtype, steps, warmup, keep_inputs=False):
    """Selective real scan forward + backward (gradients w.r.t. delta, x, B, C)."""
    import synth
    import selective_state_space_chunked_amd as ssm
    cfg = synth.make_real(B=B, D=D, N=N, L=L, dtype=dtype, seed=0)
    bf = dtype == "bf16"
    t = {k: to_dev(cfg[k], bf) for k in ("delta", "x", "Bm", "C")}
    t["A"] = to_dev(cfg["A"])
    gy = to_dev(cfg["gy"], bf)
    want = ("gdelta", "gx", "gBm", "gC")
    fo = ssm.scan_fwd(ssm.SSM_REAL_SELECTIVE, want_ckpt=True, **t)
    go = ssm.scan_bwd(ssm.SSM_REAL_SELECTIVE, gy=gy, ckpt=fo["ckpt"], want=want, **t)

    def step():
        ssm.scan_fwd(ssm.SSM_REAL_SELECTIVE, want_ckpt=True, out=fo, **t)
        ssm.scan_bwd(ssm.SSM_REAL_SELECTIVE, gy=gy, ckpt=fo["ckpt"], want=want, out=go, **t)

    ms = time_steps(step, steps, warmup)
    es = 2 if bf else 4
    nc = -(-L // 256)
    BDL, BLN, ck = B * D * L, B * L * N, B * D * nc * N * 4
    fwd = 3 * BDL * es + 2 * BLN * es + D * N * 4 + ck            # read delta, x, B, C, A; write y, ckpt
    bwd_k = 5 * BDL * es + 2 * BLN * es + D * N * 4 + ck          # read delta, x, gy, B, C, A, ckpt; write gdelta, gx
    bwd = bwd_k + 2 * BLN * es                                    # + write gB, gC
    return dict(name=name, elements=B * D * N * L, ms=ms, kernels=profile_kernels(step),
                bytes_total=fwd + bwd, bytes_kernel={"selective forward": fwd, "selective backward": bwd_k},
                config=dict(B=B, D=D, N=N, L=L, streams=dtype, chunk_len=256),
                inputs=cfg if keep_inputs else None, step=step)


def w_impulse(steps, warmup):
    """Impulse response y and sensitivity dy[L-1]/dx[t], B=1 D=1024 N=16 L=128000 fp32."""
    import synth
    import selective_state_space_chunked_amd as ssm
    B, D, N, L = 1, 1024, 16, 128000
    cfg = synth.make_impulse(B=B, D=D, N=N, L=L, seed=0)
    t = {k: to_dev(cfg[k]) for k in ("delta", "x", "Bm", "C", "A")}
    out = ssm.impulse_sensitivity(**t)

    def step():
        ssm.impulse_sensitivity(out=out, **t)

    ms = time_steps(step, max(3, steps // 4), max(1, warmup // 2))
    BDL, BLN = B * D * L, B * L * N
    byts = (2 * BDL + 2 * BLN + BDL) * 4 + (BDL + BLN + BDL) * 4  # forward: x, delta, B, C -> y; sens: delta, B -> s
    return dict(name="impulse", elements=BDL * N, ms=ms, kernels=profile_kernels(step, reps=2),
                bytes_total=byts, config=dict(B=B, D=D, N=N, L=L, streams="f32", t_out=L - 1))


def w_sens_rows(steps, warmup):
    """The last 16 rows of the input Jacobian, dy[t]/dx for t = L-16 .. L-1, on the impulse workload,
    B=1 D=1024 N=16 L=128000 fp32."""
    import synth
    import selective_state_space_chunked_amd as ssm
    B, D, N, L, R = 1, 1024, 16, 128000, 16
    cfg = synth.make_impulse(B=B, D=D, N=N, L=L, seed=0)
    t = {k: to_dev(cfg[k]) for k in ("delta", "x", "Bm", "C", "A")}
    s = ssm.sensitivity_rows(t_out0=L - R, rows=R, **t)

    def step():
        ssm.sensitivity_rows(t_out0=L - R, rows=R, out=s, **t)

    ms = time_steps(step, max(3, steps // 4), max(1, warmup // 2))
    BDL, BLN = B * D * L, B * L * N
    byts = (BDL + BLN) * 4 + R * BDL * 4   # read delta, B; write R rows of s
    return dict(name="sens-rows", elements=R * BDL * N, ms=ms, kernels=profile_kernels(step, reps=2),
                bytes_total=byts, config=dict(B=B, D=D, N=N, L=L, rows=R, streams="f32", t_out0=L - R),
                note=f"elements counts every output row: {R} rows x B*D*N*L, so el_per_s is not comparable "
                     "with the single-output workloads")


def w_output_sens(steps, warmup):
    """y and dy[L-1]/dx[t], dy[L-1]/ddelta[t] on the impulse workload, B=1 D=1024 N=16 L=128000 fp32."""
    import synth
    import selective_state_space_chunked_amd as ssm
    B, D, N, L = 1, 1024, 16, 128000
    cfg = synth.make_impulse(B=B, D=D, N=N, L=L, seed=0)
    t = {k: to_dev(cfg[k]) for k in ("delta", "x", "Bm", "C", "A")}
    out = ssm.output_sensitivity(want_y=True, **t)

    def step():
        ssm.output_sensitivity(want_y=True, out=out, **t)

    ms = time_steps(step, max(3, steps // 4), max(1, warmup // 2))
    BDL, BLN = B * D * L, B * L * N
    ck = B * D * (-(-L // 256)) * N * 4
    # forward: x, delta, B, C -> y, checkpoints; sensitivities: delta, x, B, checkpoints -> s_x, s_delta
    byts = (2 * BDL + 2 * BLN + BDL) * 4 + ck + (2 * BDL + BLN + 2 * BDL) * 4 + ck
    return dict(name="output-sens", elements=BDL * N, ms=ms, kernels=profile_kernels(step, reps=2),
                bytes_total=byts, config=dict(B=B, D=D, N=N, L=L, streams="f32", t_out=L - 1))


def w_complex(steps, warmup):
    """Complex shared-control scan, B=16 H=8 M=64 L=2048, forward + backward."""
    import synth
    import selective_state_space_chunked_amd as ssm
    B, H, M, L = 16, 8, 64, 2048
    cfg = synth.make_complex(B=B, H=H, M=M, L=L, seed=0)
    t = {k: to_dev(cfg[k]) for k in ("r", "phi", "lam", "theta", "u", "c")}
    gy = to_dev(cfg["gy"])
    fo = ssm.scan_fwd(ssm.SSM_COMPLEX_SHARED, want_ckpt=True, **t)
    go = ssm.scan_bwd(ssm.SSM_COMPLEX_SHARED, gy=gy, ckpt=fo["ckpt"], **t)

    def step():
        ssm.scan_fwd(ssm.SSM_COMPLEX_SHARED, want_ckpt=True, out=fo, **t)
        ssm.scan_bwd(ssm.SSM_COMPLEX_SHARED, gy=gy, ckpt=fo["ckpt"], out=go, **t)

    ms = time_steps(step, steps, warmup)
    BHL, E = B * H * L, B * H * L * M
    ck = B * H * (-(-L // 32)) * M * 8
    fwd = E * 8 + 2 * BHL * 4 + BHL * 4 + ck                       # read u, r, phi; write y, ckpt
    bwd = E * 8 + 3 * BHL * 4 + ck + E * 8 + 2 * BHL * 4            # read u, r, phi, gy, ckpt; write gu, gr, gphi
    return dict(name="complex", elements=E, ms=ms, kernels=profile_kernels(step), bytes_total=fwd + bwd,
                config=dict(B=B, H=H, M=M, L=L, streams="complex64", chunk_len=32))


def w_complex_dense(steps, warmup):
    """Complex scan with given transitions, B=16 H=8 M=64 L=2048, forward + backward."""
    import synth
    import selective_state_space_chunked_amd as ssm
    B, H, M, L = 16, 8, 64, 2048
    cfg = synth.make_complex_dense(B=B, H=H, M=M, L=L, seed=0)
    t = {k: to_dev(cfg[k]) for k in ("a", "u", "c")}
    gy = to_dev(cfg["gy"])
    fo = ssm.scan_fwd(ssm.SSM_COMPLEX_DENSE, want_ckpt=True, **t)
    go = ssm.scan_bwd(ssm.SSM_COMPLEX_DENSE, gy=gy, ckpt=fo["ckpt"], **t)

    def step():
        ssm.scan_fwd(ssm.SSM_COMPLEX_DENSE, want_ckpt=True, out=fo, **t)
        ssm.scan_bwd(ssm.SSM_COMPLEX_DENSE, gy=gy, ckpt=fo["ckpt"], out=go, **t)

    ms = time_steps(step, steps, warmup)
    BHL, E = B * H * L, B * H * L * M
    ck = B * H * (-(-L // 32)) * M * 8
    fwd = 2 * E * 8 + BHL * 4 + ck                                  # read a, u; write y, ckpt
    bwd = 2 * E * 8 + BHL * 4 + ck + 2 * E * 8                      # read a, u, gy, ckpt; write ga, gu
    return dict(name="complex-dense", elements=E, ms=ms, kernels=profile_kernels(step), bytes_total=fwd + bwd,
                config=dict(B=B, H=H, M=M, L=L, streams="complex64", chunk_len=32))


def w_complex_rtrl(steps, warmup):
    """Forward-mode glam, gtheta of the complex scan (with y), B=16 H=8 M=64 L=2048."""
    import synth
    import selective_state_space_chunked_amd as ssm
    B, H, M, L = 16, 8, 64, 2048
    cfg = synth.make_complex(B=B, H=H, M=M, L=L, seed=0)
    t = {k: to_dev(cfg[k]) for k in ("r", "phi", "lam", "theta", "u", "c")}
    gy = to_dev(cfg["gy"])
    o = ssm.complex_rtrl(gy=gy, **t)

    def step():
        ssm.complex_rtrl(gy=gy, out=o, **t)

    ms = time_steps(step, steps, warmup)
    BHL, E = B * H * L, B * H * L * M
    nbytes = E * 8 + 3 * BHL * 4 + BHL * 4                         # read u, r, phi, gy; write y
    return dict(name="complex-rtrl", elements=E, ms=ms, kernels=profile_kernels(step), bytes_total=nbytes,
                config=dict(B=B, H=H, M=M, L=L, streams="complex64", state="fp64 (h, dh/dlambda, dh/dtheta)"))


def w_pd(steps, warmup):
    """PD scan, B=8 H=32 N=16 L=17000 K=8, forward (with selection) + backward."""
    import synth
    import selective_state_space_chunked_amd as ssm
    B, H, N, L, K = 8, 32, 16, 17000, 8
    cfg = synth.make_pd(B=B, H=H, N=N, L=L, K=K, seed=0)
    t = {k: to_dev(cfg[k]) for k in ("logits", "dict", "d", "b", "C")}
    gy = to_dev(cfg["gy"])
    fo = ssm.pd_scan_fwd(want_ckpt=True, **t)
    tb = dict(t)
    tb.pop("logits")
    go = ssm.pd_scan_bwd(gy=gy, ckpt=fo["ckpt"], sel=fo["sel"], **tb)

    def step():
        ssm.pd_scan_fwd(want_ckpt=True, out=fo, **t)
        ssm.pd_scan_bwd(gy=gy, ckpt=fo["ckpt"], sel=fo["sel"], out=go, **tb)

    ms = time_steps(step, steps, warmup)
    BHL, E = B * H * L, B * H * L * N
    ck = B * H * (-(-L // 64)) * N * 4
    fwd = BHL * K * 4 + 3 * E * 4 + BHL * 4 * 2 + ck               # read logits, d, b, C; write y, sel, ckpt
    bwd = BHL * 4 + 3 * E * 4 + BHL * 4 + ck + 3 * E * 4            # read sel, d, b, C, gy, ckpt; write gd, gb, gC
    return dict(name="pd", elements=E, ms=ms, kernels=profile_kernels(step), bytes_total=fwd + bwd,
                config=dict(B=B, H=H, N=N, L=L, K=K, chunk_len=64))


def w_pd_ste(steps, warmup):
    """PD scan as w_pd, the backward also producing the straight-through gradient of the scores (tau 1)."""
    import synth
    import selective_state_space_chunked_amd as ssm
    B, H, N, L, K = 8, 32, 16, 17000, 8
    cfg = synth.make_pd(B=B, H=H, N=N, L=L, K=K, seed=0)
    t = {k: to_dev(cfg[k]) for k in ("logits", "dict", "d", "b", "C")}
    gy = to_dev(cfg["gy"])
    fo = ssm.pd_scan_fwd(want_ckpt=True, **t)
    tb = dict(t)
    lg = tb.pop("logits")
    want = ("gd", "gb", "gC", "gh0", "glogits")
    go = ssm.pd_scan_bwd(gy=gy, ckpt=fo["ckpt"], sel=fo["sel"], ste_logits=lg, tau=1.0, want=want, **tb)

    def step():
        ssm.pd_scan_fwd(want_ckpt=True, out=fo, **t)
        ssm.pd_scan_bwd(gy=gy, ckpt=fo["ckpt"], sel=fo["sel"], ste_logits=lg, tau=1.0, want=want, out=go, **tb)

    ms = time_steps(step, steps, warmup)
    BHL, E = B * H * L, B * H * L * N
    ck = B * H * (-(-L // 64)) * N * 4
    fwd = BHL * K * 4 + 3 * E * 4 + BHL * 4 * 2 + ck
    bwd = BHL * 4 + 3 * E * 4 + BHL * 4 + ck + 3 * E * 4 + 2 * BHL * K * 4   # + read logits, write glogits
    return dict(name="pd-ste", elements=E, ms=ms, kernels=profile_kernels(step), bytes_total=fwd + bwd,
                config=dict(B=B, H=H, N=N, L=L, K=K, chunk_len=64, tau=1.0))


def w_dense(steps, warmup):
    """Dense a_t, b_t scan at the Mamba-layer shape B=8 D=2048 N=16 L=4096, fp32."""
    import torch
    import selective_state_space_chunked_amd as ssm
    B, D, N, L = 8, 2048, 16, 4096
    gen = torch.Generator(device="cuda").manual_seed(0)
    a = torch.rand((B, D, L, N), device="cuda", generator=gen) * 0.5 + 0.5
    b = torch.randn((B, D, L, N), device="cuda", generator=gen) * 0.25
    C = torch.randn((B, L, N), device="cuda", generator=gen) * 0.25
    gy = torch.randn((B, D, L), device="cuda", generator=gen)
    t = dict(a=a, b=b, C=C)
    fo = ssm.scan_fwd(ssm.SSM_REAL_DENSE, want_ckpt=True, **t)
    go = ssm.scan_bwd(ssm.SSM_REAL_DENSE, gy=gy, ckpt=fo["ckpt"], **t)

    def step():
        ssm.scan_fwd(ssm.SSM_REAL_DENSE, want_ckpt=True, out=fo, **t)
        ssm.scan_bwd(ssm.SSM_REAL_DENSE, gy=gy, ckpt=fo["ckpt"], out=go, **t)

    ms = time_steps(step, max(3, steps // 4), max(1, warmup // 2))
    E, BDL, BLN = B * D * L * N, B * D * L, B * L * N
    ck = B * D * (L // 32) * N * 4
    fwd = 2 * E * 4 + BLN * 4 + BDL * 4 + ck                       # read a, b, C; write y, ckpt
    bwd = 2 * E * 4 + BLN * 4 + BDL * 4 + ck + 2 * E * 4 + BLN * 4  # read a, b, C, gy, ckpt; write ga, gb, gC
    return dict(name="dense", elements=E, ms=ms, kernels=profile_kernels(step, reps=2), bytes_total=fwd + bwd,
                config=dict(B=B, D=D, N=N, L=L, streams="f32", chunk_len=32, data="torch-generated on device"))


# fp32 MFMA peak of MI355X (dense): 256 CUs x 4 SIMDs x 64 flops per cycle x 2.4 GHz
MFMA_F32_PEAK = 256 * 4 * 64 * 2.4e9


def w_head(steps, warmup):
    """Scalar transition per head (the chunked matrix form on the matrix cores, forward and its exact
    adjoint): B=8 H=32 P=64 (D=2048) N=16 L=4096, bf16 streams, the element count of the Mamba-layer
    workload.  Reports the matrix-core rate of the four MFMA passes."""
    import torch
    import selective_state_space_chunked_amd as ssm
    B, H, P, N, L = 8, 32, 64, 16, 4096
    D = H * P
    gen = torch.Generator(device="cuda").manual_seed(0)
    bf = torch.bfloat16
    t = dict(delta=torch.nn.functional.softplus(torch.randn((B, H, L), device="cuda", generator=gen)).to(bf),
             x=torch.randn((B, D, L), device="cuda", generator=gen).to(bf),
             A=-torch.exp(torch.rand((H,), device="cuda", generator=gen) * 2 - 3),
             Bm=(torch.randn((B, L, N), device="cuda", generator=gen) / 4).to(bf),
             C=(torch.randn((B, L, N), device="cuda", generator=gen) / 4).to(bf))
    gy = torch.randn((B, D, L), device="cuda", generator=gen).to(bf)
    fo = ssm.scan_fwd(ssm.SSM_HEAD_SCALAR, want_ckpt=True, **t)
    go = ssm.scan_bwd(ssm.SSM_HEAD_SCALAR, gy=gy, ckpt=fo["ckpt"], want=("gdelta", "gx", "gBm", "gC"), **t)

    def step():
        ssm.scan_fwd(ssm.SSM_HEAD_SCALAR, want_ckpt=True, out=fo, **t)
        ssm.scan_bwd(ssm.SSM_HEAD_SCALAR, gy=gy, ckpt=fo["ckpt"], want=("gdelta", "gx", "gBm", "gC"), out=go, **t)

    ms = time_steps(step, max(3, steps // 4), max(1, warmup // 2))
    kern = profile_kernels(step, reps=2)
    nch = L // 64
    # MFMAs (v_mfma_f32_16x16x4_f32, 2048 flops each) executed per 64-step chunk.  States: (P/16)(N/16)
    # tiles of K = 64.  Outputs: the wave with row block rb (0..3) forms G tiles up to the diagonal
    # ((rb+1) N/4), multiplies M by X over K = 16 (rb+1) for P/16 column tiles, and adds the carried term
    # (N/4 per column tile).  Backward chunk sums: the state pass on (gy, C).  Backward: the ten causal
    # 16 x 16 blocks of G (K = N) and K = dY X^T (K = P); for each 16-step block w and 16-state block,
    # gB = Kd^T C over the row blocks >= w and X G_out^T (K = P), gC = dY H_in^T (K = P) and Kd B over the
    # column blocks <= w; for each 16-channel block, Z = Mf^T dY over the row blocks >= each column block
    # and B G_out (K = N).  SQ_VALU_MFMA_BUSY_CYCLES / 32 per chunk reads the same counts.
    per_chunk = {"head chunk states (matrix cores)": (P // 16) * (N // 16) * 16,
                 "head outputs (matrix cores)": sum((rb + 1) * (N // 4) + (P // 16) * 4 * (rb + 1)
                                                    + (P // 16) * (N // 4) for rb in range(4)),
                 "head backward chunk sums (matrix cores)": (P // 16) * (N // 16) * 16,
                 "head backward (matrix cores)": 10 * (N // 4 + P // 4) + (80 + 2 * P) * (N // 16)
                                                 + (40 + N) * (P // 16)}
    mfma = {}
    for k, n_mfma in per_chunk.items():
        if k in kern:
            fl = n_mfma * 2048.0 * B * H * nch
            rate = fl / (kern[k][0] * 1e-3)
            mfma[k] = {"mfma_per_chunk": n_mfma, "TFLOP/s": round(rate / 1e12, 2),
                       "busy_frac": round(rate / MFMA_F32_PEAK, 3)}
    BDL, BHL, BLN = B * D * L, B * H * L, B * L * N
    ck = B * D * nch * N * 4
    fwd = 2 * (BHL + BDL + 2 * BLN) + 2 * BDL + ck                 # read delta, x, B, C; write y, ckpt
    bwd = 2 * (BHL + 2 * BDL + 2 * BLN) + ck + 2 * (BHL + BDL + 2 * BLN)  # + gy; write gdelta, gx, gB, gC
    return dict(name="head", elements=B * D * N * L, ms=ms, kernels=kern, bytes_total=fwd + bwd,
                config=dict(B=B, H=H, P=P, D=D, N=N, L=L, streams="bf16", chunk_len=64,
                            data="torch-generated on device"),
                mfma=dict(kernels=mfma, peak_TFLOP_s=round(MFMA_F32_PEAK / 1e12, 1),
                          note="busy_frac: executed fp32 MFMA flops over the dense fp32 matrix-core peak, "
                               "i.e. the fraction of SIMD cycles the matrix cores are busy"))


def summarize(w):
    ms = w["ms"]
    r = dict(el_per_s=w["elements"] / (ms * 1e-3), ms_per_step=ms,
             hbm_frac=w["bytes_total"] / (ms * 1e-3) / HBM_PEAK, algorithmic_bytes=w["bytes_total"],
             config=w["config"], kernels_ms={k: round(v[0], 4) for k, v in w["kernels"].items()})
    if w.get("note"):
        r["note"] = w["note"]
    if w.get("mfma"):
        r["mfma"] = w["mfma"]
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


def cpu_per_core(seconds=3.0):
    """The oracle on one thread, forward + backward of the small fp32 selective case (B=1 D=16 N=16 L=1024),
    repeated for about `seconds`: the per-core rate."""
    import oracle
    import synth
    cfg = synth.make_real(B=1, D=16, N=16, L=1024, seed=0)
    kw = dict(delta=cfg["delta"], x=cfg["x"], A=cfg["A"], Bm=cfg["Bm"], C=cfg["C"], B=1, D=16, L=1024, N=16)
    prev = oracle.threads()
    oracle.set_threads(1)
    try:
        n, t0 = 0, time.perf_counter()
        while True:
            oracle.real_fwd(**kw)
            oracle.real_bwd(**kw, gy=cfg["gy"])
            n += 1
            if time.perf_counter() - t0 >= seconds:
                break
        dt = time.perf_counter() - t0
    finally:
        oracle.set_threads(prev)
    return n * 16 * 1024 * 16 / dt


def step_stats(step, n, flush):
    """Per-step times (ms) from HIP events on the current stream: p10, median, p90.  With `flush`, a 1 GiB
    buffer is written before every step (outside the events) so the 256 MB Infinity Cache holds none of the
    step's inputs."""
    import torch
    buf = torch.empty(1 << 28, dtype=torch.float32, device="cuda") if flush else None
    ts = []
    for i in range(n):
        if flush:
            buf.fill_(float(i))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        step()
        e1.record()
        e1.synchronize()
        ts.append(e0.elapsed_time(e1))
    del buf
    q = np.percentile(np.array(ts), [10, 50, 90])
    return {"p10": round(float(q[0]), 4), "median": round(float(q[1]), 4), "p90": round(float(q[2]), 4), "n": n}


def copy_ceiling():
    """Device-to-device copy of 1 GiB, best of 5: GB/s counting read + write bytes."""
    import torch
    src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    best = float("inf")
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        e1.synchronize()
        best = min(best, e0.elapsed_time(e1))
    del src, dst
    return 2 * (1 << 30) / (best * 1e-3) / 1e9


def device_info():
    import glob
    import torch
    pr = torch.cuda.get_device_properties(0)
    info = {"name": pr.name, "arch": getattr(pr, "gcnArchName", None), "compute_units": pr.multi_processor_count,
            "hip": torch.version.hip, "torch": torch.__version__}
    for f in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            lines = open(f).read().split("\n")
        except OSError:
            continue
        cur = [l for l in lines if l.strip().endswith("*")]
        info["sclk"] = (cur[0] if cur else lines[0]).strip()
        info["sclk_max"] = [l for l in lines if l.strip()][-1].strip()
        break
    return info


ROOF_KINDS = {0: "v_fma_f32", 1: "v_mul_f32", 2: "v_exp_f32", 3: "v_fmac_f32 (DPP source)",
              4: "v_permlane32_swap", 5: "v_permlane16_swap", 6: "v_add_f32", 7: "v_fmac_f32"}


def roof_probes(iters=2000):
    """Issue rate (lane operations per second, whole chip) of every instruction class at 1, 2, 4 and 8 waves
    per SIMD, each lane running independent chains (8, or 4 for the DPP form); and the fp32 FMA ceiling in
    TFLOP/s (2 flops per lane operation) at the best occupancy."""
    import torch
    from selective_state_space_chunked_amd import lib
    L = lib()
    L.ssm_roof_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                 ctypes.POINTER(ctypes.c_double), ctypes.c_void_p]
    simds = 4 * torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(8 * simds * 64, dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    table = {}
    for kind, name in ROOF_KINDS.items():
        chains = 4 if kind == 3 else 8
        row = {}
        for w in (1, 2, 4, 8):
            r = ctypes.c_double(0.0)
            for _ in range(2):   # the second launch is the one kept (the first pays for loading the code)
                rc = L.ssm_roof_probe(kind, chains, w * simds, iters, ctypes.c_void_p(sink.data_ptr()),
                                      ctypes.byref(r), ctypes.c_void_p(st))
                assert rc == 0, rc
            row[f"{w}_waves_per_simd"] = r.value
        table[name] = {k: round(v / 1e12, 3) for k, v in row.items()}
        table[name]["cycles_per_wave64_instr_best"] = round(simds * 64 * 2.4e9 / max(row.values()), 3)
    # the fp32 FMA ceiling: the faster of the two encodings (VOP3 v_fma_f32, VOP2 v_fmac_f32)
    fma_best = max(v for name in ("v_fma_f32", "v_fmac_f32") for k, v in table[name].items()
                   if k.endswith("simd")) * 1e12
    return {"unit": "T lane-ops/s (whole chip)", "iters": iters, "classes": table,
            "fp32_fma_TFLOPs_measured": round(2 * fma_best / 1e12, 2),
            "note": "cycles_per_wave64_instr_best = 64 lanes x SIMDs x 2.4 GHz / best rate"}


def calib_copy():
    """One device copy of exactly 1 GiB (reads 1 GiB, writes 1 GiB)."""
    import torch
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


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
    if args.calib_copy:
        calib_copy()
    head = w_real(HEADLINE, 8, 2048, 16, 4096, "bf16", args.steps, args.warmup, keep_inputs=not args.no_cpu)
    s = summarize(head)
    kern = head["kernels"]
    dom = max((k for k in kern if k in head["bytes_kernel"]), key=lambda k: kern[k][0] * kern[k][1])
    dur = kern[dom][0] * 1e-3
    flops = FLOPS_PER_ELEMENT[dom] * head["elements"]
    meas = MEASURED_TRAFFIC.get(dom)
    traffic = valu_busy = issue = barrier = None
    if meas and meas["sources_sha256"] == kernel_sources_sha256():
        traffic = meas["read_bytes"] + meas["written_bytes"]
        valu_busy = meas.get("valu_busy")
        issue, barrier = meas.get("issue_model_frac"), meas.get("barrier_wait_frac")
    roof = {"kernel": dom, "bound": "alu", "achieved": flops / dur / 1e12, "peak": VALU_F32_PEAK / 1e12,
            "unit": "TFLOP/s", "frac": flops / dur / VALU_F32_PEAK, "traffic": traffic,
            "traffic_unit": "HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "duration_ms": kern[dom][0], "hbm_frac": head["bytes_kernel"][dom] / dur / HBM_PEAK,
            "flops_per_element": FLOPS_PER_ELEMENT[dom],
            "valu_busy_frac": valu_busy,
            "valu_busy_note": "fraction of SIMD cycles with a VALU instruction in flight (rocprofv3 counters)",
            "issue_model_frac": issue, "barrier_wait_frac": barrier,
            "issue_note": "issue_model_frac: per-class VALU counts x measured cycles per class / kernel cycles; "
                          "barrier_wait_frac: wave cycles at barriers / wave cycles (rocprofv3 counters)"}
    others = {}
    if not args.no_others:
        todo = [w.strip() for w in args.workloads.split(",") if w.strip()] or \
            ["impulse", "output-sens", "sens-rows", "complex", "complex-dense", "complex-rtrl", "pd", "pd-ste", "dense",
             "head", "real-small"]
        for w in todo:
            # each workload starts from an empty allocator cache: blocks cached by the previous
            # workload's differently sized tensors otherwise fragment the next one's allocations
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
            if w == "impulse":
                others[w] = summarize(w_impulse(args.steps, args.warmup))
            elif w == "output-sens":
                others[w] = summarize(w_output_sens(args.steps, args.warmup))
            elif w == "sens-rows":
                others[w] = summarize(w_sens_rows(args.steps, args.warmup))
            elif w == "complex":
                others[w] = summarize(w_complex(args.steps, args.warmup))
            elif w == "complex-dense":
                others[w] = summarize(w_complex_dense(args.steps, args.warmup))
            elif w == "complex-rtrl":
                others[w] = summarize(w_complex_rtrl(args.steps, args.warmup))
            elif w == "pd":
                others[w] = summarize(w_pd(args.steps, args.warmup))
            elif w == "pd-ste":
                others[w] = summarize(w_pd_ste(args.steps, args.warmup))
            elif w == "dense":
                others[w] = summarize(w_dense(args.steps, args.warmup))
            elif w == "head":
                others[w] = summarize(w_head(args.steps, args.warmup))
            elif w == "real-small":
                others[w] = summarize(w_real(w, 1, 16, 16, 1024, "f32", args.steps, args.warmup))
            torch.cuda.empty_cache()
    timing = {"back_to_back_ms": step_stats(head["step"], 20, False),
              "cache_flushed_ms": step_stats(head["step"], 20, True),
              "note": "per-step HIP-event times of the headline step; cache_flushed writes 1 GiB before each step"}
    hbm_copy = copy_ceiling()
    roof_meas = None if args.no_roof else roof_probes()
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(head["inputs"], args.cpu_batches)
        cpu["per_core_value"] = cpu_per_core()
        cpu["per_core_sample"] = ("one thread, forward + backward of B=1 D=16 N=16 L=1024 fp32 "
                                  "(the small selective case), repeated for 3 s")
    line = {
        "metric": METRIC, "value": s["el_per_s"], "unit": "elements/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": s["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "dtype_note": "arithmetic (state, recurrences, accumulation) in fp32; the streams x, delta, B, C, gy, "
                      "y and the gradients are bf16 in HBM",
        "config": {"workload": "real-mamba: selective scan fwd+bwd, B=8 D=2048 N=16 L=4096, bf16 streams, "
                               "fp32 state, chunk 256", **head["config"]},
        "hbm_frac": s["hbm_frac"], "algorithmic_bytes_per_step": head["bytes_total"],
        "kernels_ms": s["kernels_ms"], "roofline": roof, "cpu_baseline": cpu, "others": others,
        "timing": timing, "hbm_copy_GBps": round(hbm_copy, 1), "device": device_info(),
    }
    if roof_meas:
        line["roof_measured"] = roof_meas
        roof["peak_measured"] = roof_meas["fp32_fma_TFLOPs_measured"]
        roof["frac_of_measured"] = roof["achieved"] / roof_meas["fp32_fma_TFLOPs_measured"]
    print(json.dumps(line))


if __name__ == "__main__":
    main()
