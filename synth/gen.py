"""Seeded input generators for the five selective-scan workloads.

Every array is drawn with numpy's ``Generator(PCG64(seed))`` in a fixed order,
in float64, then rounded to float32 (round-to-nearest-even) and, where a
workload streams bfloat16, rounded again to bfloat16 (round-to-nearest-even on
the float32 bits).  The distribution transforms below (softplus for step
sizes and retention, the logistic function for PD diagonals) shape the
*inputs*; the scan consumes their results as given.

Workloads (sizes are the defaults; tests pass smaller sizes with the same
distributions):

* ``real-small``   diagonal real selective scan, fp32, B=1 D=16 N=16 L=1024
  (Mamba-style selection and discretisation, lpnh.cn "S3M" page, section 1.1;
  log(-A) uniform in [-3,-1] follows that page's troubleshooting section 5.1).
* ``real-mamba``   the same distributions at B=8 D=2048 N=16 L=4096, bf16
  streams, fp32 A.
* ``impulse``      B=1 D=1024 N=16 L=128000, fp32, x = impulse at t=0,
  softplus(N(-2, 0.5)) step sizes (the PGF page's 128,000-step
  impulse-response benchmark, abstract).
* ``complex``      B=16 H=8 M=64 L=2048 complex64 with shared retention and
  phase controls (SPARC page, abstract).
* ``pd``           B=8 H=32 N=16 L=17000 K=8 PD transitions (Flash PD-SSM page,
  "Neuer Selektionsmechanismus"); L=17000 mirrors the >17,000-step time series
  of that page's experiments.
"""
from __future__ import annotations

import math

import numpy as np

CONFIGS = {
    "real-small": dict(B=1, D=16, N=16, L=1024, dtype="f32"),
    "real-mamba": dict(B=8, D=2048, N=16, L=4096, dtype="bf16"),
    "impulse": dict(B=1, D=1024, N=16, L=128000, dtype="f32"),
    "complex": dict(B=16, H=8, M=64, L=2048),
    "pd": dict(B=8, H=32, N=16, L=17000, K=8),
}


# ----------------------------------------------------------------------------
# number formats
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    bias = ((u >> 16) & 1) + 0x7FFF
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def widen(arr) -> np.ndarray:
    """Exact float64 value of a float32 array or of a bf16 bit array (uint16)."""
    arr = np.asarray(arr)
    if arr.dtype == np.uint16:
        return bf16_bits_to_f32(arr).astype(np.float64)
    return arr.astype(np.float64)


def _softplus(z):
    # log(1 + e^z) evaluated without overflow; an input-shaping transform.
    return np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))


def _logistic(z):
    return 0.5 * (1.0 + np.tanh(0.5 * z))


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _stream(a, dtype):
    a32 = _f32(a)
    return f32_to_bf16_bits(a32) if dtype == "bf16" else a32


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------
def make_real(B=1, D=16, N=16, L=1024, dtype="f32", seed=0, with_grad=True, projection_output=False):
    """Diagonal real selective-scan inputs.

    Draw order: x, z (delta = softplus(z)), U (A = -exp(U)), Bm, C, gy.
    Shapes: x, delta, gy (B,D,L); A (D,N); Bm, C (B,L,N).  h0 = 0.
    ``dtype`` 'bf16' rounds the streamed tensors (x, delta, Bm, C, gy) to
    bfloat16; A always stays float32.
    ``projection_output``: ``delta`` holds the pre-activation z - bias instead
    (so softplus(delta + bias) is the same step-size distribution) and
    ``delta_bias`` a per-channel bias ~ N(0, 1/4), drawn last.
    """
    g = np.random.Generator(np.random.PCG64(seed))
    x = g.standard_normal((B, D, L))
    z = g.standard_normal((B, D, L))
    delta = _softplus(z)
    U = g.uniform(-3.0, -1.0, (D, N))
    A = -np.exp(U)
    s = 1.0 / math.sqrt(N)
    Bm = g.standard_normal((B, L, N)) * s
    C = g.standard_normal((B, L, N)) * s
    out = dict(
        B=B, D=D, N=N, L=L, dtype=dtype,
        x=_stream(x, dtype), delta=_stream(delta, dtype), A=_f32(A),
        Bm=_stream(Bm, dtype), C=_stream(C, dtype),
    )
    if with_grad:
        out["gy"] = _stream(g.standard_normal((B, D, L)), dtype)
    if projection_output:
        bias = g.standard_normal(D) * 0.5
        out["delta_bias"] = _f32(bias)
        out["delta"] = _stream(z - _f32(bias).astype(np.float64)[None, :, None], dtype)
    return out


def make_impulse(B=1, D=1024, N=16, L=128000, seed=0, with_xrand=False):
    """Impulse-response sensitivity inputs (fp32).

    Draw order: z ~ N(-2, 0.5) (delta = softplus(z)), U (A = -exp(U)), Bm, C,
    then optionally x_rand ~ N(0,1) for linearity checks.  x is zero except
    x[:, :, 0] = 1.
    """
    g = np.random.Generator(np.random.PCG64(seed))
    z = g.normal(-2.0, 0.5, (B, D, L))
    delta = _softplus(z)
    U = g.uniform(-3.0, -1.0, (D, N))
    A = -np.exp(U)
    s = 1.0 / math.sqrt(N)
    Bm = g.standard_normal((B, L, N)) * s
    C = g.standard_normal((B, L, N)) * s
    x = np.zeros((B, D, L), dtype=np.float32)
    x[:, :, 0] = 1.0
    out = dict(B=B, D=D, N=N, L=L, dtype="f32", x=x, delta=_f32(delta), A=_f32(A),
               Bm=_f32(Bm), C=_f32(C))
    if with_xrand:
        out["x_rand"] = _f32(g.standard_normal((B, D, L)))
    return out


def make_complex(B=16, H=8, M=64, L=2048, seed=0, with_grad=True, dtype="f32"):
    """Complex diagonal recurrence with shared retention/phase controls.

    Draw order: lam ~ U[0.9, 0.999] (H,M); theta ~ U[0, pi] (H,M);
    z ~ N(0,1), r = softplus(z) (B,H,L); phi ~ N(0,1) (B,H,L);
    u = N(0,1/2) + i N(0,1/2) (B,H,L,M); c = N(0,1/(2M)) + i N(0,1/(2M)) (H,M);
    gy ~ N(0,1) (B,H,L).  Complex arrays are complex64 (interleaved re, im).
    ``dtype`` 'bf16' rounds the streams r, phi, gy to bfloat16 bits and gives u
    as bfloat16 bits of shape (B,H,L,M,2) (re, im), plus ``u_c``, the complex
    values those bits hold; lam, theta and c stay fp32 / complex64.
    """
    g = np.random.Generator(np.random.PCG64(seed))
    lam = g.uniform(0.9, 0.999, (H, M))
    theta = g.uniform(0.0, math.pi, (H, M))
    r = _softplus(g.standard_normal((B, H, L)))
    phi = g.standard_normal((B, H, L))
    su = math.sqrt(0.5)
    u_re = g.standard_normal((B, H, L, M)) * su
    u_im = g.standard_normal((B, H, L, M)) * su
    sc = math.sqrt(1.0 / (2 * M))
    c_re = g.standard_normal((H, M)) * sc
    c_im = g.standard_normal((H, M)) * sc
    u = np.empty((B, H, L, M), dtype=np.complex64)
    u.real = u_re
    u.imag = u_im
    c = np.empty((H, M), dtype=np.complex64)
    c.real = c_re
    c.imag = c_im
    out = dict(B=B, H=H, M=M, L=L, dtype=dtype, lam=_f32(lam), theta=_f32(theta), r=_stream(r, dtype),
               phi=_stream(phi, dtype), u=u, c=c)
    if dtype == "bf16":
        bits = np.stack([f32_to_bf16_bits(u.real), f32_to_bf16_bits(u.imag)], axis=-1)
        out["u"] = np.ascontiguousarray(bits)
        u_c = np.empty((B, H, L, M), dtype=np.complex64)
        u_c.real = bf16_bits_to_f32(bits[..., 0])
        u_c.imag = bf16_bits_to_f32(bits[..., 1])
        out["u_c"] = u_c
    if with_grad:
        out["gy"] = _stream(g.standard_normal((B, H, L)), dtype)
    return out


def make_complex_dense(B=16, H=8, M=64, L=2048, seed=0, with_grad=True):
    """Complex diagonal recurrence with given per-step transitions (complex64).

    Draw order: rho ~ U[0.9, 0.999] (B,H,L,M); angle ~ U[-pi, pi] (B,H,L,M),
    a = rho e^{i angle}; u = N(0,1/2) + i N(0,1/2) (B,H,L,M);
    c = N(0,1/(2M)) + i N(0,1/(2M)) (H,M); gy ~ N(0,1) (B,H,L).
    """
    g = np.random.Generator(np.random.PCG64(seed))
    rho = g.uniform(0.9, 0.999, (B, H, L, M))
    ang = g.uniform(-math.pi, math.pi, (B, H, L, M))
    a = (rho * np.exp(1j * ang)).astype(np.complex64)
    su = math.sqrt(0.5)
    u = np.empty((B, H, L, M), dtype=np.complex64)
    u.real = g.standard_normal((B, H, L, M)) * su
    u.imag = g.standard_normal((B, H, L, M)) * su
    sc = math.sqrt(1.0 / (2 * M))
    c = np.empty((H, M), dtype=np.complex64)
    c.real = g.standard_normal((H, M)) * sc
    c.imag = g.standard_normal((H, M)) * sc
    out = dict(B=B, H=H, M=M, L=L, dtype="f32", a=a, u=u, c=c)
    if with_grad:
        out["gy"] = _f32(g.standard_normal((B, H, L)))
    return out


def make_pd(B=8, H=32, N=16, L=17000, K=8, seed=0, with_grad=True, dtype="f32"):
    """PD-transition scan inputs (fp32 values, int32 indices; ``dtype`` 'bf16'
    rounds the streams logits, d, b, C, gy to bfloat16 bits).

    Draw order: dict ~ U{0..N-1} i.i.d. per (head, entry, column) (H,K,N);
    logits ~ N(0,1) (B,H,L,K); z ~ N(0,1), d = logistic(z) (B,H,L,N);
    b ~ N(0,1)/sqrt(N); C ~ N(0,1)/sqrt(N) (B,H,L,N); gy ~ N(0,1) (B,H,L).
    Entry k of head h is the column-one-hot matrix whose column j holds its
    one at row dict[h,k,j].
    """
    g = np.random.Generator(np.random.PCG64(seed))
    dct = g.integers(0, N, (H, K, N)).astype(np.int32)
    logits = g.standard_normal((B, H, L, K))
    d = _logistic(g.standard_normal((B, H, L, N)))
    s = 1.0 / math.sqrt(N)
    b = g.standard_normal((B, H, L, N)) * s
    C = g.standard_normal((B, H, L, N)) * s
    out = dict(B=B, H=H, N=N, L=L, K=K, dict=np.ascontiguousarray(dct), dtype=dtype,
               logits=_stream(logits, dtype), d=_stream(d, dtype), b=_stream(b, dtype), C=_stream(C, dtype))
    if with_grad:
        out["gy"] = _stream(g.standard_normal((B, H, L)), dtype)
    return out
