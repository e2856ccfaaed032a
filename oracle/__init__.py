"""fp64 CPU oracle for the selective scan -- TEST INFRASTRUCTURE ONLY.

Only tests/, ``__graft_entry__.smoke()`` and bench.py's CPU-baseline leg may
import this package.  It wraps ``oracle.c`` (plain sequential double-precision
loops, built with gcc, no fast-math) through ctypes.  It shares nothing with
the HIP path: no kernels, headers, helpers or tables; both sides only consume
the seeded arrays from ``synth``.

All routines take numpy arrays holding the exact values the GPU consumes
(float32, bfloat16 bits as uint16, complex64, int32) and widen them to float64
here; results come back as float64 (int32 for selections).

Pinned by tests/test_oracle_pins.py: scalar transition per head ``head_fwd`` /
``head_bwd`` (the quadratic form y_t = sum_s (C_t . B_s) exp(A sum delta) delta_s
x_s written out as a matrix product, equality with the diagonal scan on expanded
arrays, finite differences); general selective scan ``sel_fwd`` / ``sel_bwd``
(zero-order hold: the exact solution of dh/dt = A h + B x for inputs held
constant, the A = 0 limit equal to the Euler scan, central finite differences;
per-channel B and C: brute-force O(L^2) sums, equality with the shared form
for channel-independent B, C, finite differences; Euler form equal to
real_fwd / real_bwd), real forward (brute-force O(L^2) sums,
geometric closed form, prefix-sum special case), real backward (central finite
differences, adjoint identity), impulse sensitivity (closed form with exactly
rounded step-size sums, linearity, equality with the general backward),
complex forward (2x2 real-matrix route, geometric closed form, reduction to the
real scan, modulus invariance), complex backward (finite differences), PD
forward (DFA simulation of the dictionary read as an automaton, dense-matrix
route, column-sum invariant, reduction to the real scan), PD backward (finite
differences), selection (brute-force argmax).  No routine is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_I = ctypes.POINTER(ctypes.c_int32)
_L = ctypes.c_longlong


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (-O2 -fopenmp, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
                               "-fno-fast-math", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        lib.orc_real_fwd.argtypes = [ctypes.c_int, _L, _L, _L, _L] + [_D] * 10
        lib.orc_real_bwd.argtypes = [ctypes.c_int, _L, _L, _L, _L] + [_D] * 18
        lib.orc_sel_fwd.argtypes = [ctypes.c_int, ctypes.c_int, _L, _L, _L, _L] + [_D] * 8
        lib.orc_sel_bwd.argtypes = [ctypes.c_int, ctypes.c_int, _L, _L, _L, _L] + [_D] * 14
        lib.orc_head_fwd.argtypes = [_L, _L, _L, _L, _L] + [_D] * 8
        lib.orc_head_bwd.argtypes = [_L, _L, _L, _L, _L] + [_D] * 14
        lib.orc_impulse_sens.argtypes = [_L, _L, _L, _L, _L] + [_D] * 5
        lib.orc_output_sens.argtypes = [_L, _L, _L, _L, _L] + [_D] * 8
        lib.orc_complex_fwd.argtypes = [_L, _L, _L, _L] + [_D] * 9
        lib.orc_complex_dense_fwd.argtypes = [_L, _L, _L, _L] + [_D] * 6
        lib.orc_complex_dense_bwd.argtypes = [_L, _L, _L, _L] + [_D] * 10
        lib.orc_complex_bwd.argtypes = [_L, _L, _L, _L] + [_D] * 16
        lib.orc_complex_rtrl.argtypes = [_L, _L, _L, _L] + [_D] * 12
        lib.orc_pd_select.argtypes = [_L, _L, _L, _L, _D, _I]
        lib.orc_pd_fwd.argtypes = [_L, _L, _L, _L, _L, _I, _I] + [_D] * 6
        lib.orc_pd_dense_fwd.argtypes = [_L, _L, _L, _L, _L, _I, _I] + [_D] * 6
        lib.orc_pd_bwd.argtypes = [_L, _L, _L, _L, _L, _I, _I] + [_D] * 10
        lib.orc_pd_ste.argtypes = [_L, _L, _L, _L, _L, _D, _I, _I] + [_D] * 6 + [ctypes.c_double, _D, _D]
        lib.orc_pd_mix_fwd.argtypes = [_L, _L, _L, _L, _L, _D, _I] + [_D] * 6
        lib.orc_threads.restype = ctypes.c_int
        lib.orc_set_threads.argtypes = [ctypes.c_int]
        _lib = lib
    return _lib


def threads() -> int:
    return int(_load().orc_threads())


def set_threads(n: int) -> None:
    """Thread count of later calls (n >= 1)."""
    _load().orc_set_threads(int(n))


def _w(a):
    """Exact float64 copy (bf16 bit arrays are uint16)."""
    if a is None:
        return None
    a = np.asarray(a)
    if a.dtype == np.uint16:
        a = (a.astype(np.uint32) << 16).view(np.float32)
    if np.iscomplexobj(a):
        a = np.ascontiguousarray(a.astype(np.complex128)).view(np.float64)
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a):
    return None if a is None else a.ctypes.data_as(_D)


def _pi(a):
    return None if a is None else a.ctypes.data_as(_I)


def _z(shape):
    return np.zeros(shape, dtype=np.float64)


# ---------------------------------------------------------------------------
# diagonal real scan
# ---------------------------------------------------------------------------
def real_fwd(*, delta=None, x=None, A=None, Bm=None, a=None, b=None, C, h0=None,
             B, D, L, N):
    """y (B,D,L) and h_last (B,D,N).  Selective if ``a`` is None, else dense."""
    mode = 0 if a is None else 1
    args = [_w(v) for v in (delta, x, A, Bm, a, b, C, h0)]
    y, hl = _z((B, D, L)), _z((B, D, N))
    _load().orc_real_fwd(mode, B, D, L, N, *[_p(v) for v in args], _p(y), _p(hl))
    return y, hl


def sel_fwd(*, delta, x, A, Bm, C, h0=None, disc=0, perd=False, B, D, L, N):
    """Selective scan, general form: y (B,D,L) and h_last (B,D,N).  ``disc`` 0 is the Euler input term
    delta x B, 1 the zero-order hold (exp(delta A) - 1) / A x B (delta x B where A = 0).  ``perd``: Bm and
    C are (B,D,L,N), one per channel, else (B,L,N) shared by the channels."""
    args = [_w(v) for v in (delta, x, A, Bm, C, h0)]
    y, hl = _z((B, D, L)), _z((B, D, N))
    _load().orc_sel_fwd(int(disc), int(bool(perd)), B, D, L, N, *[_p(v) for v in args], _p(y), _p(hl))
    return y, hl


def sel_bwd(*, delta, x, A, Bm, C, h0=None, gy, ghlast=None, disc=0, perd=False, B, D, L, N):
    """Gradients of sum<gy,y> + <ghlast,h_last> of ``sel_fwd``: dict(gdelta, gx, gA, gBm, gC, gh0), with
    gBm, gC (B,L,N) sums over the channels, or (B,D,L,N) when ``perd``."""
    args = [_w(v) for v in (delta, x, A, Bm, C, h0, gy, ghlast)]
    gbc = (B, D, L, N) if perd else (B, L, N)
    out = dict(gdelta=_z((B, D, L)), gx=_z((B, D, L)), gA=_z((D, N)), gBm=_z(gbc), gC=_z(gbc), gh0=_z((B, D, N)))
    _load().orc_sel_bwd(int(disc), int(bool(perd)), B, D, L, N, *[_p(v) for v in args],
                        *[_p(out[k]) for k in ("gdelta", "gx", "gA", "gBm", "gC", "gh0")])
    return out


def head_fwd(*, delta, x, A, Bm, C, h0=None, B, H, P, L, N):
    """Scalar transition per head: y (B,H*P,L), h_last (B,H*P,N).  delta (B,H,L), x (B,H*P,L), A (H),
    Bm, C (B,L,N); channel d = h*P + p belongs to head h."""
    args = [_w(v) for v in (delta, x, A, Bm, C, h0)]
    y, hl = _z((B, H * P, L)), _z((B, H * P, N))
    _load().orc_head_fwd(B, H, P, L, N, *[_p(v) for v in args], _p(y), _p(hl))
    return y, hl


def head_bwd(*, delta, x, A, Bm, C, h0=None, gy, ghlast=None, B, H, P, L, N):
    """Gradients of sum<gy,y> + <ghlast,h_last> of ``head_fwd``: gdelta (B,H,L), gx (B,H*P,L), gA (H),
    gBm, gC (B,L,N), gh0 (B,H*P,N)."""
    args = [_w(v) for v in (delta, x, A, Bm, C, h0, gy, ghlast)]
    out = dict(gdelta=_z((B, H, L)), gx=_z((B, H * P, L)), gA=_z((H,)), gBm=_z((B, L, N)), gC=_z((B, L, N)),
               gh0=_z((B, H * P, N)))
    _load().orc_head_bwd(B, H, P, L, N, *[_p(v) for v in args],
                         *[_p(out[k]) for k in ("gdelta", "gx", "gA", "gBm", "gC", "gh0")])
    return out


def real_bwd(*, delta=None, x=None, A=None, Bm=None, a=None, b=None, C, h0=None,
             gy, ghlast=None, B, D, L, N):
    """Gradients of sum<gy,y> + <ghlast,h_last>.

    Selective: dict(gdelta, gx, gA, gBm, gC, gh0).  Dense: dict(ga, gb, gC, gh0).
    """
    mode = 0 if a is None else 1
    args = [_w(v) for v in (delta, x, A, Bm, a, b, C, h0, gy, ghlast)]
    out = {}
    if mode == 0:
        out["gdelta"], out["gx"] = _z((B, D, L)), _z((B, D, L))
        out["gA"], out["gBm"] = _z((D, N)), _z((B, L, N))
        ga = gb = None
    else:
        ga, gb = _z((B, D, L, N)), _z((B, D, L, N))
        out["ga"], out["gb"] = ga, gb
    out["gC"], out["gh0"] = _z((B, L, N)), _z((B, D, N))
    _load().orc_real_bwd(mode, B, D, L, N, *[_p(v) for v in args],
                         _p(out.get("gdelta")), _p(out.get("gx")), _p(out.get("gA")),
                         _p(out.get("gBm")), _p(ga), _p(gb), _p(out["gC"]), _p(out["gh0"]))
    return out


def step_sizes(z, delta_bias=None, softplus=False):
    """Step sizes from the input-projection output (the discretisation input of
    the S3M page, section 1.1: delta = softplus(projection(x))), in fp64:
    delta = softplus(z + bias[d]) with softplus(v) = log(1 + e^v), or z + bias
    without softplus.  z (B,D,L) (bf16 bit arrays accepted), bias (D,)."""
    v = _w(z).copy()
    if delta_bias is not None:
        v += _w(delta_bias)[None, :, None]
    return np.logaddexp(0.0, v) if softplus else v


def step_size_grads(gdelta, z, delta_bias=None, softplus=False):
    """Pull-back of dLoss/ddelta to the pre-activation: gz = gdelta * sigmoid(z + bias)
    (d softplus(v)/dv = 1 / (1 + e^-v)), or gdelta without softplus; gbias = sum over b, t."""
    if softplus:
        v = _w(z).copy()
        if delta_bias is not None:
            v += _w(delta_bias)[None, :, None]
        gz = gdelta * (0.5 * (1.0 + np.tanh(0.5 * v)))   # logistic function, no overflow
    else:
        gz = np.array(gdelta, dtype=np.float64)
    return gz, gz.sum(axis=(0, 2))


def impulse_sens(*, delta, A, Bm, C, B, D, L, N, t_out=None):
    """s[b,d,t] = d y[b,d,t_out] / d x[b,d,t]  (B,D,L)."""
    t_out = L - 1 if t_out is None else int(t_out)
    args = [_w(v) for v in (delta, A, Bm, C)]
    s = _z((B, D, L))
    _load().orc_impulse_sens(B, D, L, N, t_out, *[_p(v) for v in args], _p(s))
    return s


# ---------------------------------------------------------------------------
# complex scan
# ---------------------------------------------------------------------------
def _c(a):
    return a.view(np.complex128)


def complex_fwd(*, r, phi, lam, theta, u, c, h0=None, B, H, L, M):
    args = [_w(v) for v in (r, phi, lam, theta, u, c, h0)]
    y = _z((B, H, L))
    hl = _z((B, H, M, 2))
    _load().orc_complex_fwd(B, H, L, M, *[_p(v) for v in args], _p(y), _p(hl))
    return y, _c(hl).reshape(B, H, M)


def complex_bwd(*, r, phi, lam, theta, u, c, h0=None, gy, ghlast=None, B, H, L, M):
    args = [_w(v) for v in (r, phi, lam, theta, u, c, h0, gy, ghlast)]
    gu = _z((B, H, L, M, 2))
    gr, gphi = _z((B, H, L)), _z((B, H, L))
    glam, gtheta = _z((H, M)), _z((H, M))
    gc = _z((H, M, 2))
    gh0 = _z((B, H, M, 2))
    _load().orc_complex_bwd(B, H, L, M, *[_p(v) for v in args], _p(gu), _p(gr), _p(gphi),
                            _p(glam), _p(gtheta), _p(gc), _p(gh0))
    return dict(gu=_c(gu).reshape(B, H, L, M), gr=gr, gphi=gphi, glam=glam, gtheta=gtheta,
                gc=_c(gc).reshape(H, M), gh0=_c(gh0).reshape(B, H, M))


def complex_dense_fwd(*, a, u, c, h0=None, B, H, L, M):
    """Given-transition complex scan: y (B,H,L) and h_last (B,H,M) (oracle.c orc_complex_dense_fwd)."""
    args = [_w(v) for v in (a, u, c, h0)]
    y = _z((B, H, L))
    hl = _z((B, H, M, 2))
    _load().orc_complex_dense_fwd(B, H, L, M, *[_p(v) for v in args], _p(y), _p(hl))
    return y, _c(hl).reshape(B, H, M)


def complex_dense_bwd(*, a, u, c, h0=None, gy, ghlast=None, B, H, L, M):
    """Gradients of sum<gy,y> + Re<ghlast,h_last> w.r.t. a, u, c, h0 (oracle.c orc_complex_dense_bwd)."""
    args = [_w(v) for v in (a, u, c, h0, gy, ghlast)]
    ga, gu = _z((B, H, L, M, 2)), _z((B, H, L, M, 2))
    gc, gh0 = _z((H, M, 2)), _z((B, H, M, 2))
    _load().orc_complex_dense_bwd(B, H, L, M, *[_p(v) for v in args], _p(ga), _p(gu), _p(gc), _p(gh0))
    return dict(ga=_c(ga).reshape(B, H, L, M), gu=_c(gu).reshape(B, H, L, M), gc=_c(gc).reshape(H, M),
                gh0=_c(gh0).reshape(B, H, M))


def complex_rtrl(*, r, phi, lam, theta, u, c, h0=None, gy, ghlast=None, B, H, L, M):
    """Forward-mode gradients of sum_t gy_t y_t (+ <ghlast, h_L>) w.r.t. lambda and theta, and y."""
    args = [_w(v) for v in (r, phi, lam, theta, u, c, h0, gy, ghlast)]
    y = _z((B, H, L))
    glam, gtheta = _z((H, M)), _z((H, M))
    _load().orc_complex_rtrl(B, H, L, M, *[_p(v) for v in args], _p(y), _p(glam), _p(gtheta))
    return dict(y=y, glam=glam, gtheta=gtheta)


# ---------------------------------------------------------------------------
# PD scan
# ---------------------------------------------------------------------------
def pd_select(logits):
    """Index of the first maximum over the last axis, compared on the given values."""
    logits = np.asarray(logits)
    B, H, L, K = logits.shape
    lw = _w(logits)
    sel = np.zeros((B, H, L), dtype=np.int32)
    _load().orc_pd_select(B, H, L, K, _p(lw), _pi(sel))
    return sel


def _pd_common(sel, dct):
    return (np.ascontiguousarray(sel, dtype=np.int32), np.ascontiguousarray(dct, dtype=np.int32))


def pd_fwd(*, sel, dict, d, b, C, h0=None, B, H, L, N, K, dense=False):
    sel, dct = _pd_common(sel, dict)
    args = [_w(v) for v in (d, b, C, h0)]
    y, hl = _z((B, H, L)), _z((B, H, N))
    fn = _load().orc_pd_dense_fwd if dense else _load().orc_pd_fwd
    fn(B, H, L, N, K, _pi(sel), _pi(dct), *[_p(v) for v in args], _p(y), _p(hl))
    return y, hl


def pd_bwd(*, sel, dict, d, b, C, h0=None, gy, ghlast=None, B, H, L, N, K):
    sel, dct = _pd_common(sel, dict)
    args = [_w(v) for v in (d, b, C, h0, gy, ghlast)]
    gd, gb, gC = _z((B, H, L, N)), _z((B, H, L, N)), _z((B, H, L, N))
    gh0 = _z((B, H, N))
    _load().orc_pd_bwd(B, H, L, N, K, _pi(sel), _pi(dct), *[_p(v) for v in args],
                       _p(gd), _p(gb), _p(gC), _p(gh0))
    return {"gd": gd, "gb": gb, "gC": gC, "gh0": gh0}


def pd_ste(*, logits, sel, dict, d, b, C, h0=None, gy, ghlast=None, tau, B, H, L, N, K):
    """Straight-through surrogate gradients of the PD selection: gw = dLoss/dw
    of the mixture weights at the hard selection, glogits through the tempered
    softmax.  Returns dict(gw, glogits), each (B, H, L, K)."""
    sel, dct = _pd_common(sel, dict)
    lw = _w(logits)
    args = [_w(v) for v in (d, b, C, h0, gy, ghlast)]
    gw, gl = _z((B, H, L, K)), _z((B, H, L, K))
    _load().orc_pd_ste(B, H, L, N, K, _p(lw), _pi(sel), _pi(dct), *[_p(v) for v in args], float(tau),
                       _p(gw), _p(gl))
    return {"gw": gw, "glogits": gl}


def pd_mix_fwd(*, w, dict, d, b, C, h0=None, B, H, L, N, K):
    """Forward of the mixture transition sum_k w[t,k] P_k diag(d_t) (dense matrices)."""
    dct = np.ascontiguousarray(dict, dtype=np.int32)
    args = [_w(v) for v in (w, d, b, C, h0)]
    y, hl = _z((B, H, L)), _z((B, H, N))
    _load().orc_pd_mix_fwd(B, H, L, N, K, _p(args[0]), _pi(dct), *[_p(v) for v in args[1:]], _p(y), _p(hl))
    return y, hl


def output_sens(*, delta, x, A, Bm, C, h0=None, B, D, L, N, t_out=None):
    """d y[b,d,t_out] / d x[b,d,t] and / d delta[b,d,t] of the selective scan.
    Returns (s_x, s_delta), each (B, D, L)."""
    t_out = L - 1 if t_out is None else t_out
    args = [_w(v) for v in (delta, x, A, Bm, C, h0)]
    sx, sd = _z((B, D, L)), _z((B, D, L))
    _load().orc_output_sens(B, D, L, N, t_out, *[_p(v) for v in args], _p(sx), _p(sd))
    return sx, sd
