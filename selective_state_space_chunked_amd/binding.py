"""ctypes binding of libssmscan.so (include/ssmscan.h).

Argument marshalling only: tensors are checked for device, dtype and
contiguity, outputs and the workspace are allocated with torch on the
tensors' device, and every step of the scan runs in the library's HIP
kernels on torch's current stream.  There is no CPU fallback: if the library
is missing or a call fails, this module raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libssmscan.so")

SSM_F32, SSM_BF16 = 0, 1
SSM_REAL_SELECTIVE, SSM_REAL_DENSE, SSM_COMPLEX_SHARED, SSM_COMPLEX_DENSE = 0, 1, 2, 3
_COMPLEX_MODES = (SSM_COMPLEX_SHARED, SSM_COMPLEX_DENSE)
(SSM_OP_SCAN_FWD, SSM_OP_SCAN_BWD, SSM_OP_IMPULSE, SSM_OP_PD_FWD, SSM_OP_PD_BWD, SSM_OP_COMPLEX_RTRL,
 SSM_OP_OUTPUT_SENS, SSM_OP_SENS_ROWS) = range(8)

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64


class ScanArgs(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("batch", _i64), ("channels", _i64), ("length", _i64), ("state", _i64), ("chunk_len", _i64),
                ("delta", _vp), ("x", _vp), ("A", _vp), ("Bm", _vp), ("a", _vp), ("b", _vp), ("C", _vp),
                ("r", _vp), ("phi", _vp), ("lam", _vp), ("theta", _vp), ("u", _vp), ("c", _vp), ("h0", _vp),
                ("delta_bias", _vp), ("delta_softplus", ctypes.c_int32)]


class ScanFwdOut(ctypes.Structure):
    _fields_ = [("y", _vp), ("h_last", _vp), ("ckpt", _vp)]


class ScanBwdIn(ctypes.Structure):
    _fields_ = [("gy", _vp), ("gh_last", _vp), ("ckpt", _vp)]


class ScanGrads(ctypes.Structure):
    _fields_ = [("gdelta", _vp), ("gx", _vp), ("gA", _vp), ("gBm", _vp), ("ga", _vp), ("gb", _vp),
                ("gC", _vp), ("gu", _vp), ("gr", _vp), ("gphi", _vp), ("glam", _vp), ("gtheta", _vp),
                ("gc", _vp), ("gh0", _vp), ("gdelta_bias", _vp)]


class PDArgs(ctypes.Structure):
    _fields_ = [("batch", _i64), ("heads", _i64), ("length", _i64), ("state", _i64), ("dict_size", _i64),
                ("chunk_len", _i64), ("logits", _vp), ("sel", _vp), ("dict", _vp), ("d", _vp), ("b", _vp),
                ("C", _vp), ("h0", _vp), ("dtype", ctypes.c_int32)]


class PDFwdOut(ctypes.Structure):
    _fields_ = [("y", _vp), ("sel", _vp), ("h_last", _vp), ("ckpt", _vp)]


class PDBwdIn(ctypes.Structure):
    _fields_ = [("gy", _vp), ("gh_last", _vp), ("ckpt", _vp), ("ste_logits", _vp), ("tau", ctypes.c_float)]


class PDGrads(ctypes.Structure):
    _fields_ = [("gd", _vp), ("gb", _vp), ("gC", _vp), ("gh0", _vp), ("glogits", _vp)]


_lib = None


def lib():
    """Load libssmscan.so; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library {LIB_PATH} is missing: run __graft_entry__.build() "
                               "(or python selective_state_space_chunked_amd/build.py)")
        L = ctypes.CDLL(LIB_PATH)
        L.ssm_workspace_bytes.argtypes = [ctypes.c_int, _vp, ctypes.POINTER(ctypes.c_size_t)]
        L.ssm_scan_fwd.argtypes = [ctypes.POINTER(ScanArgs), ctypes.POINTER(ScanFwdOut), _vp, ctypes.c_size_t, _vp]
        L.ssm_scan_bwd.argtypes = [ctypes.POINTER(ScanArgs), ctypes.POINTER(ScanBwdIn), ctypes.POINTER(ScanGrads),
                                   _vp, ctypes.c_size_t, _vp]
        L.ssm_impulse_sensitivity.argtypes = [ctypes.POINTER(ScanArgs), _i64, _vp, _vp, _vp, ctypes.c_size_t, _vp]
        L.ssm_output_sensitivity.argtypes = [ctypes.POINTER(ScanArgs), _i64, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
        L.ssm_sensitivity_rows.argtypes = [ctypes.POINTER(ScanArgs), _i64, ctypes.c_int32, _vp, _vp, ctypes.c_size_t,
                                           _vp]
        L.ssm_complex_rtrl.argtypes = [ctypes.POINTER(ScanArgs), _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
        L.pd_scan_fwd.argtypes = [ctypes.POINTER(PDArgs), ctypes.POINTER(PDFwdOut), _vp, ctypes.c_size_t, _vp]
        L.pd_scan_bwd.argtypes = [ctypes.POINTER(PDArgs), ctypes.POINTER(PDBwdIn), ctypes.POINTER(PDGrads),
                                  _vp, ctypes.c_size_t, _vp]
        L.ssm_status_string.restype = ctypes.c_char_p
        L.ssm_status_string.argtypes = [ctypes.c_int]
        L.ssm_last_error_detail.restype = ctypes.c_char_p
        L.ssm_abi_version.restype = ctypes.c_int
        _lib = L
    return _lib


class SSMError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{lib().ssm_status_string(status).decode()}: {detail}")
        self.status = status


def _check(rc: int):
    if rc != 0:
        raise SSMError(rc, lib().ssm_last_error_detail().decode())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(dev):
    return torch.cuda.current_stream(dev).cuda_stream


def _need(t, name, dtype=None, shape=None, device=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _workspace(op, args_ptr, device):
    n = ctypes.c_size_t(0)
    _check(lib().ssm_workspace_bytes(op, args_ptr, ctypes.byref(n)))
    if n.value == 0:
        return None, 0
    ws = torch.empty(n.value + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    return ws[off:off + n.value], n.value


def n_chunks(L, chunk_len):
    return -(-L // chunk_len)


# ---------------------------------------------------------------------------
# diagonal scans
# ---------------------------------------------------------------------------
def _scan_args(mode, *, delta=None, x=None, A=None, Bm=None, a=None, b=None, C=None, r=None, phi=None, lam=None,
               theta=None, u=None, c=None, h0=None, delta_bias=None, delta_softplus=False, chunk_len=0):
    """Marshal the scan arguments.  Selective mode: with ``delta_bias`` (D,) or
    ``delta_softplus`` set, ``delta`` is the projection output z and the scan uses
    softplus(z + delta_bias) (or z + delta_bias)."""
    if mode == SSM_REAL_SELECTIVE:
        _need(delta, "delta")
        Bsz, D, L = delta.shape
        N = A.shape[1]
        st = delta.dtype
        if st not in (torch.float32, torch.bfloat16):
            raise TypeError("delta must be float32 or bfloat16")
        dev = delta.device
        for nm, t, shp in (("x", x, (Bsz, D, L)), ("Bm", Bm, (Bsz, L, N)), ("C", C, (Bsz, L, N))):
            _need(t, nm, st, shp, dev)
        _need(A, "A", torch.float32, (D, N), dev)
        _need(h0, "h0", torch.float32, (Bsz, D, N), dev)
        _need(delta_bias, "delta_bias", torch.float32, (D,), dev)
        dt = SSM_BF16 if st == torch.bfloat16 else SSM_F32
    elif mode == SSM_REAL_DENSE:
        _need(a, "a", torch.float32)
        Bsz, D, L, N = a.shape
        dev = a.device
        _need(b, "b", torch.float32, (Bsz, D, L, N), dev)
        _need(C, "C", torch.float32, (Bsz, L, N), dev)
        _need(h0, "h0", torch.float32, (Bsz, D, N), dev)
        dt = SSM_F32
    elif mode == SSM_COMPLEX_DENSE:
        if a is None:
            raise ValueError("SSM_COMPLEX_DENSE needs the transitions a")
        _need(a, "a", torch.complex64)
        Bsz, D, L, N = a.shape
        dev = a.device
        _need(u, "u", torch.complex64, (Bsz, D, L, N), dev)
        _need(c, "c", torch.complex64, (D, N), dev)
        _need(h0, "h0", torch.complex64, (Bsz, D, N), dev)
        dt = SSM_F32
    else:
        # u: complex64 (B,H,L,M), or bfloat16 (B,H,L,M,2) holding (re, im) pairs; r, phi follow
        _need(u, "u")
        if u.dtype == torch.complex64:
            Bsz, D, L, N = u.shape
            st = torch.float32
        elif u.dtype == torch.bfloat16 and u.dim() == 5 and u.shape[-1] == 2:
            Bsz, D, L, N = u.shape[:4]
            st = torch.bfloat16
        else:
            raise TypeError("u must be complex64 (B,H,L,M) or bfloat16 (B,H,L,M,2)")
        dev = u.device
        for nm, t in (("r", r), ("phi", phi)):
            _need(t, nm, st, (Bsz, D, L), dev)
        for nm, t in (("lam", lam), ("theta", theta)):
            _need(t, nm, torch.float32, (D, N), dev)
        _need(c, "c", torch.complex64, (D, N), dev)
        _need(h0, "h0", torch.complex64, (Bsz, D, N), dev)
        dt = SSM_BF16 if st == torch.bfloat16 else SSM_F32
    args = ScanArgs(mode=mode, dtype=dt, batch=Bsz, channels=D, length=L, state=N, chunk_len=chunk_len,
                    delta=_ptr(delta), x=_ptr(x), A=_ptr(A), Bm=_ptr(Bm), a=_ptr(a), b=_ptr(b), C=_ptr(C),
                    r=_ptr(r), phi=_ptr(phi), lam=_ptr(lam), theta=_ptr(theta), u=_ptr(u), c=_ptr(c),
                    h0=_ptr(h0), delta_bias=_ptr(delta_bias), delta_softplus=int(bool(delta_softplus)))
    return args, (Bsz, D, L, N), dev


def _stream_dtype(mode, tensors):
    """Element type of the per-step streams (y, gy and their gradients) of a call."""
    if mode == SSM_REAL_SELECTIVE:
        return tensors["delta"].dtype
    if mode == SSM_COMPLEX_SHARED and tensors["u"].dtype == torch.bfloat16:
        return torch.bfloat16
    return torch.float32


def _chunk(mode, chunk_len):
    if chunk_len:
        return chunk_len
    return 256 if mode == SSM_REAL_SELECTIVE else 32


def scan_fwd(mode, *, want_y=True, want_h_last=False, want_ckpt=False, chunk_len=0, out=None, **tensors):
    """Forward scan.  Returns dict with y, h_last, ckpt (those requested).

    ``out`` may hold preallocated output tensors (keys y, h_last, ckpt).
    """
    args, (Bsz, D, L, N), dev = _scan_args(mode, chunk_len=chunk_len, **tensors)
    out = dict(out or {})
    ydt = _stream_dtype(mode, tensors)
    sdt = torch.complex64 if mode in _COMPLEX_MODES else torch.float32
    nc = n_chunks(L, _chunk(mode, chunk_len))
    if want_y and "y" not in out:
        out["y"] = torch.empty((Bsz, D, L), dtype=ydt, device=dev)
    if want_h_last and "h_last" not in out:
        out["h_last"] = torch.empty((Bsz, D, N), dtype=sdt, device=dev)
    if want_ckpt and "ckpt" not in out:
        out["ckpt"] = torch.empty((Bsz, D, nc, N), dtype=sdt, device=dev)
    o = ScanFwdOut(y=_ptr(out.get("y")), h_last=_ptr(out.get("h_last")), ckpt=_ptr(out.get("ckpt")))
    ws, nws = _workspace(SSM_OP_SCAN_FWD, ctypes.byref(args), dev)
    _check(lib().ssm_scan_fwd(ctypes.byref(args), ctypes.byref(o), _ptr(ws), nws, _stream(dev)))
    return out


_GRADS = {
    SSM_REAL_SELECTIVE: ("gdelta", "gx", "gA", "gBm", "gC", "gh0"),   # gdelta_bias on request
    SSM_REAL_DENSE: ("ga", "gb", "gC", "gh0"),
    SSM_COMPLEX_SHARED: ("gu", "gr", "gphi", "glam", "gtheta", "gc", "gh0"),
    SSM_COMPLEX_DENSE: ("ga", "gu", "gc", "gh0"),
}


def scan_bwd(mode, *, gy, gh_last=None, ckpt=None, want=None, chunk_len=0, out=None, **tensors):
    """Backward scan.  ``want`` lists gradient names (default: all of the mode)."""
    args, (Bsz, D, L, N), dev = _scan_args(mode, chunk_len=chunk_len, **tensors)
    ydt = _stream_dtype(mode, tensors)
    sdt = torch.complex64 if mode in _COMPLEX_MODES else torch.float32
    _need(gy, "gy", ydt, (Bsz, D, L), dev)
    _need(gh_last, "gh_last", sdt, (Bsz, D, N), dev)
    nc = n_chunks(L, _chunk(mode, chunk_len))
    _need(ckpt, "ckpt", sdt, (Bsz, D, nc, N), dev)
    want = tuple(want) if want is not None else _GRADS[mode]
    shapes = {
        "gdelta": ((Bsz, D, L), ydt), "gx": ((Bsz, D, L), ydt), "gA": ((D, N), torch.float32),
        "gBm": ((Bsz, L, N), ydt), "gC": ((Bsz, L, N), ydt), "gh0": ((Bsz, D, N), sdt),
        "ga": ((Bsz, D, L, N), sdt), "gb": ((Bsz, D, L, N), torch.float32),
        "gu": (((Bsz, D, L, N), torch.complex64) if ydt == torch.float32 else ((Bsz, D, L, N, 2), ydt)),
        "gr": ((Bsz, D, L), ydt), "gphi": ((Bsz, D, L), ydt), "glam": ((D, N), torch.float32),
        "gtheta": ((D, N), torch.float32), "gc": ((D, N), torch.complex64),
        "gdelta_bias": ((D,), torch.float32),
    }
    out = dict(out or {})
    for k in want:
        if k not in _GRADS[mode] and not (k == "gdelta_bias" and mode == SSM_REAL_SELECTIVE):
            raise ValueError(f"gradient {k} does not exist for mode {mode}")
        if k not in out:
            shp, dt = shapes[k]
            out[k] = torch.empty(shp, dtype=dt, device=dev)
    g = ScanGrads(**{f[0]: _ptr(out.get(f[0])) for f in ScanGrads._fields_})
    i = ScanBwdIn(gy=_ptr(gy), gh_last=_ptr(gh_last), ckpt=_ptr(ckpt))
    ws, nws = _workspace(SSM_OP_SCAN_BWD, ctypes.byref(args), dev)
    _check(lib().ssm_scan_bwd(ctypes.byref(args), ctypes.byref(i), ctypes.byref(g), _ptr(ws), nws, _stream(dev)))
    return out


def impulse_sensitivity(*, t_out=-1, want_y=True, chunk_len=0, out=None, **tensors):
    """s[b,d,t] = d y[b,d,t_out] / d x[b,d,t] of a selective real scan (and y)."""
    args, (Bsz, D, L, N), dev = _scan_args(SSM_REAL_SELECTIVE, chunk_len=chunk_len, **tensors)
    dt = tensors["delta"].dtype
    out = dict(out or {})
    if "s" not in out:
        out["s"] = torch.empty((Bsz, D, L), dtype=dt, device=dev)
    if want_y and "y" not in out:
        out["y"] = torch.empty((Bsz, D, L), dtype=dt, device=dev)
    ws, nws = _workspace(SSM_OP_IMPULSE, ctypes.byref(args), dev)
    _check(lib().ssm_impulse_sensitivity(ctypes.byref(args), int(t_out), _ptr(out.get("y")), _ptr(out["s"]),
                                         _ptr(ws), nws, _stream(dev)))
    return out


def output_sensitivity(*, t_out=-1, want_y=False, want_s_x=True, chunk_len=0, out=None, **tensors):
    """d y[b,d,t_out] / d x[b,d,t] (s_x) and / d delta[b,d,t] (s_delta) of a selective real scan (and y)."""
    args, (Bsz, D, L, N), dev = _scan_args(SSM_REAL_SELECTIVE, chunk_len=chunk_len, **tensors)
    dt = tensors["delta"].dtype
    out = dict(out or {})
    for k, want in (("s_delta", True), ("s_x", want_s_x), ("y", want_y)):
        if want and k not in out:
            out[k] = torch.empty((Bsz, D, L), dtype=dt, device=dev)
    ws, nws = _workspace(SSM_OP_OUTPUT_SENS, ctypes.byref(args), dev)
    _check(lib().ssm_output_sensitivity(ctypes.byref(args), int(t_out), _ptr(out.get("y")), _ptr(out.get("s_x")),
                                        _ptr(out["s_delta"]), _ptr(ws), nws, _stream(dev)))
    return out


def sensitivity_rows(*, t_out0, rows, out=None, **tensors):
    """s[r,b,d,t] = d y[b,d,t_out0+r] / d x[b,d,t] for r < rows (rows 1..16) of a selective real scan."""
    args, (Bsz, D, L, N), dev = _scan_args(SSM_REAL_SELECTIVE, **tensors)
    dt = tensors["delta"].dtype
    s = out if out is not None else torch.empty((int(rows), Bsz, D, L), dtype=dt, device=dev)
    ws, nws = _workspace(SSM_OP_SENS_ROWS, ctypes.byref(args), dev)
    _check(lib().ssm_sensitivity_rows(ctypes.byref(args), int(t_out0), int(rows), _ptr(s), _ptr(ws), nws,
                                      _stream(dev)))
    return s


def complex_rtrl(*, gy, gh_last=None, want_y=True, chunk_len=0, out=None, **tensors):
    """Forward-mode (real-time recurrent) glam and gtheta of the complex mode (and y).

    Loss = sum_t gy_t y_t + <gh_last, h_{L-1}>; returns dict with glam, gtheta
    ((H, M) float32) and y ((B, H, L) float32) when ``want_y``.
    """
    args, (Bsz, H, L, M), dev = _scan_args(SSM_COMPLEX_SHARED, chunk_len=chunk_len, **tensors)
    ydt = _stream_dtype(SSM_COMPLEX_SHARED, tensors)
    _need(gy, "gy", ydt, (Bsz, H, L), dev)
    _need(gh_last, "gh_last", torch.complex64, (Bsz, H, M), dev)
    out = dict(out or {})
    for k in ("glam", "gtheta"):
        if k not in out:
            out[k] = torch.empty((H, M), dtype=torch.float32, device=dev)
    if want_y and "y" not in out:
        out["y"] = torch.empty((Bsz, H, L), dtype=ydt, device=dev)
    ws, nws = _workspace(SSM_OP_COMPLEX_RTRL, ctypes.byref(args), dev)
    _check(lib().ssm_complex_rtrl(ctypes.byref(args), _ptr(gy), _ptr(gh_last), _ptr(out.get("y")),
                                  _ptr(out["glam"]), _ptr(out["gtheta"]), _ptr(ws), nws, _stream(dev)))
    return out


# ---------------------------------------------------------------------------
# PD scan
# ---------------------------------------------------------------------------
def _pd_args(*, logits=None, sel=None, dict, d, b, C, h0=None, chunk_len=0):
    """Streams (logits, d, b, C) are all float32 or all bfloat16 (the dtype of d)."""
    _need(d, "d")
    st = d.dtype
    if st not in (torch.float32, torch.bfloat16):
        raise TypeError("d must be float32 or bfloat16")
    Bsz, H, L, N = d.shape
    dev = d.device
    K = dict.shape[1]
    _need(dict, "dict", torch.int32, (H, K, N), dev)
    _need(logits, "logits", st, (Bsz, H, L, K), dev)
    _need(sel, "sel", torch.int32, (Bsz, H, L), dev)
    if logits is None and sel is None:
        raise ValueError("logits or sel is required")
    for nm, t in (("b", b), ("C", C)):
        _need(t, nm, st, (Bsz, H, L, N), dev)
    _need(h0, "h0", torch.float32, (Bsz, H, N), dev)
    args = PDArgs(batch=Bsz, heads=H, length=L, state=N, dict_size=K, chunk_len=chunk_len,
                  logits=_ptr(logits), sel=_ptr(sel), dict=_ptr(dict), d=_ptr(d), b=_ptr(b), C=_ptr(C),
                  h0=_ptr(h0), dtype=SSM_BF16 if st == torch.bfloat16 else SSM_F32)
    return args, (Bsz, H, L, N, K), dev


def pd_scan_fwd(*, want_y=True, want_sel=True, want_h_last=False, want_ckpt=False, chunk_len=0, out=None,
                **tensors):
    args, (Bsz, H, L, N, K), dev = _pd_args(chunk_len=chunk_len, **tensors)
    nc = n_chunks(L, chunk_len or 64)
    out = dict(out or {})
    if want_y and "y" not in out:
        out["y"] = torch.empty((Bsz, H, L), dtype=tensors["d"].dtype, device=dev)
    if want_sel and "sel" not in out:
        out["sel"] = torch.empty((Bsz, H, L), dtype=torch.int32, device=dev)
    if want_h_last and "h_last" not in out:
        out["h_last"] = torch.empty((Bsz, H, N), dtype=torch.float32, device=dev)
    if want_ckpt and "ckpt" not in out:
        out["ckpt"] = torch.empty((Bsz, H, nc, N), dtype=torch.float32, device=dev)
    o = PDFwdOut(y=_ptr(out.get("y")), sel=_ptr(out.get("sel")), h_last=_ptr(out.get("h_last")),
                 ckpt=_ptr(out.get("ckpt")))
    ws, nws = _workspace(SSM_OP_PD_FWD, ctypes.byref(args), dev)
    _check(lib().pd_scan_fwd(ctypes.byref(args), ctypes.byref(o), _ptr(ws), nws, _stream(dev)))
    return out


def pd_scan_bwd(*, gy, gh_last=None, ckpt=None, want=("gd", "gb", "gC", "gh0"), ste_logits=None, tau=1.0,
                chunk_len=0, out=None, **tensors):
    """PD backward with the selection held fixed.  ``want`` may also name
    "glogits", the straight-through surrogate gradient of ``ste_logits``
    (B, H, L, K) through softmax(ste_logits / tau)."""
    args, (Bsz, H, L, N, K), dev = _pd_args(chunk_len=chunk_len, **tensors)
    st = tensors["d"].dtype
    _need(gy, "gy", st, (Bsz, H, L), dev)
    _need(gh_last, "gh_last", torch.float32, (Bsz, H, N), dev)
    nc = n_chunks(L, chunk_len or 64)
    _need(ckpt, "ckpt", torch.float32, (Bsz, H, nc, N), dev)
    _need(ste_logits, "ste_logits", st, (Bsz, H, L, K), dev)
    out = dict(out or {})
    shapes = {"gd": (Bsz, H, L, N), "gb": (Bsz, H, L, N), "gC": (Bsz, H, L, N), "gh0": (Bsz, H, N),
              "glogits": (Bsz, H, L, K)}
    for k in want:
        if k not in shapes:
            raise ValueError(f"unknown PD gradient {k}")
        if k not in out:
            out[k] = torch.empty(shapes[k], dtype=torch.float32 if k == "gh0" else st, device=dev)
    g = PDGrads(**{f[0]: _ptr(out.get(f[0])) for f in PDGrads._fields_})
    i = PDBwdIn(gy=_ptr(gy), gh_last=_ptr(gh_last), ckpt=_ptr(ckpt), ste_logits=_ptr(ste_logits), tau=float(tau))
    ws, nws = _workspace(SSM_OP_PD_BWD, ctypes.byref(args), dev)
    _check(lib().pd_scan_bwd(ctypes.byref(args), ctypes.byref(i), ctypes.byref(g), _ptr(ws), nws, _stream(dev)))
    return out
