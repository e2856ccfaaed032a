"""ctypes binding of libssmscan.so (include/ssmscan.h).

Argument marshalling only: input tensors and caller-supplied outputs
(``out=``) are checked for device, dtype, shape and contiguity, missing
outputs and the workspace are allocated on the tensors' device (with
torch.empty, or with the allocator installed by ``set_allocator``), and every
step of the scan runs in the library's HIP kernels on torch's current stream.
There is no CPU fallback: tensors that are not on a GPU are rejected, and if
the library is missing or a call fails, this module raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libssmscan.so")

SSM_F32, SSM_BF16 = 0, 1
SSM_EULER, SSM_ZOH = 0, 1
# roles of the strided views (ssm_layout)
(V_DELTA, V_X, V_A, V_BM, V_C, V_Y, V_GY, V_GDELTA, V_GX, V_R, V_PHI, V_U, V_LAM, V_THETA, V_CC, V_LOGITS,
 V_PD_D, V_PD_B, V_PD_C, V_DICT) = range(20)
V_COUNT = 20
SSM_REAL_SELECTIVE, SSM_REAL_DENSE, SSM_COMPLEX_SHARED, SSM_COMPLEX_DENSE, SSM_HEAD_SCALAR = 0, 1, 2, 3, 4
_COMPLEX_MODES = (SSM_COMPLEX_SHARED, SSM_COMPLEX_DENSE)
(SSM_OP_SCAN_FWD, SSM_OP_SCAN_BWD, SSM_OP_IMPULSE, SSM_OP_PD_FWD, SSM_OP_PD_BWD, SSM_OP_COMPLEX_RTRL,
 SSM_OP_OUTPUT_SENS, SSM_OP_SENS_ROWS) = range(8)

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64


class Layout(ctypes.Structure):
    _fields_ = [("given", ctypes.c_uint64), ("stride", (ctypes.c_int64 * 4) * V_COUNT)]


class _Views:
    """The strides of the tensors of one call that are views (non-dense or broadcast)."""

    def __init__(self):
        self.lay = Layout()
        self.any = False

    def set(self, role, strides, dense):
        strides = tuple(int(v) for v in strides)
        if strides != tuple(int(v) for v in dense):
            self.lay.given |= 1 << role
            for i, v in enumerate(strides):
                self.lay.stride[role][i] = v
            self.any = True

    def ptr(self):
        return ctypes.pointer(self.lay) if self.any else None


def _dense_strides(shape):
    st, acc = [], 1
    for n in reversed(shape):
        st.append(acc)
        acc *= int(n)
    return tuple(reversed(st))


class ScanArgs(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("batch", _i64), ("channels", _i64), ("length", _i64), ("state", _i64), ("chunk_len", _i64),
                ("delta", _vp), ("x", _vp), ("A", _vp), ("Bm", _vp), ("a", _vp), ("b", _vp), ("C", _vp),
                ("r", _vp), ("phi", _vp), ("lam", _vp), ("theta", _vp), ("u", _vp), ("c", _vp), ("h0", _vp),
                ("delta_bias", _vp), ("delta_softplus", ctypes.c_int32), ("discretization", ctypes.c_int32),
                ("layout", ctypes.POINTER(Layout)), ("head_dim", _i64)]


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
                ("C", _vp), ("h0", _vp), ("dtype", ctypes.c_int32), ("layout", ctypes.POINTER(Layout))]


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
        L.ssm_scan_fwd_noalloc.argtypes = [ctypes.POINTER(ScanArgs), ctypes.POINTER(ScanFwdOut), _vp]
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


def _need(t, name, dtype=None, shape=None, device=None, view=False):
    """Check a tensor argument.  ``view``: a strided view is accepted (any strides with the last dimension
    contiguous; the library takes its strides), otherwise the tensor must be contiguous."""
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
    if view:
        if t.dim() > 1 and t.shape[-1] > 1 and t.stride(-1) != 1:
            raise ValueError(f"{name}: the last dimension must be contiguous (stride 1)")
    elif not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


_allocator = None


def set_allocator(fn):
    """Install ``fn(shape, dtype, device, role) -> tensor`` for the outputs this module allocates
    (role "output") and the workspaces (role "workspace", uint8); None restores torch.empty.  A caller
    can route allocations to its own memory pool, or fill them with a sentinel (tests fill outputs
    with NaN, integers with -1, so an element a kernel never writes cannot pass as a result)."""
    global _allocator
    _allocator = fn


def _alloc(shape, dtype, device, role="output"):
    if _allocator is not None:
        t = _allocator(tuple(shape), dtype, device, role)
        if tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != torch.device(device) \
                or not t.is_contiguous():
            raise ValueError(f"allocator returned {tuple(t.shape)} {t.dtype} on {t.device}, "
                             f"expected {tuple(shape)} {dtype} on {device}")
        return t
    return torch.empty(shape, dtype=dtype, device=device)


def _out(out, key, shape, dtype, device, view=False):
    """out[key]: the caller's tensor, checked like an input, or a new one of the given shape and dtype.
    ``view``: the caller's tensor may be a strided view (distinct elements, last dimension contiguous)."""
    if key in out and out[key] is not None:
        t = _need(out[key], f"out[{key!r}]", dtype, shape, device, view=view)
        if view and not _distinct(t):
            raise ValueError(f"out[{key!r}]: an output view needs distinct elements (no stride 0)")
        return t
    out[key] = _alloc(shape, dtype, device)
    return out[key]


def _distinct(t):
    """True when no two indices of t address the same element."""
    dims = sorted((st, n) for st, n in zip(t.stride(), t.shape) if n > 1)
    span = 1
    for st, n in dims:
        if st < span:
            return False
        span += st * (n - 1)
    return True


def _on_gpu(device):
    """The library takes device pointers only: host tensors would reach the kernels as bad addresses."""
    if torch.device(device).type != "cuda":
        raise ValueError(f"tensors must be on a GPU device (got {device}); there is no CPU path")


def _workspace(op, args_ptr, device):
    n = ctypes.c_size_t(0)
    _check(lib().ssm_workspace_bytes(op, args_ptr, ctypes.byref(n)))
    if n.value == 0:
        return None, 0
    ws = _alloc((n.value + 256,), torch.uint8, device, "workspace")
    off = (-ws.data_ptr()) % 256
    return ws[off:off + n.value], n.value


def n_chunks(L, chunk_len):
    return -(-L // chunk_len)


# ---------------------------------------------------------------------------
# diagonal scans
# ---------------------------------------------------------------------------
def _scan_args(mode, *, delta=None, x=None, A=None, Bm=None, a=None, b=None, C=None, r=None, phi=None, lam=None,
               theta=None, u=None, c=None, h0=None, delta_bias=None, delta_softplus=False, discretization=SSM_EULER,
               chunk_len=0):
    """Marshal the scan arguments.  Selective mode: with ``delta_bias`` (D,) or
    ``delta_softplus`` set, ``delta`` is the projection output z and the scan uses
    softplus(z + delta_bias) (or z + delta_bias); ``discretization`` SSM_ZOH selects the
    zero-order-hold input term.  Inputs may be strided views (slices, ``expand``): the
    selective delta, x, A, Bm, C (Bm, C either (B, L, N), shared by the channels, or
    (B, D, L, N), per channel unless expanded along D) and the complex r, phi, u, lam,
    theta, c; their strides go to the library."""
    vw = _Views()
    perd = False
    head_dim = 0
    if mode == SSM_HEAD_SCALAR:
        # delta (B,H,L) and A (H) one per head; x (B,H*P,L); Bm, C (B,L,N)
        _need(delta, "delta", view=True)
        Bsz, H, L = delta.shape
        st = delta.dtype
        if st not in (torch.float32, torch.bfloat16):
            raise TypeError("delta must be float32 or bfloat16")
        dev = delta.device
        _need(x, "x", view=True)
        if x.dim() != 3 or x.shape[0] != Bsz or x.shape[2] != L or x.shape[1] % H:
            raise ValueError(f"x has shape {tuple(x.shape)}; expected (B, H*P, L) with B={Bsz} H={H} L={L}")
        D = x.shape[1]
        head_dim = D // H
        N = Bm.shape[-1]
        _need(x, "x", st, (Bsz, D, L), dev, view=True)
        for nm, t, role in (("Bm", Bm, V_BM), ("C", C, V_C)):
            _need(t, nm, st, (Bsz, L, N), dev, view=True)
            vw.set(role, (t.stride(0), 0, t.stride(1), t.stride(2)), (L * N, 0, N, 1))
        _need(A, "A", torch.float32, (H,), dev, view=True)
        _need(h0, "h0", torch.float32, (Bsz, D, N), dev)
        vw.set(V_DELTA, delta.stride(), (H * L, L, 1))
        vw.set(V_X, x.stride(), (D * L, L, 1))
        vw.set(V_A, A.stride(), (1,))
        dt = SSM_BF16 if st == torch.bfloat16 else SSM_F32
    elif mode == SSM_REAL_SELECTIVE:
        _need(delta, "delta", view=True)
        Bsz, D, L = delta.shape
        N = A.shape[1]
        st = delta.dtype
        if st not in (torch.float32, torch.bfloat16):
            raise TypeError("delta must be float32 or bfloat16")
        dev = delta.device
        _need(x, "x", st, (Bsz, D, L), dev, view=True)
        for nm, t, role in (("Bm", Bm, V_BM), ("C", C, V_C)):
            if t is not None and t.dim() == 4:
                _need(t, nm, st, (Bsz, D, L, N), dev, view=True)
                vw.set(role, t.stride(), (L * N, 0, N, 1))
                perd = perd or (t.stride(1) != 0 and D > 1)
            else:
                _need(t, nm, st, (Bsz, L, N), dev, view=True)
                if t is not None:
                    vw.set(role, (t.stride(0), 0, t.stride(1), t.stride(2)), (L * N, 0, N, 1))
        _need(A, "A", torch.float32, (D, N), dev, view=True)
        _need(h0, "h0", torch.float32, (Bsz, D, N), dev)
        _need(delta_bias, "delta_bias", torch.float32, (D,), dev)
        vw.set(V_DELTA, delta.stride(), (D * L, L, 1))
        vw.set(V_X, x.stride(), (D * L, L, 1))
        vw.set(V_A, A.stride(), (N, 1))
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
        _need(u, "u", view=True)
        if u.dtype == torch.complex64:
            Bsz, D, L, N = u.shape
            st = torch.float32
            vw.set(V_U, u.stride(), _dense_strides(u.shape))
        elif u.dtype == torch.bfloat16 and u.dim() == 5 and u.shape[-1] == 2:
            Bsz, D, L, N = u.shape[:4]
            st = torch.bfloat16
            if u.stride(3) != 2 and N > 1:
                raise ValueError("u: the (re, im) pairs of the modes must be contiguous")
            if any(v % 2 for v in u.stride()[:3]):
                raise ValueError("u: strides must be whole (re, im) pairs")
            vw.set(V_U, tuple(v // 2 for v in u.stride()[:3]) + (1,), _dense_strides(u.shape[:4]))
        else:
            raise TypeError("u must be complex64 (B,H,L,M) or bfloat16 (B,H,L,M,2)")
        dev = u.device
        for nm, t, role in (("r", r, V_R), ("phi", phi, V_PHI)):
            _need(t, nm, st, (Bsz, D, L), dev, view=True)
            vw.set(role, t.stride(), (D * L, L, 1))
        for nm, t, role in (("lam", lam, V_LAM), ("theta", theta, V_THETA)):
            _need(t, nm, torch.float32, (D, N), dev, view=True)
            vw.set(role, t.stride(), (N, 1))
        _need(c, "c", torch.complex64, (D, N), dev, view=True)
        vw.set(V_CC, c.stride(), (N, 1))
        _need(h0, "h0", torch.complex64, (Bsz, D, N), dev)
        dt = SSM_BF16 if st == torch.bfloat16 else SSM_F32
    args = ScanArgs(mode=mode, dtype=dt, batch=Bsz, channels=D, length=L, state=N, chunk_len=chunk_len,
                    delta=_ptr(delta), x=_ptr(x), A=_ptr(A), Bm=_ptr(Bm), a=_ptr(a), b=_ptr(b), C=_ptr(C),
                    r=_ptr(r), phi=_ptr(phi), lam=_ptr(lam), theta=_ptr(theta), u=_ptr(u), c=_ptr(c),
                    h0=_ptr(h0), delta_bias=_ptr(delta_bias), delta_softplus=int(bool(delta_softplus)),
                    discretization=int(discretization), head_dim=head_dim)
    args._views = vw          # kept with the struct: the library reads it during the call
    args._perd = perd
    args.layout = vw.ptr()
    return args, (Bsz, D, L, N), dev


def _set_layout(args):
    args.layout = args._views.ptr()


def _stream_dtype(mode, tensors):
    """Element type of the per-step streams (y, gy and their gradients) of a call."""
    if mode in (SSM_REAL_SELECTIVE, SSM_HEAD_SCALAR):
        return tensors["delta"].dtype
    if mode == SSM_COMPLEX_SHARED and tensors["u"].dtype == torch.bfloat16:
        return torch.bfloat16
    return torch.float32


def _chunk(mode, chunk_len):
    if chunk_len:
        return chunk_len
    return {SSM_REAL_SELECTIVE: 256, SSM_HEAD_SCALAR: 64}.get(mode, 32)


def scan_fwd(mode, *, want_y=True, want_h_last=False, want_ckpt=False, chunk_len=0, out=None, **tensors):
    """Forward scan.  Returns dict with y, h_last, ckpt (those requested).

    ``out`` may hold preallocated output tensors (keys y, h_last, ckpt).
    """
    return _scan_fwd(mode, want_y, want_h_last, want_ckpt, chunk_len, out, tensors, noalloc=False)


def scan_fwd_noalloc(mode, *, want_y=True, want_h_last=False, want_ckpt=False, chunk_len=0, out=None, **tensors):
    """ssm_scan_fwd_noalloc: the forward scan with the library's static device scratch in place of a
    workspace (nothing is allocated when ``out`` holds every requested output).  Same results as
    scan_fwd; calls that overlap on one device race on the shared scratch."""
    return _scan_fwd(mode, want_y, want_h_last, want_ckpt, chunk_len, out, tensors, noalloc=True)


def _scan_fwd(mode, want_y, want_h_last, want_ckpt, chunk_len, out, tensors, noalloc):
    args, (Bsz, D, L, N), dev = _scan_args(mode, chunk_len=chunk_len, **tensors)
    out = dict(out or {})
    ydt = _stream_dtype(mode, tensors)
    sdt = torch.complex64 if mode in _COMPLEX_MODES else torch.float32
    nc = n_chunks(L, _chunk(mode, chunk_len))
    sel = mode in (SSM_REAL_SELECTIVE, SSM_HEAD_SCALAR)
    for k, want, shp, dt in (("y", want_y, (Bsz, D, L), ydt), ("h_last", want_h_last, (Bsz, D, N), sdt),
                             ("ckpt", want_ckpt, (Bsz, D, nc, N), sdt)):
        if want or out.get(k) is not None:
            _out(out, k, shp, dt, dev, view=sel and k == "y")
    if sel and out.get("y") is not None:
        args._views.set(V_Y, out["y"].stride(), (D * L, L, 1))
        _set_layout(args)
    _on_gpu(dev)
    o = ScanFwdOut(y=_ptr(out.get("y")), h_last=_ptr(out.get("h_last")), ckpt=_ptr(out.get("ckpt")))
    if noalloc:
        _check(lib().ssm_scan_fwd_noalloc(ctypes.byref(args), ctypes.byref(o), _stream(dev)))
        return out
    ws, nws = _workspace(SSM_OP_SCAN_FWD, ctypes.byref(args), dev)
    _check(lib().ssm_scan_fwd(ctypes.byref(args), ctypes.byref(o), _ptr(ws), nws, _stream(dev)))
    return out


_GRADS = {
    SSM_REAL_SELECTIVE: ("gdelta", "gx", "gA", "gBm", "gC", "gh0"),   # gdelta_bias on request
    SSM_HEAD_SCALAR: ("gdelta", "gx", "gA", "gBm", "gC", "gh0"),
    SSM_REAL_DENSE: ("ga", "gb", "gC", "gh0"),
    SSM_COMPLEX_SHARED: ("gu", "gr", "gphi", "glam", "gtheta", "gc", "gh0"),
    SSM_COMPLEX_DENSE: ("ga", "gu", "gc", "gh0"),
}


def scan_bwd(mode, *, gy, gh_last=None, ckpt=None, want=None, chunk_len=0, out=None, **tensors):
    """Backward scan.  ``want`` lists gradient names (default: all of the mode)."""
    args, (Bsz, D, L, N), dev = _scan_args(mode, chunk_len=chunk_len, **tensors)
    ydt = _stream_dtype(mode, tensors)
    sdt = torch.complex64 if mode in _COMPLEX_MODES else torch.float32
    sel = mode in (SSM_REAL_SELECTIVE, SSM_HEAD_SCALAR)
    _need(gy, "gy", ydt, (Bsz, D, L), dev, view=sel)
    _need(gh_last, "gh_last", sdt, (Bsz, D, N), dev)
    nc = n_chunks(L, _chunk(mode, chunk_len))
    _need(ckpt, "ckpt", sdt, (Bsz, D, nc, N), dev)
    want = tuple(want) if want is not None else _GRADS[mode]
    gbc = (Bsz, D, L, N) if args._perd else (Bsz, L, N)   # per-channel B_t, C_t: per-channel gradients
    shapes = {
        "gdelta": ((Bsz, D, L), ydt), "gx": ((Bsz, D, L), ydt), "gA": ((D, N), torch.float32),
        "gBm": (gbc, ydt), "gC": (gbc, ydt), "gh0": ((Bsz, D, N), sdt),
        "ga": ((Bsz, D, L, N), sdt), "gb": ((Bsz, D, L, N), torch.float32),
        "gu": (((Bsz, D, L, N), torch.complex64) if ydt == torch.float32 else ((Bsz, D, L, N, 2), ydt)),
        "gr": ((Bsz, D, L), ydt), "gphi": ((Bsz, D, L), ydt), "glam": ((D, N), torch.float32),
        "gtheta": ((D, N), torch.float32), "gc": ((D, N), torch.complex64),
        "gdelta_bias": ((D,), torch.float32),
    }
    if mode == SSM_HEAD_SCALAR:   # per-head step sizes and transitions
        H = tensors["delta"].shape[1]
        shapes["gdelta"] = ((Bsz, H, L), ydt)
        shapes["gA"] = ((H,), torch.float32)
    out = dict(out or {})
    def exists(k):
        return k in _GRADS[mode] or (k == "gdelta_bias" and mode == SSM_REAL_SELECTIVE)
    for k in set(want) | {k for k, v in out.items() if v is not None}:
        if not exists(k):
            raise ValueError(f"gradient {k} does not exist for mode {mode}")
        _out(out, k, *shapes[k], dev, view=sel and k in ("gdelta", "gx"))
    if sel:
        args._views.set(V_GY, gy.stride(), (D * L, L, 1))
        for k, role in (("gdelta", V_GDELTA), ("gx", V_GX)):
            if out.get(k) is not None:
                args._views.set(role, out[k].stride(), _dense_strides(out[k].shape))
        _set_layout(args)
    _on_gpu(dev)
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
    _out(out, "s", (Bsz, D, L), dt, dev)
    if want_y or out.get("y") is not None:
        _out(out, "y", (Bsz, D, L), dt, dev)
    _on_gpu(dev)
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
        if want or out.get(k) is not None:
            _out(out, k, (Bsz, D, L), dt, dev)
    _on_gpu(dev)
    ws, nws = _workspace(SSM_OP_OUTPUT_SENS, ctypes.byref(args), dev)
    _check(lib().ssm_output_sensitivity(ctypes.byref(args), int(t_out), _ptr(out.get("y")), _ptr(out.get("s_x")),
                                        _ptr(out["s_delta"]), _ptr(ws), nws, _stream(dev)))
    return out


def sensitivity_rows(*, t_out0, rows, out=None, **tensors):
    """s[r,b,d,t] = d y[b,d,t_out0+r] / d x[b,d,t] for r < rows (rows 1..16) of a selective real scan."""
    args, (Bsz, D, L, N), dev = _scan_args(SSM_REAL_SELECTIVE, **tensors)
    dt = tensors["delta"].dtype
    shp = (int(rows), Bsz, D, L)
    s = _need(out, "out", dt, shp, dev) if out is not None else _alloc(shp, dt, dev)
    _on_gpu(dev)
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
        _out(out, k, (H, M), torch.float32, dev)
    if want_y or out.get("y") is not None:
        _out(out, "y", (Bsz, H, L), ydt, dev)
    _on_gpu(dev)
    ws, nws = _workspace(SSM_OP_COMPLEX_RTRL, ctypes.byref(args), dev)
    _check(lib().ssm_complex_rtrl(ctypes.byref(args), _ptr(gy), _ptr(gh_last), _ptr(out.get("y")),
                                  _ptr(out["glam"]), _ptr(out["gtheta"]), _ptr(ws), nws, _stream(dev)))
    return out


# ---------------------------------------------------------------------------
# PD scan
# ---------------------------------------------------------------------------
def _pd_args(*, logits=None, sel=None, dict, d, b, C, h0=None, chunk_len=0):
    """Streams (logits, d, b, C) are all float32 or all bfloat16 (the dtype of d).  logits, d, b, C and
    the dictionary may be strided views (a dictionary expanded along the heads is shared by them)."""
    _need(d, "d", view=True)
    st = d.dtype
    if st not in (torch.float32, torch.bfloat16):
        raise TypeError("d must be float32 or bfloat16")
    Bsz, H, L, N = d.shape
    dev = d.device
    K = dict.shape[1]
    vw = _Views()
    _need(dict, "dict", torch.int32, (H, K, N), dev, view=True)
    _need(logits, "logits", st, (Bsz, H, L, K), dev, view=True)
    _need(sel, "sel", torch.int32, (Bsz, H, L), dev)
    if logits is None and sel is None:
        raise ValueError("logits or sel is required")
    for nm, t in (("b", b), ("C", C)):
        _need(t, nm, st, (Bsz, H, L, N), dev, view=True)
    _need(h0, "h0", torch.float32, (Bsz, H, N), dev)
    for t, role in ((d, V_PD_D), (b, V_PD_B), (C, V_PD_C)):
        vw.set(role, t.stride(), (H * L * N, L * N, N, 1))
    if logits is not None:
        vw.set(V_LOGITS, logits.stride(), (H * L * K, L * K, K, 1))
    vw.set(V_DICT, dict.stride(), (K * N, N, 1))
    args = PDArgs(batch=Bsz, heads=H, length=L, state=N, dict_size=K, chunk_len=chunk_len,
                  logits=_ptr(logits), sel=_ptr(sel), dict=_ptr(dict), d=_ptr(d), b=_ptr(b), C=_ptr(C),
                  h0=_ptr(h0), dtype=SSM_BF16 if st == torch.bfloat16 else SSM_F32)
    args._views = vw
    args.layout = vw.ptr()
    return args, (Bsz, H, L, N, K), dev


def pd_scan_fwd(*, want_y=True, want_sel=True, want_h_last=False, want_ckpt=False, chunk_len=0, out=None,
                **tensors):
    args, (Bsz, H, L, N, K), dev = _pd_args(chunk_len=chunk_len, **tensors)
    nc = n_chunks(L, chunk_len or 64)
    out = dict(out or {})
    for k, want, shp, dt in (("y", want_y, (Bsz, H, L), tensors["d"].dtype),
                             ("sel", want_sel, (Bsz, H, L), torch.int32),
                             ("h_last", want_h_last, (Bsz, H, N), torch.float32),
                             ("ckpt", want_ckpt, (Bsz, H, nc, N), torch.float32)):
        if want or out.get(k) is not None:
            _out(out, k, shp, dt, dev)
    _on_gpu(dev)
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
    for k in set(want) | {k for k, v in out.items() if v is not None}:
        if k not in shapes:
            raise ValueError(f"unknown PD gradient {k}")
        _out(out, k, shapes[k], torch.float32 if k == "gh0" else st, dev)
    _on_gpu(dev)
    g = PDGrads(**{f[0]: _ptr(out.get(f[0])) for f in PDGrads._fields_})
    i = PDBwdIn(gy=_ptr(gy), gh_last=_ptr(gh_last), ckpt=_ptr(ckpt), ste_logits=_ptr(ste_logits), tau=float(tau))
    ws, nws = _workspace(SSM_OP_PD_BWD, ctypes.byref(args), dev)
    _check(lib().pd_scan_bwd(ctypes.byref(args), ctypes.byref(i), ctypes.byref(g), _ptr(ws), nws, _stream(dev)))
    return out
