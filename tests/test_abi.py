"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects invalid arguments on the host before anything is
enqueued (no compute call reaches the device here)."""
import ctypes
import os
import re

import pytest

from selective_state_space_chunked_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssmscan.h")


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", src, flags=re.M)))


def test_exports_every_declared_function():
    names = header_functions()
    assert {"ssm_scan_fwd", "ssm_scan_bwd", "ssm_impulse_sensitivity", "pd_scan_fwd", "pd_scan_bwd",
            "ssm_complex_rtrl", "ssm_output_sensitivity", "ssm_sensitivity_rows",
            "ssm_workspace_bytes"} <= set(names)
    lib = B.lib()
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_header_constants_match_binding():
    src = open(HEADER).read()
    consts = dict((k, int(v)) for k, v in re.findall(r"#define\s+(SSM_\w+)\s+(-?\d+)", src))
    assert consts["SSM_F32"] == B.SSM_F32 and consts["SSM_BF16"] == B.SSM_BF16
    assert consts["SSM_REAL_SELECTIVE"] == B.SSM_REAL_SELECTIVE
    assert consts["SSM_REAL_DENSE"] == B.SSM_REAL_DENSE
    assert consts["SSM_COMPLEX_SHARED"] == B.SSM_COMPLEX_SHARED
    assert consts["SSM_COMPLEX_DENSE"] == B.SSM_COMPLEX_DENSE
    assert consts["SSM_HEAD_SCALAR"] == B.SSM_HEAD_SCALAR
    assert consts["SSM_OP_PD_BWD"] == B.SSM_OP_PD_BWD
    assert consts["SSM_OP_COMPLEX_RTRL"] == B.SSM_OP_COMPLEX_RTRL
    assert consts["SSM_OP_OUTPUT_SENS"] == B.SSM_OP_OUTPUT_SENS
    assert consts["SSM_OP_SENS_ROWS"] == B.SSM_OP_SENS_ROWS
    assert B.lib().ssm_abi_version() == consts["SSM_ABI_VERSION"]


def test_struct_layouts():
    # 2 x int32 + 5 x int64 + 14 pointers
    # + delta_bias pointer + delta_softplus, discretization int32 + layout pointer
    assert ctypes.sizeof(B.ScanArgs) == 8 + 5 * 8 + 15 * 8 + 8 + 8 + 8   # + head_dim
    assert ctypes.sizeof(B.ScanGrads) == 15 * 8
    assert ctypes.sizeof(B.PDArgs) == 6 * 8 + 7 * 8 + 8 + 8   # + dtype (int32, padded) + layout pointer
    assert ctypes.sizeof(B.Layout) == 8 + 20 * 4 * 8
    assert ctypes.sizeof(B.PDBwdIn) == 4 * 8 + 8   # 4 pointers + float tau (padded)
    assert ctypes.sizeof(B.PDGrads) == 5 * 8


FAKE = 1 << 20  # never dereferenced: validation fails or only sizes are computed


def sel_args(**over):
    a = B.ScanArgs(mode=B.SSM_REAL_SELECTIVE, dtype=B.SSM_F32, batch=2, channels=32, length=1000, state=16,
                   chunk_len=0, delta=FAKE, x=FAKE * 2, A=FAKE * 3, Bm=FAKE * 4, C=FAKE * 5)
    for k, v in over.items():
        setattr(a, k, v)
    return a


def ws_bytes(op, args):
    n = ctypes.c_size_t(123)
    rc = B.lib().ssm_workspace_bytes(op, ctypes.byref(args), ctypes.byref(n))
    return rc, n.value


def status(name):
    src = open(HEADER).read()
    return int(re.search(r"#define\s+%s\s+(-?\d+)" % name, src).group(1))


def test_workspace_query_valid():
    for op in (B.SSM_OP_SCAN_FWD, B.SSM_OP_SCAN_BWD, B.SSM_OP_IMPULSE):
        rc, n = ws_bytes(op, sel_args())
        assert rc == 0, B.lib().ssm_last_error_detail()
        assert n > 0 and n % 1 == 0


@pytest.mark.parametrize("over,code", [
    (dict(delta=None), "SSM_ERR_NULL"),
    (dict(C=None), "SSM_ERR_NULL"),
    (dict(batch=-1), "SSM_ERR_SHAPE"),
    (dict(length=-1), "SSM_ERR_SHAPE"),
    (dict(state=0), "SSM_ERR_SHAPE"),
    (dict(state=17), "SSM_ERR_SHAPE"),
    (dict(dtype=7), "SSM_ERR_DTYPE"),
    (dict(mode=9), "SSM_ERR_UNSUPPORTED"),
    (dict(chunk_len=100), "SSM_ERR_UNSUPPORTED"),
    (dict(x=FAKE * 2 + 2), "SSM_ERR_LAYOUT"),
    (dict(delta_softplus=2), "SSM_ERR_SHAPE"),
    (dict(delta_bias=FAKE * 6 + 2), "SSM_ERR_LAYOUT"),
])
def test_validation_errors(over, code):
    rc, _ = ws_bytes(B.SSM_OP_SCAN_FWD, sel_args(**over))
    assert rc == status(code), (rc, B.lib().ssm_last_error_detail())
    assert B.lib().ssm_last_error_detail()
    assert B.lib().ssm_status_string(rc).decode() == code


@pytest.mark.parametrize("over", [dict(batch=0), dict(channels=0), dict(length=0)])
def test_empty_problems_are_valid(over):
    """No batch rows, channels or steps: a valid call with an empty workspace; streamed inputs and outputs
    with no elements may be NULL."""
    L = B.lib()
    for op in (B.SSM_OP_SCAN_FWD, B.SSM_OP_SCAN_BWD):
        for args in (sel_args(**over), cplx_args(**over)):
            rc, n = ws_bytes(op, args)
            assert rc == 0 and n == 0, (op, over, L.ssm_last_error_detail())
    a = sel_args(delta=None, x=None, Bm=None, C=None, A=None, **over)
    assert ws_bytes(B.SSM_OP_SCAN_FWD, a) == (0, 0)
    rc, _ = ws_bytes(B.SSM_OP_SCAN_FWD, sel_args(delta=None))   # not empty: inputs are required
    assert rc == status("SSM_ERR_NULL")
    if over.get("length") != 0:   # the sensitivity calls need 0 <= t_out < L
        assert ws_bytes(B.SSM_OP_IMPULSE, sel_args(**over)) == (0, 0)
        assert ws_bytes(B.SSM_OP_SENS_ROWS, sel_args(**over)) == (0, 0)
    else:
        assert ws_bytes(B.SSM_OP_IMPULSE, sel_args(**over))[0] == status("SSM_ERR_SHAPE")


def test_bf16_only_for_selective():
    a = sel_args(mode=B.SSM_REAL_DENSE, dtype=B.SSM_BF16, a=FAKE * 6, b=FAKE * 7)
    rc, _ = ws_bytes(B.SSM_OP_SCAN_FWD, a)
    assert rc == status("SSM_ERR_DTYPE")


def test_errors_before_enqueue():
    """Entry points reject bad calls without touching the device."""
    L = B.lib()
    a = sel_args()
    out = B.ScanFwdOut(y=FAKE * 2 + 64, h_last=None, ckpt=None)  # y overlaps x
    rc = L.ssm_scan_fwd(ctypes.byref(a), ctypes.byref(out), None, 0, None)
    assert rc == status("SSM_ERR_LAYOUT"), L.ssm_last_error_detail()
    out = B.ScanFwdOut(y=FAKE * 64, h_last=None, ckpt=None)
    rc = L.ssm_scan_fwd(ctypes.byref(a), ctypes.byref(out), None, 0, None)  # no workspace
    assert rc == status("SSM_ERR_WORKSPACE"), L.ssm_last_error_detail()
    rc = L.ssm_scan_fwd(ctypes.byref(a), ctypes.byref(out), FAKE * 128, 16, None)  # too small
    assert rc == status("SSM_ERR_WORKSPACE")
    rc = L.ssm_scan_fwd(ctypes.byref(a), None, None, 0, None)
    assert rc == status("SSM_ERR_NULL")
    gi = B.ScanBwdIn(gy=None)
    gr = B.ScanGrads()
    rc = L.ssm_scan_bwd(ctypes.byref(a), ctypes.byref(gi), ctypes.byref(gr), None, 0, None)
    assert rc == status("SSM_ERR_NULL")
    rc = L.ssm_impulse_sensitivity(ctypes.byref(a), 1000, None, FAKE * 64, None, 0, None)
    assert rc == status("SSM_ERR_SHAPE")  # t_out outside [0, L)


def test_sensitivity_workspace_grows_by_a_few_numbers_per_chunk():
    """The sensitivity path needs O(n_chunks) scratch: per chunk a few numbers, no per-step state."""
    _, n1 = ws_bytes(B.SSM_OP_IMPULSE, sel_args(length=16384, batch=1, channels=64))
    _, n2 = ws_bytes(B.SSM_OP_IMPULSE, sel_args(length=131072, batch=1, channels=64))
    chunks1, chunks2 = 16384 // 256, 131072 // 256
    per_chunk = (n2 - n1) / (chunks2 - chunks1)
    # at most ~ (3 segment arrays x N floats + one float + one double) per chunk and channel
    assert per_chunk <= 64 * (3 * 16 * 4 + 4 + 8) + 64


def pd_args(**over):
    a = B.PDArgs(batch=2, heads=4, length=500, state=16, dict_size=8, chunk_len=0, logits=FAKE, sel=None,
                 dict=FAKE * 2, d=FAKE * 3, b=FAKE * 4, C=FAKE * 5)
    for k, v in over.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("over,code", [
    (dict(logits=None), "SSM_ERR_NULL"),
    (dict(dict=None), "SSM_ERR_NULL"),
    (dict(state=17), "SSM_ERR_SHAPE"),
    (dict(dict_size=65), "SSM_ERR_SHAPE"),
    (dict(length=-1), "SSM_ERR_SHAPE"),
    (dict(state=0), "SSM_ERR_SHAPE"),
    (dict(chunk_len=32), "SSM_ERR_UNSUPPORTED"),
])
def test_pd_validation(over, code):
    n = ctypes.c_size_t()
    rc = B.lib().ssm_workspace_bytes(B.SSM_OP_PD_FWD, ctypes.byref(pd_args(**over)), ctypes.byref(n))
    assert rc == status(code), B.lib().ssm_last_error_detail()


def test_pd_workspace_query():
    n = ctypes.c_size_t()
    assert B.lib().ssm_workspace_bytes(B.SSM_OP_PD_BWD, ctypes.byref(pd_args()), ctypes.byref(n)) == 0
    assert n.value > 0


def cplx_args(**over):
    a = B.ScanArgs(mode=B.SSM_COMPLEX_SHARED, dtype=B.SSM_F32, batch=2, channels=4, length=1000, state=64,
                   chunk_len=0, r=FAKE, phi=FAKE * 2, lam=FAKE * 3, theta=FAKE * 4, u=FAKE * 8, c=FAKE * 16)
    for k, v in over.items():
        setattr(a, k, v)
    return a


def test_complex_rtrl_host_checks():
    """Workspace query and argument checks of the forward-mode gradient entry point."""
    L = B.lib()
    rc, n = ws_bytes(B.SSM_OP_COMPLEX_RTRL, cplx_args())
    assert rc == 0 and n > 0, L.ssm_last_error_detail()
    # one segment workspace grows with B*H*M only, not with L
    _, n2 = ws_bytes(B.SSM_OP_COMPLEX_RTRL, cplx_args(length=100000))
    assert n2 < 64 * n
    rc, _ = ws_bytes(B.SSM_OP_COMPLEX_RTRL, sel_args())
    assert rc == status("SSM_ERR_UNSUPPORTED")
    a = cplx_args()
    gy, gl, gt = FAKE * 32, FAKE * 64, FAKE * 65
    rc = L.ssm_complex_rtrl(ctypes.byref(a), None, None, None, gl, gt, None, 0, None)
    assert rc == status("SSM_ERR_NULL")
    rc = L.ssm_complex_rtrl(ctypes.byref(a), gy, None, None, FAKE * 2 + 4, gt, None, 0, None)  # glam inside phi
    assert rc == status("SSM_ERR_LAYOUT"), L.ssm_last_error_detail()
    rc = L.ssm_complex_rtrl(ctypes.byref(a), gy, FAKE * 40 + 4, None, gl, gt, None, 0, None)  # gh_last misaligned
    assert rc == status("SSM_ERR_LAYOUT")
    rc = L.ssm_complex_rtrl(ctypes.byref(a), gy, None, None, gl, gt, None, 0, None)
    assert rc == status("SSM_ERR_WORKSPACE")


def cdense_args(**over):
    a = B.ScanArgs(mode=B.SSM_COMPLEX_DENSE, dtype=B.SSM_F32, batch=2, channels=4, length=1000, state=64,
                   chunk_len=0, a=FAKE * 8, u=FAKE * 16, c=FAKE * 32)
    for k, v in over.items():
        setattr(a, k, v)
    return a


def test_complex_dense_host_checks():
    """Given complex transitions: f32 only, a / u / c required, 8-byte alignment, up to 64 modes,
    no sensitivity or forward-mode entry points; an empty problem needs no tensors."""
    L = B.lib()
    for op in (B.SSM_OP_SCAN_FWD, B.SSM_OP_SCAN_BWD):
        rc, n = ws_bytes(op, cdense_args())
        assert rc == 0, L.ssm_last_error_detail()
    assert ws_bytes(B.SSM_OP_SCAN_FWD, cdense_args(dtype=B.SSM_BF16))[0] == status("SSM_ERR_DTYPE")
    assert ws_bytes(B.SSM_OP_SCAN_FWD, cdense_args(a=None))[0] == status("SSM_ERR_NULL")
    assert ws_bytes(B.SSM_OP_SCAN_FWD, cdense_args(u=None))[0] == status("SSM_ERR_NULL")
    assert ws_bytes(B.SSM_OP_SCAN_FWD, cdense_args(a=FAKE * 8 + 4))[0] == status("SSM_ERR_LAYOUT")
    assert ws_bytes(B.SSM_OP_SCAN_FWD, cdense_args(state=65))[0] == status("SSM_ERR_SHAPE")
    assert ws_bytes(B.SSM_OP_SCAN_FWD, cdense_args(chunk_len=64))[0] == status("SSM_ERR_UNSUPPORTED")
    for op in (B.SSM_OP_COMPLEX_RTRL, B.SSM_OP_IMPULSE, B.SSM_OP_SENS_ROWS):
        assert ws_bytes(op, cdense_args())[0] == status("SSM_ERR_UNSUPPORTED")
    assert ws_bytes(B.SSM_OP_SCAN_BWD, cdense_args(length=0, a=None, u=None, c=None)) == (0, 0)
    # the complex transitions are B*H*L*M complex64: a gradient placed inside them overlaps
    a = cdense_args()
    gi = B.ScanBwdIn(gy=FAKE * 64)
    gr = B.ScanGrads(ga=FAKE * 8 + 2 * 4 * 1000 * 64 * 8 - 64)
    rc = L.ssm_scan_bwd(ctypes.byref(a), ctypes.byref(gi), ctypes.byref(gr), None, 0, None)
    assert rc == status("SSM_ERR_LAYOUT"), L.ssm_last_error_detail()


def test_pd_ste_host_checks():
    """The surrogate selection gradient needs the scores and a positive finite temperature."""
    L = B.lib()
    a = pd_args()
    g = B.PDGrads(gd=FAKE * 64, glogits=FAKE * 128)
    for ste, tau, code in [(None, 1.0, "SSM_ERR_NULL"), (FAKE * 256, 0.0, "SSM_ERR_SHAPE"),
                           (FAKE * 256, -1.0, "SSM_ERR_SHAPE"), (FAKE * 256, float("inf"), "SSM_ERR_SHAPE"),
                           (FAKE * 256, float("nan"), "SSM_ERR_SHAPE"), (FAKE * 256, 1e-45, "SSM_ERR_SHAPE"),
                           (FAKE * 256 + 2, 1.0, "SSM_ERR_LAYOUT"), (FAKE * 128 + 64, 1.0, "SSM_ERR_LAYOUT"),
                           (FAKE * 256, 1.0, "SSM_ERR_WORKSPACE")]:
        i = B.PDBwdIn(gy=FAKE * 32, ste_logits=ste, tau=tau)
        rc = L.pd_scan_bwd(ctypes.byref(a), ctypes.byref(i), ctypes.byref(g), None, 0, None)
        assert rc == status(code), (ste, tau, L.ssm_last_error_detail())
    # the scores are not read (and tau not checked) when glogits is not wanted
    i = B.PDBwdIn(gy=FAKE * 32, ste_logits=None, tau=0.0)
    rc = L.pd_scan_bwd(ctypes.byref(a), ctypes.byref(i), ctypes.byref(B.PDGrads(gd=FAKE * 64)), None, 0, None)
    assert rc == status("SSM_ERR_WORKSPACE")


def test_output_sensitivity_host_checks():
    """s_delta is required.  With 16 states and the sequence cut into segments the forward's main pass forms
    the sensitivities and the workspace is the impulse path's; otherwise (here 5 states) it also holds the
    per-tile checkpoints a separate pass re-runs (growing with L)."""
    L = B.lib()
    rc, n1 = ws_bytes(B.SSM_OP_OUTPUT_SENS, sel_args(length=4096))
    assert rc == 0
    _, m1 = ws_bytes(B.SSM_OP_IMPULSE, sel_args(length=4096))
    assert n1 == m1
    _, k1 = ws_bytes(B.SSM_OP_OUTPUT_SENS, sel_args(length=4096, state=5))
    _, k2 = ws_bytes(B.SSM_OP_OUTPUT_SENS, sel_args(length=8192, state=5))
    _, j1 = ws_bytes(B.SSM_OP_IMPULSE, sel_args(length=4096, state=5))
    assert k2 - k1 >= 2 * 32 * 16 * 5 * 4 and k1 > j1   # 16 more tiles x 5 states per channel
    a = sel_args()
    rc = L.ssm_output_sensitivity(ctypes.byref(a), -1, None, FAKE * 64, None, None, 0, None)
    assert rc == status("SSM_ERR_NULL")
    rc = L.ssm_output_sensitivity(ctypes.byref(a), -1, None, None, FAKE * 2 + 8, None, 0, None)   # inside x
    assert rc == status("SSM_ERR_LAYOUT")
    rc = L.ssm_output_sensitivity(ctypes.byref(a), 5000, None, None, FAKE * 64, None, 0, None)
    assert rc == status("SSM_ERR_SHAPE")
    rc = L.ssm_output_sensitivity(ctypes.byref(a), -1, None, None, FAKE * 64, None, 0, None)
    assert rc == status("SSM_ERR_WORKSPACE")
    rc, _ = ws_bytes(B.SSM_OP_OUTPUT_SENS, cplx_args())
    assert rc == status("SSM_ERR_UNSUPPORTED")


def test_sensitivity_rows_host_checks():
    """Rows 1..16 inside [0, L), s required and disjoint from the inputs, 64-step tiles, selective mode only."""
    L = B.lib()
    rc, n1 = ws_bytes(B.SSM_OP_SENS_ROWS, sel_args(length=4096))
    assert rc == 0, L.ssm_last_error_detail()
    _, n2 = ws_bytes(B.SSM_OP_SENS_ROWS, sel_args(length=8192))
    assert n2 - n1 >= 2 * 32 * 64 * 12   # one float and one double per 64-step tile and channel
    for over in ({"chunk_len": 128}, {"chunk_len": 256}):
        rc, _ = ws_bytes(B.SSM_OP_SENS_ROWS, sel_args(**over))
        assert rc == status("SSM_ERR_UNSUPPORTED")
    rc, _ = ws_bytes(B.SSM_OP_SENS_ROWS, cplx_args())
    assert rc == status("SSM_ERR_UNSUPPORTED")
    a = sel_args()
    for t0, rows in ((0, 0), (0, 17), (-1, 4), (997, 4), (999, 2)):
        rc = L.ssm_sensitivity_rows(ctypes.byref(a), t0, rows, FAKE * 64, None, 0, None)
        assert rc == status("SSM_ERR_SHAPE"), (t0, rows)
    rc = L.ssm_sensitivity_rows(ctypes.byref(a), 10, 4, None, None, 0, None)
    assert rc == status("SSM_ERR_NULL")
    rc = L.ssm_sensitivity_rows(ctypes.byref(a), 10, 4, FAKE + 8, None, 0, None)   # inside delta
    assert rc == status("SSM_ERR_LAYOUT")
    for t0, rows in ((0, 1), (996, 4), (984, 16)):
        rc = L.ssm_sensitivity_rows(ctypes.byref(a), t0, rows, FAKE * 64, None, 0, None)
        assert rc == status("SSM_ERR_WORKSPACE"), (t0, rows)


def test_step_size_transform_selective_only():
    rc, _ = ws_bytes(B.SSM_OP_SCAN_FWD, cplx_args(delta_softplus=1))
    assert rc == status("SSM_ERR_UNSUPPORTED")
    rc, _ = ws_bytes(B.SSM_OP_SCAN_FWD, sel_args(mode=B.SSM_REAL_DENSE, a=FAKE * 6, b=FAKE * 7, delta_bias=FAKE * 8))
    assert rc == status("SSM_ERR_UNSUPPORTED")
    rc, n = ws_bytes(B.SSM_OP_SCAN_BWD, sel_args(delta_bias=FAKE * 8, delta_softplus=1))
    assert rc == 0 and n > 0


def test_pd_dtype_checks():
    L = B.lib()
    rc, _ = ws_bytes_pd(pd_args(dtype=5))
    assert rc == status("SSM_ERR_DTYPE")
    rc, _ = ws_bytes_pd(pd_args(dtype=B.SSM_BF16, d=FAKE * 3 + 2))   # 2-byte aligned is fine for bf16
    assert rc == 0, L.ssm_last_error_detail()
    rc, _ = ws_bytes_pd(pd_args(d=FAKE * 3 + 2))                      # but not for fp32
    assert rc == status("SSM_ERR_LAYOUT")
    a = pd_args(dtype=B.SSM_BF16, dict_size=32)
    i = B.PDBwdIn(gy=FAKE * 32, ste_logits=FAKE * 256, tau=1.0)
    g = B.PDGrads(gd=FAKE * 64, glogits=FAKE * 128)
    rc = L.pd_scan_bwd(ctypes.byref(a), ctypes.byref(i), ctypes.byref(g), None, 0, None)
    assert rc == status("SSM_ERR_UNSUPPORTED")   # bf16 glogits needs K <= 16


def ws_bytes_pd(args):
    n = ctypes.c_size_t(0)
    rc = B.lib().ssm_workspace_bytes(B.SSM_OP_PD_FWD, ctypes.byref(args), ctypes.byref(n))
    return rc, n.value


# ---------------------------------------------------------------------------
# binding: caller-supplied outputs are checked like inputs; host tensors are refused
# ---------------------------------------------------------------------------
def _cpu_sel(L=40, D=3, N=4, dtype=None):
    import torch
    dt = dtype or torch.float32
    g = torch.Generator().manual_seed(0)
    return dict(delta=torch.rand(2, D, L, generator=g).to(dt), x=torch.randn(2, D, L, generator=g).to(dt),
                A=-torch.rand(D, N, generator=g), Bm=torch.randn(2, L, N, generator=g).to(dt),
                C=torch.randn(2, L, N, generator=g).to(dt))


@pytest.mark.parametrize("key,make,exc", [
    ("y", lambda t: t.zeros(2, 3, 41), ValueError),                      # wrong shape
    ("y", lambda t: t.zeros(2, 3, 40, dtype=t.bfloat16), TypeError),     # wrong dtype
    ("y", lambda t: t.zeros(2, 40, 3).transpose(1, 2), ValueError),      # not contiguous
    ("h_last", lambda t: t.zeros(2, 3, 5), ValueError),
    ("ckpt", lambda t: t.zeros(2, 3, 1, 4, dtype=t.float64), TypeError),
])
def test_scan_fwd_rejects_bad_out(key, make, exc):
    import torch
    with pytest.raises(exc):
        B.scan_fwd(B.SSM_REAL_SELECTIVE, want_h_last=True, want_ckpt=True, out={key: make(torch)}, **_cpu_sel())


@pytest.mark.parametrize("key,make,exc", [
    ("gdelta", lambda t: t.zeros(2, 3, 39), ValueError),
    ("gBm", lambda t: t.zeros(2, 40, 4, dtype=t.bfloat16), TypeError),
    ("gA", lambda t: t.zeros(4, 3).t(), ValueError),
    ("gphi", lambda t: t.zeros(2, 3, 40), ValueError),                   # no such gradient in this mode
])
def test_scan_bwd_rejects_bad_out(key, make, exc):
    import torch
    t = _cpu_sel()
    with pytest.raises(exc):
        B.scan_bwd(B.SSM_REAL_SELECTIVE, gy=torch.zeros(2, 3, 40), out={key: make(torch)}, **t)


def test_other_entry_points_reject_bad_out():
    import torch
    t = _cpu_sel()
    with pytest.raises(ValueError):
        B.impulse_sensitivity(out={"s": torch.zeros(2, 3, 7)}, **t)
    with pytest.raises(TypeError):
        B.output_sensitivity(out={"s_delta": torch.zeros(2, 3, 40, dtype=torch.float64)}, **t)
    with pytest.raises(ValueError):
        B.sensitivity_rows(t_out0=0, rows=2, out=torch.zeros(3, 2, 3, 40), **t)
    g = torch.Generator().manual_seed(1)
    pd = dict(logits=torch.randn(2, 2, 30, 4, generator=g), dict=torch.randint(0, 5, (2, 4, 5), dtype=torch.int32),
              d=torch.rand(2, 2, 30, 5, generator=g), b=torch.randn(2, 2, 30, 5, generator=g),
              C=torch.randn(2, 2, 30, 5, generator=g))
    with pytest.raises(TypeError):
        B.pd_scan_fwd(out={"sel": torch.zeros(2, 2, 30, dtype=torch.int64)}, **pd)
    with pytest.raises(ValueError):
        B.pd_scan_bwd(gy=torch.zeros(2, 2, 30), out={"gd": torch.zeros(2, 2, 30, 4)}, **pd)


def test_host_tensors_are_refused():
    """Valid arguments on the host never reach the library: it takes device pointers only."""
    import torch
    t = _cpu_sel()
    with pytest.raises(ValueError, match="GPU"):
        B.scan_fwd(B.SSM_REAL_SELECTIVE, **t)
    with pytest.raises(ValueError, match="GPU"):
        B.scan_bwd(B.SSM_REAL_SELECTIVE, gy=torch.zeros(2, 3, 40), **t)
    with pytest.raises(ValueError, match="GPU"):
        B.impulse_sensitivity(**t)


def test_allocator_hook_shapes_are_checked():
    import torch
    B.set_allocator(lambda shape, dtype, device, role: torch.zeros(1))
    try:
        with pytest.raises(ValueError, match="allocator"):
            B.scan_fwd(B.SSM_REAL_SELECTIVE, **_cpu_sel())
    finally:
        B.set_allocator(None)


def test_every_forward_fits_the_static_scratch():
    """ssm_scan_fwd_noalloc's static scratch holds the workspace of every forward: the largest needs come
    from the segment summaries when few sequences leave room for many segments."""
    cap = 32 * 1024 * 1024
    worst = 0
    for mode, N in ((B.SSM_REAL_SELECTIVE, 16), (B.SSM_REAL_DENSE, 16), (B.SSM_COMPLEX_SHARED, 64),
                    (B.SSM_COMPLEX_DENSE, 64)):
        for bd in (1, 2, 3, 7, 16, 100, 255, 1000, 2049, 4095, 4097, 16383, 16385, 65536):
            a = sel_args(mode=mode, batch=1, channels=bd, length=1 << 20, state=N, dtype=B.SSM_F32,
                         a=FAKE * 7, b=FAKE * 8, u=FAKE * 9, c=FAKE * 10, r=FAKE * 11, phi=FAKE * 12,
                         lam=FAKE * 13, theta=FAKE * 14)
            rc, n = ws_bytes(B.SSM_OP_SCAN_FWD, a)
            assert rc == 0, (mode, bd)
            worst = max(worst, n)
    assert 0 < worst <= cap


def test_head_mode_noalloc_refuses_chunk_states_beyond_the_scratch():
    """The per-head forward keeps 4 B D N ceil(L/64) + 4 B H ceil(L/64) bytes of chunk states; the
    allocation-free forward takes them up to the static array's size and refuses more before any device
    call (SSM_ERR_WORKSPACE)."""
    cap = 32 * 1024 * 1024

    def head(B_, H, P, L):
        return sel_args(mode=B.SSM_HEAD_SCALAR, dtype=B.SSM_BF16, batch=B_, channels=H * P, length=L, state=16,
                        head_dim=P)
    for B_, H, P, L in ((8, 32, 64, 4096), (1, 2, 16, 65), (2, 4, 64, 1000)):
        rc, n = ws_bytes(B.SSM_OP_SCAN_FWD, head(B_, H, P, L))
        assert rc == 0, B.lib().ssm_last_error_detail()
        nch = -(-L // 64)
        assert n >= 4 * B_ * H * P * 16 * nch + 4 * B_ * H * nch
    big = head(8, 32, 64, 4096)   # 67 MB of chunk states
    o = B.ScanFwdOut(y=FAKE * 9, h_last=None, ckpt=None)
    rc = B.lib().ssm_scan_fwd_noalloc(ctypes.byref(big), ctypes.byref(o), None)
    assert rc == status("SSM_ERR_WORKSPACE")
    assert ws_bytes(B.SSM_OP_SCAN_FWD, head(2, 4, 64, 1000))[1] <= cap


# ---------------------------------------------------------------------------
# strided views (ssm_layout) and the discretisation selector: host-side checks
# ---------------------------------------------------------------------------
def _lay(**roles):
    lay = B.Layout()
    for role, st in roles.items():
        r = getattr(B, "V_" + role.upper())
        lay.given |= 1 << r
        for i, v in enumerate(st):
            lay.stride[r][i] = v
    return lay


def _fwd_rc(a, out_y=FAKE * 9):
    o = B.ScanFwdOut(y=out_y, h_last=None, ckpt=None)
    return B.lib().ssm_scan_fwd(ctypes.byref(a), ctypes.byref(o), None, 0, None)


@pytest.mark.parametrize("roles,code", [
    (dict(x=(32000, 1000, 2)), "SSM_ERR_LAYOUT"),            # innermost stride must be 1
    (dict(delta=(-1000, 1000, 1)), "SSM_ERR_LAYOUT"),        # negative stride
    (dict(y=(32000, 0, 1)), "SSM_ERR_LAYOUT"),               # output with stride 0 (channels alias)
    (dict(y=(1000, 1000, 1)), "SSM_ERR_LAYOUT"),             # output rows that overlap
    (dict(gy=(32000, 1000, 1)), "SSM_ERR_UNSUPPORTED"),      # gy is no forward argument
    (dict(r=(32000, 1000, 1)), "SSM_ERR_UNSUPPORTED"),       # a complex role in the selective mode
    (dict(dict=(0, 16, 1)), "SSM_ERR_UNSUPPORTED"),          # a PD role in a diagonal scan
])
def test_layout_errors(roles, code):
    a = sel_args()
    lay = _lay(**roles)
    a.layout = ctypes.pointer(lay)
    assert _fwd_rc(a) == status(code), B.lib().ssm_last_error_detail()


def test_layout_accepts_views():
    """Broadcast inputs (stride 0), slices and per-channel B_t, C_t pass validation (sizes only)."""
    for roles in (dict(delta=(0, 1000, 1), x=(64000, 2000, 1), a=(0, 1)),
                  dict(bm=(0, 0, 16, 1), c=(0, 0, 16, 1)),
                  dict(bm=(32 * 16000, 16000, 16, 1), c=(32 * 16000, 16000, 16, 1)),
                  dict(bm=(16000, 16, 16, 1)),   # per-channel Bm next to a shared C
                  dict(y=(64000, 2000, 1))):
        a = sel_args()
        lay = _lay(**roles)
        a.layout = ctypes.pointer(lay)
        rc, n = ws_bytes(B.SSM_OP_SCAN_FWD, a)
        assert rc == 0, (roles, B.lib().ssm_last_error_detail())


def test_perd_and_zoh_limits():
    """Per-channel B_t, C_t and the ZOH term are scan-only; ZOH is the selective mode's; unknown selector."""
    perd = _lay(bm=(32 * 16000, 16000, 16, 1), c=(32 * 16000, 16000, 16, 1))
    a = sel_args()
    a.layout = ctypes.pointer(perd)
    rc, _ = ws_bytes(B.SSM_OP_IMPULSE, a)
    assert rc == status("SSM_ERR_UNSUPPORTED")
    rc, _ = ws_bytes(B.SSM_OP_SCAN_BWD, a)
    assert rc == 0
    a = sel_args(discretization=B.SSM_ZOH)
    assert ws_bytes(B.SSM_OP_SCAN_FWD, a)[0] == 0
    assert ws_bytes(B.SSM_OP_SCAN_BWD, a)[0] == 0
    assert ws_bytes(B.SSM_OP_IMPULSE, a)[0] == status("SSM_ERR_UNSUPPORTED")
    assert ws_bytes(B.SSM_OP_SENS_ROWS, a)[0] == status("SSM_ERR_UNSUPPORTED")
    a.layout = ctypes.pointer(perd)
    assert ws_bytes(B.SSM_OP_SCAN_FWD, a)[0] == status("SSM_ERR_UNSUPPORTED")
    a = sel_args(discretization=7)
    assert ws_bytes(B.SSM_OP_SCAN_FWD, a)[0] == status("SSM_ERR_SHAPE")
    c = sel_args(mode=B.SSM_COMPLEX_SHARED, state=8, u=FAKE * 9, c=FAKE * 10, r=FAKE * 11, phi=FAKE * 12,
                 lam=FAKE * 13, theta=FAKE * 14, discretization=B.SSM_ZOH)
    assert ws_bytes(B.SSM_OP_SCAN_FWD, c)[0] == status("SSM_ERR_UNSUPPORTED")


def test_pd_layout_checks():
    shared = _lay(dict=(0, 16, 1), pd_d=(2 * 4 * 500 * 16, 500 * 16, 16, 1))
    a = pd_args()
    a.layout = ctypes.pointer(shared)
    assert ws_bytes_pd(a)[0] == 0
    bad = _lay(dict=(128, 16, 2))
    a.layout = ctypes.pointer(bad)
    assert ws_bytes_pd(a)[0] == status("SSM_ERR_LAYOUT")
    bad = _lay(x=(1, 1, 1))
    a.layout = ctypes.pointer(bad)
    assert ws_bytes_pd(a)[0] == status("SSM_ERR_UNSUPPORTED")


def test_binding_passes_views():
    """The binding takes strided views of its inputs (no copies) and describes them to the library."""
    import torch
    t = _cpu_sel(L=40, D=3, N=4)
    big = torch.randn(2, 6, 40)
    t["x"] = big[:, ::2]                                  # channel stride 80
    t["A"] = (-torch.rand(1, 4)).expand(3, 4)             # one A row for every channel
    args, _, _ = B._scan_args(B.SSM_REAL_SELECTIVE, **t)
    lay = args.layout.contents
    assert lay.given == (1 << B.V_X) | (1 << B.V_A)
    assert list(lay.stride[B.V_X])[:3] == [240, 80, 1]
    assert list(lay.stride[B.V_A])[:2] == [0, 1]
    t = _cpu_sel(L=40, D=3, N=4)
    args, _, _ = B._scan_args(B.SSM_REAL_SELECTIVE, **t)
    assert not args.layout                                 # dense: no layout at all
    t["Bm"] = torch.randn(2, 3, 40, 4)
    t["C"] = torch.randn(2, 40, 4).unsqueeze(1).expand(2, 3, 40, 4)
    args, _, _ = B._scan_args(B.SSM_REAL_SELECTIVE, **t)
    lay = args.layout.contents
    # per-channel Bm is a view; C expanded over the channels is the default shared layout
    assert args._perd and (lay.given >> B.V_BM) & 1 and not (lay.given >> B.V_C) & 1
    assert list(lay.stride[B.V_BM]) == [480, 160, 4, 1]


def test_roof_probe_argument_checks():
    """The issue-rate probe refuses unknown kinds, chain counts a kind does not run, and NULL outputs before it
    touches the device."""
    L = B.lib()
    L.ssm_roof_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                 ctypes.POINTER(ctypes.c_double), ctypes.c_void_p]
    r = ctypes.c_double(0.0)
    sink = ctypes.c_void_p(FAKE)
    assert L.ssm_roof_probe(8, 8, 4, 10, sink, ctypes.byref(r), None) == status("SSM_ERR_UNSUPPORTED")
    assert L.ssm_roof_probe(-1, 8, 4, 10, sink, ctypes.byref(r), None) == status("SSM_ERR_UNSUPPORTED")
    assert L.ssm_roof_probe(3, 8, 4, 10, sink, ctypes.byref(r), None) == status("SSM_ERR_UNSUPPORTED")
    assert L.ssm_roof_probe(7, 4, 4, 10, sink, ctypes.byref(r), None) == status("SSM_ERR_UNSUPPORTED")
    assert L.ssm_roof_probe(7, 8, 0, 10, sink, ctypes.byref(r), None) == status("SSM_ERR_SHAPE")
    assert L.ssm_roof_probe(7, 8, 4, 10, None, ctypes.byref(r), None) == status("SSM_ERR_NULL")
