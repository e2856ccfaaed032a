"""GPU parity of the dense real, complex shared-control and PD scans against
the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests._compare import BF16, F32, assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def T(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _ssm():
    import selective_state_space_chunked_amd as ssm
    return ssm


# ---------------------------------------------------------------------------
# dense real
# ---------------------------------------------------------------------------
def run_dense(B, D, L, N, seed, h0=False, ghl=False):
    ssm = _ssm()
    g = np.random.default_rng(seed)
    a = g.uniform(0.5, 1.0, (B, D, L, N)).astype(np.float32)
    b = (g.standard_normal((B, D, L, N)) / 4).astype(np.float32)
    C = (g.standard_normal((B, L, N)) / 4).astype(np.float32)
    gy = g.standard_normal((B, D, L)).astype(np.float32)
    hh = g.standard_normal((B, D, N)).astype(np.float32) if h0 else None
    gl = g.standard_normal((B, D, N)).astype(np.float32) if ghl else None
    t = dict(a=T(a), b=T(b), C=T(C), h0=None if hh is None else T(hh))
    f = ssm.scan_fwd(ssm.SSM_REAL_DENSE, want_h_last=True, want_ckpt=True, **t)
    gr = ssm.scan_bwd(ssm.SSM_REAL_DENSE, gy=T(gy), ckpt=f["ckpt"], gh_last=None if gl is None else T(gl), **t)
    gr2 = ssm.scan_bwd(ssm.SSM_REAL_DENSE, gy=T(gy), gh_last=None if gl is None else T(gl), **t)
    torch.cuda.synchronize()
    y, hl = oracle.real_fwd(a=a, b=b, C=C, h0=hh, B=B, D=D, L=L, N=N)
    og = oracle.real_bwd(a=a, b=b, C=C, h0=hh, gy=gy, ghlast=gl, B=B, D=D, L=L, N=N)
    assert_close("y", f["y"], y, **F32)
    assert_close("h_last", f["h_last"], hl, **F32)
    for k in ("ga", "gb", "gC", "gh0"):
        assert_close(k, gr[k], og[k], **F32)
        assert torch.equal(gr[k], gr2[k]), k


@pytest.mark.parametrize("L", [1, 31, 32, 33, 500])
def test_dense_lengths(L):
    run_dense(2, 20, L, 16, seed=L, h0=True, ghl=True)


def test_dense_small_state():
    run_dense(1, 5, 200, 3, seed=3)


def test_dense_checkpoints_are_chunk_states():
    """ckpt[:, :, c] of the dense real scan is the state entering 32-step chunk c (c = 0 holds h0)."""
    ssm = _ssm()
    B, D, L, N = 2, 20, 1000, 16
    g = np.random.default_rng(45)
    a = g.uniform(0.5, 1.0, (B, D, L, N)).astype(np.float32)
    b = (g.standard_normal((B, D, L, N)) / 4).astype(np.float32)
    C = (g.standard_normal((B, L, N)) / 4).astype(np.float32)
    h0 = g.standard_normal((B, D, N)).astype(np.float32)
    f = ssm.scan_fwd(ssm.SSM_REAL_DENSE, want_y=False, want_ckpt=True, a=T(a), b=T(b), C=T(C), h0=T(h0))
    torch.cuda.synchronize()
    ck = f["ckpt"]
    nc = -(-L // 32)
    assert ck.shape == (B, D, nc, N)
    assert torch.equal(ck[:, :, 0].cpu(), torch.from_numpy(h0))
    for c in (1, 2, 8, 17, nc - 1):
        Lc = 32 * c
        _, hl = oracle.real_fwd(a=a[:, :, :Lc], b=b[:, :, :Lc], C=C[:, :Lc], h0=h0, B=B, D=D, L=Lc, N=N)
        assert_close(f"ckpt[{c}]", ck[:, :, c], hl, **F32)


def test_dense_many_segments():
    run_dense(1, 16, 3000, 16, seed=4, h0=True)


# ---------------------------------------------------------------------------
# complex
# ---------------------------------------------------------------------------
def S(a):
    """A stream to the device: bf16 bit arrays (uint16) as bfloat16, else as is."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).astype(np.int16)).view(torch.bfloat16).to(DEV)
    return T(a)


def _cplx_oracle_kw(cfg):
    kw = {k: cfg[k] for k in ("r", "phi", "lam", "theta", "u", "c")}
    if cfg.get("dtype") == "bf16":
        kw["u"] = cfg["u_c"]
    return kw


def run_complex(cfg, h0=None, ghl=None):
    ssm = _ssm()
    B, H, L, M = cfg["B"], cfg["H"], cfg["L"], cfg["M"]
    t = {k: S(cfg[k]) for k in ("r", "phi", "lam", "theta", "u", "c")}
    if h0 is not None:
        t["h0"] = T(h0.astype(np.complex64))
    gyt = S(cfg["gy"])
    glt = None if ghl is None else T(ghl.astype(np.complex64))
    f = ssm.scan_fwd(ssm.SSM_COMPLEX_SHARED, want_h_last=True, want_ckpt=True, **t)
    g = ssm.scan_bwd(ssm.SSM_COMPLEX_SHARED, gy=gyt, ckpt=f["ckpt"], gh_last=glt, **t)
    g2 = ssm.scan_bwd(ssm.SSM_COMPLEX_SHARED, gy=gyt, gh_last=glt, **t)
    torch.cuda.synchronize()
    kw = _cplx_oracle_kw(cfg)
    h0c = None if h0 is None else h0.astype(np.complex64)
    y, hl = oracle.complex_fwd(**kw, h0=h0c, B=B, H=H, L=L, M=M)
    og = oracle.complex_bwd(**kw, h0=h0c, gy=cfg["gy"], ghlast=None if ghl is None else ghl.astype(np.complex64),
                            B=B, H=H, L=L, M=M)
    bf = cfg.get("dtype") == "bf16"
    tol = BF16 if bf else F32
    errs = {"y": assert_close("y", f["y"], y, **tol), "h_last": assert_close("h_last", f["h_last"], hl, **F32)}
    for k in ("gu", "gr", "gphi", "glam", "gtheta", "gc", "gh0"):
        gk = g[k]
        if k == "gu" and bf:   # (re, im) bf16 pairs -> complex
            gk = torch.complex(gk[..., 0].float(), gk[..., 1].float())
        errs[k] = assert_close(k, gk, og[k], **(tol if k in ("gu", "gr", "gphi") else F32))
        assert torch.equal(g[k], g2[k]), k
    return errs


def test_complex_small():
    cfg = synth.make_complex(B=2, H=3, M=64, L=300, seed=1)
    g = np.random.default_rng(5)
    run_complex(cfg, h0=g.standard_normal((2, 3, 64)) + 1j * g.standard_normal((2, 3, 64)),
                ghl=g.standard_normal((2, 3, 64)) + 1j * g.standard_normal((2, 3, 64)))


@pytest.mark.parametrize("M,L", [(5, 100), (64, 1), (64, 33), (32, 64)])
def test_complex_shapes(M, L):
    run_complex(synth.make_complex(B=1, H=2, M=M, L=L, seed=M + L))


def test_complex_large_phase_arguments():
    """Chunks whose phase arguments phi_t * theta_m exceed 1e6 take the library sincos; the others the series path."""
    cfg = synth.make_complex(B=1, H=2, M=64, L=200, seed=21)
    cfg["phi"] = cfg["phi"].copy()
    cfg["phi"][:, :, 40:52] *= np.float32(3.0e7)   # a full chunk and part of the next
    cfg["phi"][:, :, 195:] *= np.float32(3.0e7)    # the partial last chunk
    run_complex(cfg)


@pytest.mark.parametrize("case", ["no_rotation_unit_decay", "rotation_only", "retention_huge", "u_zero"])
def test_complex_degenerate_inputs(case):
    """Degenerate controls: lambda = 1 and theta = 0 (a = 1, pure accumulation), r = 0 (|a| = 1, phase rotation
    only), r = 1e3 (|a| underflows), u = 0 (no input); nonzero h0 and gh_last carry state and adjoint."""
    cfg = synth.make_complex(B=2, H=3, M=64, L=200, seed=31)
    g = np.random.default_rng(32)
    h0 = g.standard_normal((2, 3, 64)) + 1j * g.standard_normal((2, 3, 64))
    ghl = g.standard_normal((2, 3, 64)) + 1j * g.standard_normal((2, 3, 64))
    if case == "no_rotation_unit_decay":
        cfg["lam"] = np.ones_like(cfg["lam"])
        cfg["theta"] = np.zeros_like(cfg["theta"])
    elif case == "rotation_only":
        cfg["r"] = np.zeros_like(cfg["r"])
    elif case == "retention_huge":
        cfg["r"] = np.full_like(cfg["r"], 1e3)
    else:
        cfg["u"] = np.zeros_like(cfg["u"])
    run_complex(cfg, h0=h0, ghl=ghl)


def test_complex_bf16_streams():
    """bf16 r, phi, u (pairs), gy and stream gradients; fp64 recurrence, fp32 parameter gradients."""
    g = np.random.default_rng(43)
    run_complex(synth.make_complex(B=2, H=3, M=64, L=300, seed=42, dtype="bf16"),
                h0=g.standard_normal((2, 3, 64)) + 1j * g.standard_normal((2, 3, 64)))


def test_complex_rtrl_bf16():
    run_complex_rtrl(synth.make_complex(B=2, H=2, M=64, L=500, seed=44, dtype="bf16"))


def test_complex_full_config():
    """B=16 H=8 M=64 L=2048 complex64, seed 0: every output compared element-wise."""
    run_complex(synth.make_complex(B=16, H=8, M=64, L=2048, seed=0))


# ---------------------------------------------------------------------------
# complex with given transitions
# ---------------------------------------------------------------------------
def run_complex_dense(cfg, h0=None, ghl=None):
    ssm = _ssm()
    B, H, L, M = cfg["B"], cfg["H"], cfg["L"], cfg["M"]
    t = dict(a=T(cfg["a"]), u=T(cfg["u"]), c=T(cfg["c"]))
    h0c = None if h0 is None else h0.astype(np.complex64)
    ghc = None if ghl is None else ghl.astype(np.complex64)
    if h0c is not None:
        t["h0"] = T(h0c)
    gyt = T(cfg["gy"])
    glt = None if ghc is None else T(ghc)
    f = ssm.scan_fwd(ssm.SSM_COMPLEX_DENSE, want_h_last=True, want_ckpt=True, **t)
    g = ssm.scan_bwd(ssm.SSM_COMPLEX_DENSE, gy=gyt, ckpt=f["ckpt"], gh_last=glt, **t)
    g2 = ssm.scan_bwd(ssm.SSM_COMPLEX_DENSE, gy=gyt, gh_last=glt, **t)
    torch.cuda.synchronize()
    kw = dict(a=cfg["a"], u=cfg["u"], c=cfg["c"], h0=h0c, B=B, H=H, L=L, M=M)
    y, hl = oracle.complex_dense_fwd(**kw)
    og = oracle.complex_dense_bwd(**kw, gy=cfg["gy"], ghlast=ghc)
    errs = {"y": assert_close("y", f["y"], y, **F32), "h_last": assert_close("h_last", f["h_last"], hl, **F32)}
    for k in ("ga", "gu", "gc", "gh0"):
        errs[k] = assert_close(k, g[k], og[k], **F32)
        assert torch.equal(g[k], g2[k]), k
    return errs


def _cplx_state(seed, B, H, M):
    g = np.random.default_rng(seed)
    return g.standard_normal((B, H, M)) + 1j * g.standard_normal((B, H, M))


def test_complex_dense_small():
    cfg = synth.make_complex_dense(B=2, H=3, M=64, L=300, seed=1)
    run_complex_dense(cfg, h0=_cplx_state(2, 2, 3, 64), ghl=_cplx_state(3, 2, 3, 64))


@pytest.mark.parametrize("M,L", [(5, 100), (64, 1), (64, 33), (32, 64), (17, 700)])
def test_complex_dense_shapes(M, L):
    run_complex_dense(synth.make_complex_dense(B=1, H=2, M=M, L=L, seed=M + L))


def test_complex_dense_long_sequence():
    """One sequence split into many segments (summary, combine and main passes)."""
    run_complex_dense(synth.make_complex_dense(B=1, H=1, M=64, L=20000, seed=7), h0=_cplx_state(8, 1, 1, 64),
                      ghl=_cplx_state(9, 1, 1, 64))


@pytest.mark.parametrize("case", ["a_one", "a_zero", "rotation_only", "u_zero"])
def test_complex_dense_degenerate_inputs(case):
    """a = 1 (pure accumulation), a = 0 (the state restarts every step), |a| = 1 (rotation only), u = 0; nonzero
    h0 and gh_last carry state and adjoint."""
    cfg = synth.make_complex_dense(B=2, H=3, M=64, L=200, seed=33)
    a = cfg["a"]
    if case == "a_one":
        cfg["a"] = np.ones_like(a)
    elif case == "a_zero":
        cfg["a"] = np.zeros_like(a)
    elif case == "rotation_only":
        cfg["a"] = (a / np.abs(a)).astype(np.complex64)
    else:
        cfg["u"] = np.zeros_like(cfg["u"])
    run_complex_dense(cfg, h0=_cplx_state(34, 2, 3, 64), ghl=_cplx_state(35, 2, 3, 64))


def test_complex_dense_shared_control_transitions():
    """Transitions of the shared-control form a = lam^r e^{i phi theta}, formed in numpy and rounded to complex64:
    slow modes (|a| up to 0.9993) with long horizons through the given-transition kernels."""
    cfg = synth.make_complex(B=2, H=3, M=64, L=1500, seed=36)
    a = (cfg["lam"].astype(np.float64)[None, :, None, :] ** cfg["r"].astype(np.float64)[:, :, :, None]) * \
        np.exp(1j * cfg["phi"].astype(np.float64)[:, :, :, None] * cfg["theta"].astype(np.float64)[None, :, None, :])
    dense = dict(B=2, H=3, M=64, L=1500, a=a.astype(np.complex64), u=cfg["u"], c=cfg["c"], gy=cfg["gy"])
    run_complex_dense(dense, h0=_cplx_state(37, 2, 3, 64), ghl=_cplx_state(38, 2, 3, 64))


def test_complex_checkpoints_are_chunk_states():
    """ckpt[:, :, c] of both complex modes is the state entering 32-step chunk c: the oracle's final state of the
    first 32c steps (c = 0 holds h0); the sequence is long enough to be split into segments."""
    ssm = _ssm()
    B, H, M, L = 1, 2, 64, 700
    h0 = _cplx_state(40, B, H, M).astype(np.complex64)
    sh = synth.make_complex(B=B, H=H, M=M, L=L, seed=41)
    dn = synth.make_complex_dense(B=B, H=H, M=M, L=L, seed=42)
    fs = ssm.scan_fwd(ssm.SSM_COMPLEX_SHARED, want_y=False, want_ckpt=True, h0=T(h0),
                      **{k: T(sh[k]) for k in ("r", "phi", "lam", "theta", "u", "c")})
    fd = ssm.scan_fwd(ssm.SSM_COMPLEX_DENSE, want_y=False, want_ckpt=True, h0=T(h0),
                      **{k: T(dn[k]) for k in ("a", "u", "c")})
    torch.cuda.synchronize()
    nc = -(-L // 32)
    for ck in (fs["ckpt"], fd["ckpt"]):
        assert ck.shape == (B, H, nc, M)
        assert torch.equal(ck[:, :, 0].cpu(), torch.from_numpy(h0))
    for c in (1, 2, 7, 8, 9, nc - 1):
        Lc = 32 * c
        _, hs = oracle.complex_fwd(r=sh["r"][:, :, :Lc], phi=sh["phi"][:, :, :Lc], lam=sh["lam"], theta=sh["theta"],
                                   u=sh["u"][:, :, :Lc], c=sh["c"], h0=h0, B=B, H=H, L=Lc, M=M)
        _, hd = oracle.complex_dense_fwd(a=dn["a"][:, :, :Lc], u=dn["u"][:, :, :Lc], c=dn["c"], h0=h0,
                                         B=B, H=H, L=Lc, M=M)
        assert_close(f"shared ckpt[{c}]", fs["ckpt"][:, :, c], hs, **F32)
        assert_close(f"dense ckpt[{c}]", fd["ckpt"][:, :, c], hd, **F32)


def test_complex_dense_full_config():
    """B=16 H=8 M=64 L=2048 complex64, seed 0: every output compared element-wise."""
    run_complex_dense(synth.make_complex_dense(B=16, H=8, M=64, L=2048, seed=0))


# ---------------------------------------------------------------------------
# complex: forward-mode (RTRL) gradients of lambda and theta
# ---------------------------------------------------------------------------
def run_complex_rtrl(cfg, h0=None, ghl=None):
    """GPU forward-mode glam, gtheta against the oracle's forward-mode recursion,
    and against the GPU reverse-mode (BPTT) gradients of the same loss."""
    ssm = _ssm()
    B, H, L, M = cfg["B"], cfg["H"], cfg["L"], cfg["M"]
    t = {k: S(cfg[k]) for k in ("r", "phi", "lam", "theta", "u", "c")}
    if h0 is not None:
        t["h0"] = T(h0.astype(np.complex64))
    gyt = S(cfg["gy"])
    glt = None if ghl is None else T(ghl.astype(np.complex64))
    g = ssm.complex_rtrl(gy=gyt, gh_last=glt, **t)
    g2 = ssm.complex_rtrl(gy=gyt, gh_last=glt, want_y=False, **t)
    bp = ssm.scan_bwd(ssm.SSM_COMPLEX_SHARED, gy=gyt, gh_last=glt, want=("glam", "gtheta"), **t)
    torch.cuda.synchronize()
    kw = _cplx_oracle_kw(cfg)
    h0c = None if h0 is None else h0.astype(np.complex64)
    o = oracle.complex_rtrl(**kw, h0=h0c, gy=cfg["gy"], ghlast=None if ghl is None else ghl.astype(np.complex64),
                            B=B, H=H, L=L, M=M)
    assert_close("y", g["y"], o["y"], **(BF16 if cfg.get("dtype") == "bf16" else F32))
    for k in ("glam", "gtheta"):
        assert_close(k, g[k], o[k], **F32)
        assert_close(k + " vs bptt", g[k], bp[k].cpu().numpy().astype(np.float64), rtol=2e-4, atol=2e-5)
        assert torch.equal(g[k], g2[k]), k


def test_complex_rtrl_small():
    cfg = synth.make_complex(B=2, H=3, M=64, L=300, seed=11)
    g = np.random.default_rng(12)
    run_complex_rtrl(cfg, h0=g.standard_normal((2, 3, 64)) + 1j * g.standard_normal((2, 3, 64)),
                     ghl=g.standard_normal((2, 3, 64)) + 1j * g.standard_normal((2, 3, 64)))


@pytest.mark.parametrize("M,L", [(5, 100), (64, 1), (64, 33), (17, 700)])
def test_complex_rtrl_shapes(M, L):
    run_complex_rtrl(synth.make_complex(B=1, H=2, M=M, L=L, seed=3 * M + L))


def test_complex_rtrl_many_segments():
    """B*H small, L long: many segments chained by the combine pass."""
    cfg = synth.make_complex(B=1, H=1, M=64, L=6000, seed=13)
    g = np.random.default_rng(14)
    run_complex_rtrl(cfg, h0=g.standard_normal((1, 1, 64)) + 1j * g.standard_normal((1, 1, 64)),
                     ghl=g.standard_normal((1, 1, 64)) + 1j * g.standard_normal((1, 1, 64)))


def test_complex_rtrl_large_phase_arguments():
    cfg = synth.make_complex(B=1, H=2, M=64, L=200, seed=22)
    cfg["phi"] = cfg["phi"].copy()
    cfg["phi"][:, :, 40:52] *= np.float32(3.0e7)
    run_complex_rtrl(cfg)


def test_complex_rtrl_full_config():
    """B=16 H=8 M=64 L=2048, seed 0."""
    run_complex_rtrl(synth.make_complex(B=16, H=8, M=64, L=2048, seed=0))


# ---------------------------------------------------------------------------
# PD
# ---------------------------------------------------------------------------
def run_pd(cfg, h0=None, ghl=None, use_sel=False):
    ssm = _ssm()
    B, H, L, N, K = cfg["B"], cfg["H"], cfg["L"], cfg["N"], cfg["K"]
    osel = oracle.pd_select(cfg["logits"])
    t = dict(dict=T(cfg["dict"]), d=S(cfg["d"]), b=S(cfg["b"]), C=S(cfg["C"]))
    if use_sel:
        t["sel"] = T(osel)
    else:
        t["logits"] = S(cfg["logits"])
    if h0 is not None:
        t["h0"] = T(h0.astype(np.float32))
    gyt = S(cfg["gy"])
    glt = None if ghl is None else T(ghl.astype(np.float32))
    f = ssm.pd_scan_fwd(want_h_last=True, want_ckpt=True, **t)
    g = ssm.pd_scan_bwd(gy=gyt, ckpt=f["ckpt"], gh_last=glt, **t)
    g2 = ssm.pd_scan_bwd(gy=gyt, gh_last=glt, **t)
    torch.cuda.synchronize()
    assert np.array_equal(f["sel"].cpu().numpy(), osel), "selection indices differ"
    kw = dict(sel=osel, dict=cfg["dict"], d=cfg["d"], b=cfg["b"], C=cfg["C"],
              h0=None if h0 is None else h0.astype(np.float32), B=B, H=H, L=L, N=N, K=K)
    y, hl = oracle.pd_fwd(**kw)
    og = oracle.pd_bwd(**kw, gy=cfg["gy"], ghlast=None if ghl is None else ghl.astype(np.float32))
    tol = BF16 if cfg.get("dtype") == "bf16" else F32
    assert_close("y", f["y"], y, **tol)
    assert_close("h_last", f["h_last"], hl, **tol)
    for k in ("gd", "gb", "gC", "gh0"):
        assert_close(k, g[k], og[k], **tol)
        assert torch.equal(g[k], g2[k]), k


def test_pd_out_of_range_indices_are_clamped():
    """Dictionary entries outside [0, N) and given selections outside [0, K) violate the documented
    precondition; the library clamps both, consistently in every pass: results equal the oracle's on the
    clamped arrays, and the reported selection is the clamped one."""
    ssm = _ssm()
    B, H, N, K, L = 2, 3, 16, 8, 700
    cfg = synth.make_pd(B=B, H=H, N=N, L=L, K=K, seed=47)
    dct = cfg["dict"].copy()
    dct[0, 1, 3], dct[1, 5, 0], dct[2, 7, 15] = -4, N + 3, 99
    sel = oracle.pd_select(cfg["logits"]).copy()
    sel[0, 0, 5], sel[1, 2, 600], sel[0, 1, 63] = -1, K, K + 20
    g = np.random.default_rng(48)
    h0 = g.standard_normal((B, H, N)).astype(np.float32)
    t = dict(sel=T(sel), dict=T(dct), d=T(cfg["d"]), b=T(cfg["b"]), C=T(cfg["C"]), h0=T(h0))
    f = ssm.pd_scan_fwd(want_h_last=True, want_ckpt=True, **t)
    gr = ssm.pd_scan_bwd(gy=T(cfg["gy"]), ckpt=f["ckpt"], **t)
    torch.cuda.synchronize()
    csel, cdict = np.clip(sel, 0, K - 1).astype(np.int32), np.clip(dct, 0, N - 1).astype(np.int32)
    assert np.array_equal(f["sel"].cpu().numpy(), csel)
    kw = dict(sel=csel, dict=cdict, d=cfg["d"], b=cfg["b"], C=cfg["C"], h0=h0, B=B, H=H, L=L, N=N, K=K)
    y, hl = oracle.pd_fwd(**kw)
    og = oracle.pd_bwd(**kw, gy=cfg["gy"])
    assert_close("y", f["y"], y, **F32)
    assert_close("h_last", f["h_last"], hl, **F32)
    for k in ("gd", "gb", "gC", "gh0"):
        assert_close(k, gr[k], og[k], **F32)


def test_pd_checkpoints_are_chunk_states():
    """ckpt[:, :, c] of the PD scan is the state entering 64-step chunk c: the oracle's final state of the first
    64c steps with the same selections (c = 0 holds h0)."""
    ssm = _ssm()
    B, H, N, K, L = 2, 3, 16, 8, 1000
    cfg = synth.make_pd(B=B, H=H, N=N, L=L, K=K, seed=43)
    h0 = np.random.default_rng(44).standard_normal((B, H, N)).astype(np.float32)
    t = dict(logits=T(cfg["logits"]), dict=T(cfg["dict"]), d=T(cfg["d"]), b=T(cfg["b"]), C=T(cfg["C"]), h0=T(h0))
    f = ssm.pd_scan_fwd(want_ckpt=True, **t)
    torch.cuda.synchronize()
    osel = oracle.pd_select(cfg["logits"])
    assert np.array_equal(f["sel"].cpu().numpy(), osel)
    ck = f["ckpt"]
    nc = -(-L // 64)
    assert ck.shape == (B, H, nc, N)
    assert torch.equal(ck[:, :, 0].cpu(), torch.from_numpy(h0))
    for c in (1, 2, 5, nc - 1):
        Lc = 64 * c
        _, hl = oracle.pd_fwd(sel=osel[:, :, :Lc], dict=cfg["dict"], d=cfg["d"][:, :, :Lc], b=cfg["b"][:, :, :Lc],
                              C=cfg["C"][:, :, :Lc], h0=h0, B=B, H=H, L=Lc, N=N, K=K)
        assert_close(f"ckpt[{c}]", ck[:, :, c], hl, **F32)


def run_pd_ste(cfg, tau, h0=None, ghl=None, with_ckpt=True):
    """Straight-through surrogate gradient of the selection scores against the
    oracle; the other PD gradients must be unchanged by asking for it."""
    ssm = _ssm()
    B, H, L, N, K = cfg["B"], cfg["H"], cfg["L"], cfg["N"], cfg["K"]
    osel = oracle.pd_select(cfg["logits"])
    t = dict(dict=T(cfg["dict"]), d=S(cfg["d"]), b=S(cfg["b"]), C=S(cfg["C"]), sel=T(osel))
    if h0 is not None:
        t["h0"] = T(h0.astype(np.float32))
    gyt = S(cfg["gy"])
    glt = None if ghl is None else T(ghl.astype(np.float32))
    lg = S(cfg["logits"])
    ck = ssm.pd_scan_fwd(want_ckpt=True, want_y=False, want_sel=False, **t)["ckpt"] if with_ckpt else None
    g = ssm.pd_scan_bwd(gy=gyt, ckpt=ck, gh_last=glt, ste_logits=lg, tau=tau,
                        want=("gd", "gb", "gC", "gh0", "glogits"), **t)
    g0 = ssm.pd_scan_bwd(gy=gyt, ckpt=ck, gh_last=glt, **t)
    torch.cuda.synchronize()
    o = oracle.pd_ste(logits=cfg["logits"], sel=osel, dict=cfg["dict"], d=cfg["d"], b=cfg["b"], C=cfg["C"],
                      h0=None if h0 is None else h0.astype(np.float32), gy=cfg["gy"],
                      ghlast=None if ghl is None else ghl.astype(np.float32), tau=tau, B=B, H=H, L=L, N=N, K=K)
    assert_close("glogits", g["glogits"], o["glogits"], **(BF16 if cfg.get("dtype") == "bf16" else F32))
    for k in ("gd", "gb", "gC", "gh0"):
        assert torch.equal(g[k], g0[k]), k


@pytest.mark.parametrize("tau", [0.5, 1.0, 4.0])
def test_pd_ste_small(tau):
    cfg = synth.make_pd(B=2, H=3, N=16, L=300, K=8, seed=31)
    g = np.random.default_rng(32)
    run_pd_ste(cfg, tau, h0=g.standard_normal((2, 3, 16)), ghl=g.standard_normal((2, 3, 16)))


@pytest.mark.parametrize("N,K,L", [(5, 3, 100), (16, 1, 70), (7, 64, 129), (16, 8, 1), (3, 17, 64)])
def test_pd_ste_shapes(N, K, L):
    run_pd_ste(synth.make_pd(B=1, H=2, N=N, L=L, K=K, seed=N * K + L), tau=1.0, with_ckpt=(L % 2 == 0))


def test_pd_ste_bf16():
    run_pd_ste(synth.make_pd(B=2, H=3, N=16, L=300, K=8, seed=33, dtype="bf16"), tau=1.0)


def test_pd_ste_full_config():
    """B=8 H=32 N=16 L=17000 K=8, seed 0, tau 1: every surrogate gradient compared."""
    run_pd_ste(synth.make_pd(B=8, H=32, N=16, L=17000, K=8, seed=0), tau=1.0)


def test_pd_bf16_streams():
    """bf16 logits, d, b, C, gy (selection bit-exact on the bf16 scores, many ties), fp32 state."""
    g = np.random.default_rng(41)
    run_pd(synth.make_pd(B=2, H=4, N=16, L=700, K=8, seed=40, dtype="bf16"),
           h0=g.standard_normal((2, 4, 16)), ghl=g.standard_normal((2, 4, 16)))


@pytest.mark.parametrize("case", ["d_one_identity", "d_zero", "b_zero"])
def test_pd_degenerate_inputs(case):
    """Degenerate PD steps: an identity dictionary with d = 1 (pure accumulation), d = 0 (the state is cleared
    every step), b = 0 (only h0 propagates); nonzero h0 and gh_last."""
    cfg = synth.make_pd(B=2, H=3, N=16, L=300, K=4, seed=33)
    g = np.random.default_rng(34)
    h0 = g.standard_normal((2, 3, 16))
    ghl = g.standard_normal((2, 3, 16))
    if case == "d_one_identity":
        cfg["dict"] = np.broadcast_to(np.arange(16, dtype=np.int32), cfg["dict"].shape).copy()
        cfg["d"] = np.ones_like(cfg["d"])
    elif case == "d_zero":
        cfg["d"] = np.zeros_like(cfg["d"])
    else:
        cfg["b"] = np.zeros_like(cfg["b"])
    run_pd(cfg, h0=h0, ghl=ghl)


def test_pd_small():
    cfg = synth.make_pd(B=2, H=3, N=16, L=500, K=8, seed=1)
    g = np.random.default_rng(2)
    run_pd(cfg, h0=g.standard_normal((2, 3, 16)), ghl=g.standard_normal((2, 3, 16)))


@pytest.mark.parametrize("N,K,L", [(16, 8, 1), (16, 8, 64), (16, 8, 65), (5, 3, 300), (16, 64, 200), (1, 1, 130)])
def test_pd_shapes(N, K, L):
    run_pd(synth.make_pd(B=1, H=2, N=N, L=L, K=K, seed=N * 100 + K + L))


@pytest.mark.parametrize("m", [16, 4, 3, 2, 1])
def test_pd_preimage_sizes(m):
    """Dictionary entries pi_k(j) = (j + k) mod m: largest preimage ceil(16 / m), so every gather round count
    (2, 4, 6, 8, 16) is exercised; rows >= m only receive b, which keeps the recurrence contractive."""
    cfg = synth.make_pd(B=1, H=2, N=16, L=400, K=8, seed=30 + m)
    j = np.arange(16)
    cfg["dict"] = np.stack([np.stack([(j + k) % m for k in range(8)]) for _ in range(2)]).astype(np.int32)
    run_pd(cfg)


def test_pd_given_selection():
    run_pd(synth.make_pd(B=1, H=2, N=16, L=777, K=8, seed=9), use_sel=True)


def test_pd_ties_lowest_index():
    cfg = synth.make_pd(B=1, H=2, N=16, L=300, K=8, seed=10)
    cfg["logits"] = np.round(cfg["logits"]).astype(np.float32)  # many exact ties
    run_pd(cfg)


def test_pd_dfa_exact():
    """Dictionary read as a 16-state automaton: d = 1, b = 0, h0 = e_q0 gives y_t = 2^{q_t} exactly."""
    ssm = _ssm()
    cfg = synth.make_pd(B=2, H=4, N=16, L=3000, K=8, seed=11)
    B, H, L, N = 2, 4, 3000, 16
    q0 = np.array([[3, 0, 15, 7], [1, 2, 9, 11]])
    h0 = np.zeros((B, H, N), np.float32)
    for bi in range(B):
        for hi in range(H):
            h0[bi, hi, q0[bi, hi]] = 1
    C = np.broadcast_to((2.0 ** np.arange(N)).astype(np.float32), (B, H, L, N)).copy()
    f = ssm.pd_scan_fwd(logits=T(cfg["logits"]), dict=T(cfg["dict"]), d=T(np.ones((B, H, L, N), np.float32)),
                        b=T(np.zeros((B, H, L, N), np.float32)), C=T(C), h0=T(h0))
    sel = f["sel"].cpu().numpy()
    y = f["y"].cpu().numpy()
    for bi in range(B):
        for hi in range(H):
            q = q0[bi, hi]
            for t in range(L):
                q = cfg["dict"][hi, sel[bi, hi, t], q]
                assert y[bi, hi, t] == 2.0 ** q


def test_pd_full_config():
    """B=8 H=32 N=16 L=17000 K=8, seed 0: selection bit-exact, values element-wise."""
    run_pd(synth.make_pd(B=8, H=32, N=16, L=17000, K=8, seed=0))
