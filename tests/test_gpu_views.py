"""GPU parity of strided and broadcast views, per-channel B_t / C_t and the zero-order-hold input term,
through the C ABI, against the fp64 oracle run on dense copies of the same values.  Gradients of a
broadcast input are compared per broadcast position (the oracle sees the expanded array)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests._compare import BF16, F32, assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _ssm():
    import selective_state_space_chunked_amd as ssm
    return ssm


def T(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def bf(a):
    """bf16 bits (uint16) -> bf16 tensor on the GPU."""
    return torch.from_numpy(np.ascontiguousarray(a).astype(np.int16)).view(torch.bfloat16).to(DEV)


def npy(t):
    """The values a view holds, as a dense array the oracle reads (bf16 as its bits)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().astype(np.uint16)
    return t.numpy()


def _embed(a, shape, index, fill=7.0):
    """A bigger tensor holding `a` at `index`, so that the result is a strided view of it."""
    big = torch.full(shape, fill, dtype=a.dtype, device=a.device)
    big[index] = a
    return big[index]


def test_selective_views_fwd_bwd():
    """x and delta as slices of bigger buffers, A shared by the channels (stride 0), B_t shared by the batch
    rows (stride 0), C_t with padded steps, y and gx written into slices of bigger outputs, gy a slice."""
    ssm = _ssm()
    B, D, N, L = 2, 24, 16, 777
    cfg = synth.make_real(B=B, D=D, N=N, L=L, seed=31)
    g = np.random.default_rng(32)
    x = _embed(T(cfg["x"]), (B, 2 * D, L), (slice(None), slice(0, 2 * D, 2)))
    delta = _embed(T(cfg["delta"]), (B, D, L + 23), (slice(None), slice(None), slice(5, 5 + L)))
    A = T(cfg["A"][:1]).expand(D, N)
    Bm = T(cfg["Bm"][:1]).expand(B, L, N)
    C = _embed(T(cfg["C"]), (B, L, 2 * N), (slice(None), slice(None), slice(N, 2 * N)))
    gy = _embed(T(cfg["gy"]), (B, D, 2 * L), (slice(None), slice(None), slice(L, 2 * L)))
    h0 = g.standard_normal((B, D, N)).astype(np.float32)
    ghl = g.standard_normal((B, D, N)).astype(np.float32)
    t = dict(delta=delta, x=x, A=A, Bm=Bm, C=C, h0=T(h0))
    ybig = torch.full((B, D + 3, L), float("nan"), device=DEV)
    gxbig = torch.full((3, B, D, L), float("nan"), device=DEV)
    f = ssm.scan_fwd(ssm.SSM_REAL_SELECTIVE, want_h_last=True, want_ckpt=True, out={"y": ybig[:, 2:2 + D]}, **t)
    # gA (a sum over batch and time of terms of both signs, at the edge of the fp32 bound for some entries)
    # is left to the dense tests; y and gdelta already depend on the shared A
    gr = ssm.scan_bwd(ssm.SSM_REAL_SELECTIVE, gy=gy, ckpt=f["ckpt"], gh_last=T(ghl),
                      want=("gdelta", "gx", "gBm", "gC", "gh0"), out={"gx": gxbig[1]}, **t)
    torch.cuda.synchronize()
    kw = dict(delta=npy(delta), x=npy(x), A=npy(A), Bm=npy(Bm), C=npy(C), h0=h0, B=B, D=D, L=L, N=N)
    y, hl = oracle.real_fwd(**kw)
    og = oracle.real_bwd(**kw, gy=npy(gy), ghlast=ghl)
    assert_close("y (view)", ybig[:, 2:2 + D], y, **F32)
    assert torch.isnan(ybig[:, :2]).all() and torch.isnan(ybig[:, 2 + D:]).all()   # nothing outside the view
    assert_close("h_last", f["h_last"], hl, **F32)
    assert_close("gx (view)", gxbig[1], og["gx"], **F32)
    assert torch.isnan(gxbig[0]).all() and torch.isnan(gxbig[2]).all()
    for k in ("gdelta", "gBm", "gC", "gh0"):
        assert_close(k, gr[k], og[k], **F32)


@pytest.mark.parametrize("dt,N,L,chunk_len", [("f32", 16, 700, 256), ("bf16", 16, 1100, 256), ("f32", 5, 500, 128),
                                              ("f32", 16, 300, 64)])
def test_selective_per_channel_BC(dt, N, L, chunk_len):
    """B_t and C_t per channel (B,D,L,N): y and every gradient, gB and gC per channel, against the oracle's
    per-channel form; C as a strided view."""
    ssm = _ssm()
    B, D = 2, 20
    cfg = synth.make_real(B=B, D=D, N=N, L=L, dtype=dt, seed=33 + N)
    g = np.random.default_rng(34)
    Bpd = g.standard_normal((B, D, L, N)) / np.sqrt(N)
    Cpd = g.standard_normal((B, D, L, N)) / np.sqrt(N)
    conv = bf if dt == "bf16" else T
    if dt == "bf16":
        Bpd, Cpd = synth.gen._stream(Bpd, "bf16"), synth.gen._stream(Cpd, "bf16")
    else:
        Bpd, Cpd = Bpd.astype(np.float32), Cpd.astype(np.float32)
    t = {k: conv(cfg[k]) for k in ("delta", "x")}
    t["A"] = T(cfg["A"])
    t["Bm"] = conv(Bpd)
    t["C"] = _embed(conv(Cpd), (B, D + 1, L, N), (slice(None), slice(1, D + 1)), fill=3.0)
    h0 = g.standard_normal((B, D, N)).astype(np.float32)
    t["h0"] = T(h0)
    f = ssm.scan_fwd(ssm.SSM_REAL_SELECTIVE, want_h_last=True, want_ckpt=True, chunk_len=chunk_len, **t)
    gr = ssm.scan_bwd(ssm.SSM_REAL_SELECTIVE, gy=conv(cfg["gy"]), ckpt=f["ckpt"], chunk_len=chunk_len,
                      want=("gdelta", "gx", "gA", "gBm", "gC", "gh0"), **t)
    gr2 = ssm.scan_bwd(ssm.SSM_REAL_SELECTIVE, gy=conv(cfg["gy"]), chunk_len=chunk_len,
                       want=("gdelta", "gx", "gBm", "gC"), **t)
    torch.cuda.synchronize()
    assert gr["gBm"].shape == (B, D, L, N) and gr["gC"].shape == (B, D, L, N)
    kw = dict(delta=cfg["delta"], x=cfg["x"], A=cfg["A"], Bm=Bpd, C=Cpd, h0=h0, perd=True, B=B, D=D, L=L, N=N)
    y, hl = oracle.sel_fwd(**kw)
    og = oracle.sel_bwd(**kw, gy=cfg["gy"])
    tol = BF16 if dt == "bf16" else F32
    assert_close("y", f["y"], y, **tol)
    assert_close("h_last", f["h_last"], hl, **F32)
    for k in ("gdelta", "gx", "gBm", "gC"):
        assert_close(k, gr[k], og[k], **tol)
        assert torch.equal(gr[k], gr2[k]), k
    assert_close("gh0", gr["gh0"], og["gh0"], **F32)
    if dt == "f32":
        assert_close("gA", gr["gA"], og["gA"], **F32)


def test_selective_per_channel_B_shared_C():
    """A per-channel B_t next to a C_t shared by the channels: both are read per channel and both gradients
    come back per channel (gC per broadcast position)."""
    ssm = _ssm()
    B, D, N, L = 1, 16, 16, 600
    cfg = synth.make_real(B=B, D=D, N=N, L=L, seed=35)
    Bpd = (np.random.default_rng(36).standard_normal((B, D, L, N)) / 4).astype(np.float32)
    t = {k: T(cfg[k]) for k in ("delta", "x", "A", "C")}
    t["Bm"] = T(Bpd)
    f = ssm.scan_fwd(ssm.SSM_REAL_SELECTIVE, want_ckpt=True, **t)
    gr = ssm.scan_bwd(ssm.SSM_REAL_SELECTIVE, gy=T(cfg["gy"]), ckpt=f["ckpt"], want=("gdelta", "gx", "gBm", "gC"),
                      **t)
    torch.cuda.synchronize()
    Cx = np.repeat(cfg["C"][:, None], D, axis=1)
    kw = dict(delta=cfg["delta"], x=cfg["x"], A=cfg["A"], Bm=Bpd, C=Cx, perd=True, B=B, D=D, L=L, N=N)
    y, _ = oracle.sel_fwd(**kw)
    og = oracle.sel_bwd(**kw, gy=cfg["gy"])
    assert_close("y", f["y"], y, **F32)
    for k in ("gdelta", "gx", "gBm", "gC"):
        assert_close(k, gr[k], og[k], **F32)


@pytest.mark.parametrize("dt,N,L,chunk_len", [("f32", 16, 777, 256), ("f32", 16, 1000, 64), ("bf16", 16, 1300, 256),
                                              ("f32", 7, 600, 128)])
def test_zoh_fwd_bwd(dt, N, L, chunk_len):
    """The zero-order-hold input term: y, h_last and every gradient (gA included) against the oracle; A has
    a zero entry (the delta x B limit) and tiny ones (the series branch of the coefficient)."""
    ssm = _ssm()
    B, D = 2, 24
    cfg = synth.make_real(B=B, D=D, N=N, L=L, dtype=dt, seed=37 + N + L)
    cfg["A"][0, 0] = 0.0
    cfg["A"][1, : min(N, 3)] = np.float32(-2e-4)
    conv = bf if dt == "bf16" else T
    g = np.random.default_rng(38)
    h0 = g.standard_normal((B, D, N)).astype(np.float32)
    ghl = g.standard_normal((B, D, N)).astype(np.float32)
    t = {k: conv(cfg[k]) for k in ("delta", "x", "Bm", "C")}
    t["A"] = T(cfg["A"])
    t["h0"] = T(h0)
    t["discretization"] = ssm.SSM_ZOH
    f = ssm.scan_fwd(ssm.SSM_REAL_SELECTIVE, want_h_last=True, want_ckpt=True, chunk_len=chunk_len, **t)
    want = ("gdelta", "gx", "gA", "gBm", "gC", "gh0")
    gr = ssm.scan_bwd(ssm.SSM_REAL_SELECTIVE, gy=conv(cfg["gy"]), ckpt=f["ckpt"], gh_last=T(ghl), want=want,
                      chunk_len=chunk_len, **t)
    gr2 = ssm.scan_bwd(ssm.SSM_REAL_SELECTIVE, gy=conv(cfg["gy"]), gh_last=T(ghl), want=want,
                       chunk_len=chunk_len, **t)
    torch.cuda.synchronize()
    kw = dict(delta=cfg["delta"], x=cfg["x"], A=cfg["A"], Bm=cfg["Bm"], C=cfg["C"], h0=h0, disc=1,
              B=B, D=D, L=L, N=N)
    y, hl = oracle.sel_fwd(**kw)
    og = oracle.sel_bwd(**kw, gy=cfg["gy"], ghlast=ghl)
    tol = BF16 if dt == "bf16" else F32
    assert_close("y", f["y"], y, **tol)
    assert_close("h_last", f["h_last"], hl, **F32)
    for k in ("gdelta", "gx", "gBm", "gC"):
        assert_close(k, gr[k], og[k], **tol)
    assert_close("gh0", gr["gh0"], og["gh0"], **F32)
    if dt == "f32":
        assert_close("gA", gr["gA"], og["gA"], **F32)
    for k in want:
        assert torch.equal(gr[k], gr2[k]), k


def test_zoh_noalloc_forward():
    """The allocation-free forward takes the ZOH term too (bit-equal to the workspace forward)."""
    ssm = _ssm()
    cfg = synth.make_real(B=1, D=32, N=16, L=3000, seed=39)
    t = {k: T(cfg[k]) for k in ("delta", "x", "Bm", "C", "A")}
    t["discretization"] = ssm.SSM_ZOH
    a = ssm.scan_fwd(ssm.SSM_REAL_SELECTIVE, want_ckpt=True, **t)
    b = ssm.scan_fwd_noalloc(ssm.SSM_REAL_SELECTIVE, want_ckpt=True, **t)
    torch.cuda.synchronize()
    assert torch.equal(a["y"], b["y"]) and torch.equal(a["ckpt"], b["ckpt"])


def test_sensitivities_take_views():
    """The impulse and output sensitivities and the Jacobian rows with delta a slice, A shared by the channels
    and B_t, C_t shared by the batch rows."""
    ssm = _ssm()
    B, D, N, L = 2, 16, 16, 1500
    cfg = synth.make_real(B=B, D=D, N=N, L=L, seed=40)
    delta = _embed(T(cfg["delta"]), (B, 2 * D, L), (slice(None), slice(D, 2 * D)))
    t = dict(delta=delta, x=T(cfg["x"]), A=T(cfg["A"][:1]).expand(D, N), Bm=T(cfg["Bm"][:1]).expand(B, L, N),
             C=T(cfg["C"][:1]).expand(B, L, N))
    out = ssm.impulse_sensitivity(t_out=1234, **t)
    rows = ssm.sensitivity_rows(t_out0=1000, rows=3, **t)
    osn = ssm.output_sensitivity(t_out=1234, want_y=True, **t)
    torch.cuda.synchronize()
    kw = dict(delta=npy(delta), A=npy(t["A"]), Bm=npy(t["Bm"]), C=npy(t["C"]), B=B, D=D, L=L, N=N)
    assert_close("s", out["s"], oracle.impulse_sens(**kw, t_out=1234), **F32)
    sx, sd = oracle.output_sens(x=cfg["x"], **kw, t_out=1234)
    assert_close("s_x", osn["s_x"], sx, **F32)
    assert_close("s_delta", osn["s_delta"], sd, **F32)
    assert_close("y (output sensitivity)", osn["y"], oracle.real_fwd(x=cfg["x"], **kw)[0], **F32)
    y, _ = oracle.real_fwd(x=cfg["x"], **kw)
    assert_close("y", out["y"], y, **F32)
    for r in range(3):
        assert_close(f"rows[{r}]", rows[r], oracle.impulse_sens(**kw, t_out=1000 + r), **F32)


def test_complex_controls_shared_by_heads():
    """r, phi one signal for all heads (stride 0 over heads), lam, theta, c shared by the heads, u a slice;
    gradients of the shared inputs come back per head."""
    ssm = _ssm()
    B, H, M, L = 2, 3, 64, 300
    cfg = synth.make_complex(B=B, H=H, M=M, L=L, seed=41)
    r = T(cfg["r"][:, :1]).expand(B, H, L)
    phi = T(cfg["phi"][:, :1]).expand(B, H, L)
    lam = T(cfg["lam"][:1]).expand(H, M)
    theta = T(cfg["theta"][:1]).expand(H, M)
    c = T(cfg["c"][:1]).expand(H, M)
    u = _embed(T(cfg["u"]), (B, H, L + 9, M), (slice(None), slice(None), slice(9, 9 + L)), fill=0.0)
    t = dict(r=r, phi=phi, lam=lam, theta=theta, u=u, c=c)
    f = ssm.scan_fwd(ssm.SSM_COMPLEX_SHARED, want_h_last=True, want_ckpt=True, **t)
    gr = ssm.scan_bwd(ssm.SSM_COMPLEX_SHARED, gy=T(cfg["gy"]), ckpt=f["ckpt"], **t)
    rt = ssm.complex_rtrl(gy=T(cfg["gy"]), **t)
    torch.cuda.synchronize()
    kw = {k: npy(v) for k, v in t.items()}
    y, hl = oracle.complex_fwd(**kw, B=B, H=H, L=L, M=M)
    og = oracle.complex_bwd(**kw, gy=cfg["gy"], B=B, H=H, L=L, M=M)
    assert_close("y", f["y"], y, **F32)
    assert_close("h_last", f["h_last"], hl, **F32)
    for k in ("gu", "gr", "gphi", "glam", "gtheta", "gc"):
        assert_close(k, gr[k], og[k], **F32)
    assert_close("rtrl glam", rt["glam"], og["glam"], **F32)
    assert_close("rtrl gtheta", rt["gtheta"], og["gtheta"], **F32)
    assert_close("rtrl y", rt["y"], y, **F32)


def test_pd_shared_dictionary_and_views():
    """One dictionary for all heads (stride 0 over heads); logits, d, b and C slices of bigger buffers."""
    ssm = _ssm()
    B, H, N, K, L = 2, 4, 16, 8, 700
    cfg = synth.make_pd(B=B, H=H, N=N, L=L, K=K, seed=42)
    dct = T(cfg["dict"][:1]).expand(H, K, N)
    sl = (slice(None), slice(None), slice(3, 3 + L))
    logits = _embed(T(cfg["logits"]), (B, H, L + 3, K), sl)
    d = _embed(T(cfg["d"]), (B, H, L + 3, N), sl)
    b = _embed(T(cfg["b"]), (B, H, L + 3, N), sl)
    C = T(cfg["C"])
    t = dict(logits=logits, dict=dct, d=d, b=b, C=C)
    f = ssm.pd_scan_fwd(want_h_last=True, want_ckpt=True, **t)
    gr = ssm.pd_scan_bwd(gy=T(cfg["gy"]), ckpt=f["ckpt"], **t)
    torch.cuda.synchronize()
    osel = oracle.pd_select(npy(logits))
    assert np.array_equal(f["sel"].cpu().numpy(), osel)
    kw = dict(sel=osel, dict=npy(dct), d=npy(d), b=npy(b), C=cfg["C"], B=B, H=H, L=L, N=N, K=K)
    y, hl = oracle.pd_fwd(**kw)
    og = oracle.pd_bwd(**kw, gy=cfg["gy"])
    assert_close("y", f["y"], y, **F32)
    assert_close("h_last", f["h_last"], hl, **F32)
    for k in ("gd", "gb", "gC", "gh0"):
        assert_close(k, gr[k], og[k], **F32)
