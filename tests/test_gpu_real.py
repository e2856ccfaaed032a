"""GPU parity of the diagonal real selective scan (forward, backward, impulse
sensitivity) against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests._compare import BF16, F32, assert_close

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _dev(arr, dtype):
    if dtype == "bf16" and arr.dtype == np.uint16:
        return torch.from_numpy(arr.astype(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(DEV)


def _ssm():
    import selective_state_space_chunked_amd as ssm
    return ssm


def run_real(cfg, *, h0=None, ghl=None, chunk_len=0, tol=F32):
    ssm = _ssm()
    B, D, L, N, dt = cfg["B"], cfg["D"], cfg["L"], cfg["N"], cfg["dtype"]
    t = {k: _dev(cfg[k], dt) for k in ("delta", "x", "Bm", "C")}
    t["A"] = _dev(cfg["A"], "f32")
    if h0 is not None:
        t["h0"] = _dev(h0.astype(np.float32), "f32")
    gy = _dev(cfg["gy"], dt)
    f = ssm.scan_fwd(ssm.SSM_REAL_SELECTIVE, want_h_last=True, want_ckpt=True, chunk_len=chunk_len, **t)
    g = ssm.scan_bwd(ssm.SSM_REAL_SELECTIVE, gy=gy, ckpt=f["ckpt"], chunk_len=chunk_len,
                     gh_last=None if ghl is None else _dev(ghl.astype(np.float32), "f32"), **t)
    g2 = ssm.scan_bwd(ssm.SSM_REAL_SELECTIVE, gy=gy, ckpt=None, chunk_len=chunk_len,
                      gh_last=None if ghl is None else _dev(ghl.astype(np.float32), "f32"), **t)
    torch.cuda.synchronize()
    kw = dict(delta=cfg["delta"], x=cfg["x"], A=cfg["A"], Bm=cfg["Bm"], C=cfg["C"],
              h0=None if h0 is None else h0.astype(np.float32), B=B, D=D, L=L, N=N)
    y, hl = oracle.real_fwd(**kw)
    og = oracle.real_bwd(**kw, gy=cfg["gy"], ghlast=None if ghl is None else ghl.astype(np.float32))
    assert_close("y", f["y"], y, **tol)
    assert_close("h_last", f["h_last"], hl, **F32 if tol is F32 else tol)
    for k in ("gdelta", "gx", "gBm", "gC", "gA", "gh0"):
        assert_close(k, g[k], og[k], **tol)
    # recomputed checkpoints give the same gradients bit for bit
    for k in ("gdelta", "gx", "gBm", "gC", "gA", "gh0"):
        assert torch.equal(g[k], g2[k]), k
    return f, g


def test_real_small_config():
    """B=1 D=16 N=16 L=1024 fp32, seed 0 (segments run in parallel along L)."""
    run_real(synth.make_real(**{k: v for k, v in synth.CONFIGS["real-small"].items()}))


@pytest.mark.parametrize("chunk_len", [64, 128, 256])
def test_real_chunk_lengths_with_state(chunk_len):
    cfg = synth.make_real(B=2, D=24, N=16, L=777, seed=1)
    g = np.random.default_rng(2)
    run_real(cfg, h0=g.standard_normal((2, 24, 16)), ghl=g.standard_normal((2, 24, 16)), chunk_len=chunk_len)


@pytest.mark.parametrize("case", ["A_zero", "delta_zero", "delta_huge", "x_zero", "gy_zero", "mixed_channels"])
def test_real_degenerate_inputs(case):
    """Degenerate transitions and inputs: a = 1 (A = 0, or delta = 0 with no input), a underflowing to 0
    (delta = 1e3), no input (x = 0), no output gradient (gy = 0), and channels of both kinds in one workgroup;
    with a nonzero h0 and gh_last so the carried state and its adjoint matter."""
    cfg = synth.make_real(B=2, D=40, N=16, L=600, seed=21)
    g = np.random.default_rng(22)
    h0 = g.standard_normal((2, 40, 16))
    ghl = g.standard_normal((2, 40, 16))
    if case == "A_zero":
        cfg["A"] = np.zeros_like(cfg["A"])
    elif case == "delta_zero":
        cfg["delta"] = np.zeros_like(cfg["delta"])
    elif case == "delta_huge":
        cfg["delta"] = np.full_like(cfg["delta"], 1e3)
        cfg["x"] = (cfg["x"] * 1e-3).astype(np.float32)   # keeps b = delta x B of order one
    elif case == "x_zero":
        cfg["x"] = np.zeros_like(cfg["x"])
    elif case == "gy_zero":
        cfg["gy"] = np.zeros_like(cfg["gy"])
    else:
        cfg["A"][::3] = 0.0                                # every third channel accumulates
        cfg["delta"][:, 1::4] = 0.0                        # every fourth channel holds its state
    run_real(cfg, h0=h0, ghl=ghl)


@pytest.mark.parametrize("chunk_len,L", [(64, 777), (128, 777), (128, 896), (128, 1024), (256, 777)])
def test_real_checkpoints_are_chunk_states(chunk_len, L):
    """ckpt[:, :, c] is the state entering chunk c: the oracle's final state of the first c*T steps
    (at 128 steps the forward writes two checkpoints per 256-step tile)."""
    ssm = _ssm()
    cfg = synth.make_real(B=2, D=20, N=16, L=L, seed=11)
    g = np.random.default_rng(12)
    h0 = g.standard_normal((2, 20, 16)).astype(np.float32)
    t = {k: _dev(cfg[k], "f32") for k in ("delta", "x", "Bm", "C", "A")}
    f = ssm.scan_fwd(ssm.SSM_REAL_SELECTIVE, want_ckpt=True, chunk_len=chunk_len, h0=_dev(h0, "f32"), **t)
    torch.cuda.synchronize()
    ck = f["ckpt"].cpu().numpy()
    nc = -(-L // chunk_len)
    assert ck.shape == (2, 20, nc, 16)
    np.testing.assert_array_equal(ck[:, :, 0], h0)
    for c in range(1, nc):
        Lc = c * chunk_len
        _, hl = oracle.real_fwd(delta=cfg["delta"][:, :, :Lc], x=cfg["x"][:, :, :Lc], A=cfg["A"],
                                Bm=cfg["Bm"][:, :Lc], C=cfg["C"][:, :Lc], h0=h0, B=2, D=20, L=Lc, N=16)
        assert_close(f"ckpt[{c}]", torch.from_numpy(ck[:, :, c]), hl, **F32)


@pytest.mark.parametrize("L", [1, 2, 3, 63, 64, 65, 255, 257, 1000])
def test_real_ragged_lengths(L):
    run_real(synth.make_real(B=1, D=16, N=16, L=L, seed=L))


@pytest.mark.parametrize("N", [1, 5, 16])
def test_real_state_sizes(N):
    run_real(synth.make_real(B=2, D=8, N=N, L=300, seed=N))


def test_real_bf16_streams():
    """bf16 streams (reduced Mamba-layer shape), fp32 state and accumulation."""
    run_real(synth.make_real(B=2, D=256, N=16, L=1024, dtype="bf16", seed=0), tol=BF16)


def test_real_deterministic():
    cfg = synth.make_real(B=1, D=48, N=16, L=900, seed=3)
    f1, g1 = run_real(cfg)
    f2, g2 = run_real(cfg)
    assert torch.equal(f1["y"], f2["y"])
    for k in g1:
        assert torch.equal(g1[k], g2[k]), k


def test_sensitivities_deterministic():
    """The forward main passes that form the sensitivities give the same bits on every call (y, s; y, s_x,
    s_delta), with NaN-filled outputs so that an element left unwritten would show."""
    ssm = _ssm()
    cfg = synth.make_real(B=2, D=24, N=16, L=3000, dtype="f32", seed=9)
    t = {k: _dev(cfg[k], "f32") for k in ("delta", "x", "Bm", "C", "A")}
    runs = []
    for _ in range(2):
        out = {k: torch.full((2, 24, 3000), float("nan"), device="cuda") for k in ("y", "s")}
        ssm.impulse_sensitivity(t_out=2222, out=out, **t)
        os_ = {k: torch.full((2, 24, 3000), float("nan"), device="cuda") for k in ("y", "s_x", "s_delta")}
        ssm.output_sensitivity(t_out=2222, want_y=True, out=os_, **t)
        runs.append({**{"imp_" + k: v for k, v in out.items()}, **{"os_" + k: v for k, v in os_.items()}})
    torch.cuda.synchronize()
    for k in runs[0]:
        assert not torch.isnan(runs[0][k]).any(), k
        assert torch.equal(runs[0][k], runs[1][k]), k


def test_real_resume_split():
    """scan(L) equals scan(L1) followed by scan(L2) started from its h_last."""
    ssm = _ssm()
    cfg = synth.make_real(B=1, D=16, N=16, L=1280, seed=5)
    t = {k: _dev(cfg[k], "f32") for k in ("delta", "x", "Bm", "C", "A")}
    full = ssm.scan_fwd(ssm.SSM_REAL_SELECTIVE, want_h_last=True, **t)
    L1 = 512
    p1 = {k: (v[:, :, :L1].contiguous() if k in ("delta", "x") else v[:, :L1].contiguous() if k in ("Bm", "C") else v)
          for k, v in t.items()}
    p2 = {k: (v[:, :, L1:].contiguous() if k in ("delta", "x") else v[:, L1:].contiguous() if k in ("Bm", "C") else v)
          for k, v in t.items()}
    a = ssm.scan_fwd(ssm.SSM_REAL_SELECTIVE, want_h_last=True, **p1)
    b = ssm.scan_fwd(ssm.SSM_REAL_SELECTIVE, want_h_last=True, h0=a["h_last"], **p2)
    ycat = torch.cat([a["y"], b["y"]], dim=2)
    assert torch.allclose(ycat, full["y"], rtol=1e-5, atol=1e-6)
    assert torch.allclose(b["h_last"], full["h_last"], rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("t_out", [-1, 1234, 0])
def test_impulse_sensitivity(t_out):
    ssm = _ssm()
    cfg = synth.make_impulse(B=1, D=32, N=16, L=5000, seed=7)
    t = {k: _dev(cfg[k], "f32") for k in ("delta", "x", "Bm", "C", "A")}
    out = ssm.impulse_sensitivity(t_out=t_out, **t)
    torch.cuda.synchronize()
    kw = dict(delta=cfg["delta"], A=cfg["A"], Bm=cfg["Bm"], C=cfg["C"], B=1, D=32, L=5000, N=16)
    s = oracle.impulse_sens(**kw, t_out=None if t_out == -1 else t_out)
    y, _ = oracle.real_fwd(x=cfg["x"], **kw)
    assert_close("s", out["s"], s, **F32)
    assert_close("y", out["y"], y, **F32)


@pytest.mark.parametrize("dt,N,chunk_len,L,t_out", [
    ("bf16", 16, 256, 5500, 2999),   # 22 tiles: the last workgroup of tiles is partial
    ("f32", 5, 128, 3000, -1),       # generic state count, 128-step tiles
    ("f32", 16, 64, 2100, 1500),     # 64-step tiles
    ("bf16", 7, 256, 700, 0),
    ("f32", 16, 256, 4100, 2047),    # t_out at the last step of a tile
    ("f32", 16, 128, 4100, 2048),    # t_out at the first step of a tile
    ("f32", 16, 256, 200, 150),      # one tile: no segments, so the separate sensitivity pass
    ("bf16", 16, 64, 64, 63),
])
def test_impulse_sensitivity_variants(dt, N, chunk_len, L, t_out):
    """Sensitivity and y for bf16 streams, generic state counts and every tile length, against the oracle.
    With 16 states and the sequence cut into segments the forward's main pass forms s itself; otherwise a
    separate sensitivity pass does (N = 7 or 5, a single tile)."""
    ssm = _ssm()
    cfg = synth.make_real(B=2, D=20, N=N, L=L, dtype=dt, seed=40 + N + L)
    t = {k: _dev(cfg[k], dt) for k in ("delta", "x", "Bm", "C")}
    t["A"] = _dev(cfg["A"], "f32")
    out = ssm.impulse_sensitivity(t_out=t_out, chunk_len=chunk_len, **t)
    torch.cuda.synchronize()
    kw = dict(delta=cfg["delta"], A=cfg["A"], Bm=cfg["Bm"], C=cfg["C"], B=2, D=20, L=L, N=N)
    s = oracle.impulse_sens(**kw, t_out=None if t_out == -1 else t_out)
    y, _ = oracle.real_fwd(x=cfg["x"], **kw)
    tol = BF16 if dt == "bf16" else F32
    assert_close("s", out["s"], s, **tol)
    assert_close("y", out["y"], y, **tol)


@pytest.mark.parametrize("dt,N,L,t0,rows", [
    ("f32", 16, 777, 0, 1),       # the first output only
    ("f32", 16, 777, 100, 16),    # 16 rows inside a 64-step tile and across its end
    ("f32", 16, 777, 761, 16),    # the last 16 outputs, ragged last tile
    ("f32", 5, 600, 250, 7),      # generic state count
    ("bf16", 16, 1024, 511, 16),  # bf16 streams, rows across a tile boundary
    ("bf16", 7, 300, 40, 3),
])
def test_sensitivity_rows(dt, N, L, t0, rows):
    """Rows t0 .. t0+rows-1 of the input Jacobian against the oracle's impulse sensitivity of each row."""
    ssm = _ssm()
    cfg = synth.make_real(B=2, D=20, N=N, L=L, dtype=dt, seed=80 + N + L + rows)
    t = {k: _dev(cfg[k], dt) for k in ("delta", "x", "Bm", "C")}
    t["A"] = _dev(cfg["A"], "f32")
    s = ssm.sensitivity_rows(t_out0=t0, rows=rows, **t)
    torch.cuda.synchronize()
    assert s.shape == (rows, 2, 20, L)
    kw = dict(delta=cfg["delta"], A=cfg["A"], Bm=cfg["Bm"], C=cfg["C"], B=2, D=20, L=L, N=N)
    tol = BF16 if dt == "bf16" else F32
    for r in range(rows):
        assert_close(f"s[{r}]", s[r], oracle.impulse_sens(**kw, t_out=t0 + r), **tol)


@pytest.mark.parametrize("softplus,with_bias", [(True, True), (True, False), (False, True)])
def test_sensitivity_rows_projection_output(softplus, with_bias):
    """Rows of the Jacobian with the step sizes taken from the projection output (bias, softplus)."""
    ssm = _ssm()
    L = 500
    cfg = synth.make_real(B=1, D=24, N=16, L=L, seed=90, projection_output=True)
    if not softplus:   # keep the step sizes positive
        pos = oracle.step_sizes(cfg["delta"], cfg["delta_bias"], softplus=True)
        cfg["delta"] = (pos - cfg["delta_bias"][None, :, None]).astype(np.float32)
    bias = cfg["delta_bias"] if with_bias else None
    t = {k: _dev(cfg[k], "f32") for k in ("delta", "x", "Bm", "C", "A")}
    if with_bias:
        t["delta_bias"] = _dev(bias, "f32")
    t["delta_softplus"] = softplus
    s = ssm.sensitivity_rows(t_out0=300, rows=12, **t)
    torch.cuda.synchronize()
    dl = oracle.step_sizes(cfg["delta"], bias, softplus=softplus)
    kw = dict(delta=dl, A=cfg["A"], Bm=cfg["Bm"], C=cfg["C"], B=1, D=24, L=L, N=16)
    for r in range(12):
        assert_close(f"s[{r}]", s[r], oracle.impulse_sens(**kw, t_out=300 + r), **F32)


def test_sensitivity_rows_impulse_config():
    """The impulse workload's inputs at full length (B=1 D=1024 N=16 L=128000), the last 16 outputs;
    sampled channels against the oracle, every channel against the single-row call."""
    ssm = _ssm()
    L, D = 128000, 1024
    cfg = synth.make_impulse(B=1, D=D, N=16, L=L, seed=0)
    t = {k: _dev(cfg[k], "f32") for k in ("delta", "x", "Bm", "C", "A")}
    s = ssm.sensitivity_rows(t_out0=L - 16, rows=16, **t)
    one = ssm.impulse_sensitivity(t_out=L - 16, want_y=False, **t)["s"]
    torch.cuda.synchronize()
    assert_close("row 0 vs single-row call", s[0], one.cpu().numpy().astype(np.float64), rtol=1e-4, atol=1e-6)
    for d in (0, 517, 1023):
        kw = dict(delta=cfg["delta"][:, d:d + 1], A=cfg["A"][d:d + 1], Bm=cfg["Bm"], C=cfg["C"], B=1, D=1, L=L, N=16)
        for r in (0, 7, 15):
            assert_close(f"s[{r}] d={d}", s[r, :, d:d + 1], oracle.impulse_sens(**kw, t_out=L - 16 + r), **F32)


@pytest.mark.parametrize("dt,N,chunk_len,L,t_out,h0", [
    ("f32", 16, 256, 1300, -1, True),    # ragged last tile, t_out at the end, nonzero h0
    ("f32", 16, 256, 3000, 1777, False),  # t_out inside a tile, zero tail after it
    ("bf16", 16, 256, 2600, 2100, True),
    ("f32", 5, 128, 900, 450, True),      # generic state count, 128-step tiles
    ("f32", 16, 64, 700, 0, True),        # t_out = 0: only the first step is sensitive
    ("f32", 16, 256, 250, 100, True),     # one tile: no segments, so checkpoints and a separate pass
    ("bf16", 16, 128, 2000, 1023, False),  # t_out at the last step of a tile
])
def test_output_sensitivity(dt, N, chunk_len, L, t_out, h0):
    """d y[t_out]/d x and d y[t_out]/d delta (and y) against the oracle; s_x equal to the impulse path's.
    With 16 states and segments the forward's main pass forms both sensitivities from the states it re-runs;
    otherwise (N = 5, a single tile) the forward writes checkpoints and a separate pass re-runs them."""
    ssm = _ssm()
    cfg = synth.make_real(B=2, D=20, N=N, L=L, dtype=dt, seed=60 + N + L)
    t = {k: _dev(cfg[k], dt) for k in ("delta", "x", "Bm", "C")}
    t["A"] = _dev(cfg["A"], "f32")
    hh = None
    if h0:
        hh = np.random.default_rng(61).standard_normal((2, 20, N)).astype(np.float32)
        t["h0"] = torch.from_numpy(hh).cuda()
    out = ssm.output_sensitivity(t_out=t_out, want_y=True, chunk_len=chunk_len, **t)
    ref = ssm.impulse_sensitivity(t_out=t_out, want_y=False, chunk_len=chunk_len,
                                  **{k: v for k, v in t.items() if k != "h0"})
    torch.cuda.synchronize()
    kw = dict(delta=cfg["delta"], x=cfg["x"], A=cfg["A"], Bm=cfg["Bm"], C=cfg["C"], h0=hh, B=2, D=20, L=L, N=N)
    sx, sd = oracle.output_sens(**kw, t_out=None if t_out == -1 else t_out)
    y, _ = oracle.real_fwd(**kw)
    tol = BF16 if dt == "bf16" else F32
    assert_close("s_delta", out["s_delta"], sd, **tol)
    assert_close("s_x", out["s_x"], sx, **tol)
    assert_close("y", out["y"], y, **tol)
    # the impulse path forms each step's costate factor with its own exp, the delta path as suffix products of
    # the transitions it needs anyway: the same closed form, equal to rounding
    assert_close("s_x against the impulse path", out["s_x"], ref["s"].double().cpu().numpy(), **tol)


def test_sensitivity_very_long_sequence():
    """L = 17,000,000 with 64-step tiles: 265,625 tiles per sequence, more than the grid's z limit (65,535)
    times the tiles a workgroup takes by default; single-row and multi-row sensitivities against the oracle."""
    ssm = _ssm()
    L, D, N = 17_000_000, 2, 2
    cfg = synth.make_impulse(B=1, D=D, N=N, L=L, seed=3)
    t = {k: _dev(cfg[k], "f32") for k in ("delta", "x", "Bm", "C", "A")}
    out = ssm.impulse_sensitivity(t_out=L - 1, chunk_len=64, **t)
    rows = ssm.sensitivity_rows(t_out0=L - 4, rows=4, **t)
    torch.cuda.synchronize()
    kw = dict(delta=cfg["delta"], A=cfg["A"], Bm=cfg["Bm"], C=cfg["C"], B=1, D=D, L=L, N=N)
    s_last = oracle.impulse_sens(**kw, t_out=L - 1)
    assert_close("s", out["s"], s_last, **F32)
    assert_close("rows[3]", rows[3], s_last, **F32)
    assert_close("rows[0]", rows[0], oracle.impulse_sens(**kw, t_out=L - 4), **F32)
    y, _ = oracle.real_fwd(x=cfg["x"], **kw)
    assert_close("y", out["y"], y, **F32)


def test_output_sensitivity_impulse_config():
    """The impulse workload's inputs (x = e_0, slow decay), B=1 D=64 N=16 L=20000, y[L-1]."""
    ssm = _ssm()
    cfg = synth.make_impulse(B=1, D=64, N=16, L=20000, seed=8)
    t = {k: _dev(cfg[k], "f32") for k in ("delta", "x", "Bm", "C", "A")}
    out = ssm.output_sensitivity(**t)
    torch.cuda.synchronize()
    kw = dict(delta=cfg["delta"], x=cfg["x"], A=cfg["A"], Bm=cfg["Bm"], C=cfg["C"], B=1, D=64, L=20000, N=16)
    sx, sd = oracle.output_sens(**kw)
    assert_close("s_delta", out["s_delta"], sd, **F32)
    assert_close("s_x", out["s_x"], sx, **F32)


@pytest.mark.parametrize("dt,softplus,with_bias,L,chunk_len", [
    ("f32", True, True, 1000, 256),
    ("f32", True, False, 777, 128),
    ("f32", False, True, 300, 64),
    ("bf16", True, True, 1100, 256),
])
def test_step_sizes_from_projection(dt, softplus, with_bias, L, chunk_len):
    """delta = softplus(z + bias) merged into the scan: y, every gradient (w.r.t. z) and gdelta_bias."""
    ssm = _ssm()
    cfg = synth.make_real(B=2, D=24, N=16, L=L, dtype=dt, seed=70 + L, projection_output=True)
    if not softplus:   # step sizes must stay positive: feed softplus(z) - bias as the projection output
        pos = synth.make_real(B=2, D=24, N=16, L=L, dtype="f32", seed=70 + L)["delta"].astype(np.float64)
        assert dt == "f32"
        cfg["delta"] = (pos - (cfg["delta_bias"][None, :, None] if with_bias else 0.0)).astype(np.float32)
    t = {k: _dev(cfg[k], dt) for k in ("delta", "x", "Bm", "C")}
    t["A"] = _dev(cfg["A"], "f32")
    bias = cfg["delta_bias"] if with_bias else None
    if with_bias:
        t["delta_bias"] = _dev(bias, "f32")
    t["delta_softplus"] = softplus
    gy = _dev(cfg["gy"], dt)
    want = ("gdelta", "gx", "gA", "gBm", "gC", "gh0", "gdelta_bias")
    f = ssm.scan_fwd(ssm.SSM_REAL_SELECTIVE, want_h_last=True, want_ckpt=True, chunk_len=chunk_len, **t)
    g = ssm.scan_bwd(ssm.SSM_REAL_SELECTIVE, gy=gy, ckpt=f["ckpt"], want=want, chunk_len=chunk_len, **t)
    g2 = ssm.scan_bwd(ssm.SSM_REAL_SELECTIVE, gy=gy, want=want, chunk_len=chunk_len, **t)
    torch.cuda.synchronize()
    delta = oracle.step_sizes(cfg["delta"], bias, softplus)
    kw = dict(delta=delta, x=cfg["x"], A=cfg["A"], Bm=cfg["Bm"], C=cfg["C"], B=2, D=24, L=L, N=16)
    y, hl = oracle.real_fwd(**kw)
    og = oracle.real_bwd(**kw, gy=cfg["gy"])
    gz, gb = oracle.step_size_grads(og["gdelta"], cfg["delta"], bias, softplus)
    tol = BF16 if dt == "bf16" else F32
    assert_close("y", f["y"], y, **tol)
    assert_close("h_last", f["h_last"], hl, **tol)
    assert_close("gdelta (w.r.t. z)", g["gdelta"], gz, **tol)
    assert_close("gdelta_bias", g["gdelta_bias"], gb, **tol)
    for k in ("gx", "gBm", "gC", "gh0"):
        assert_close(k, g[k], og[k], **tol)
    for k in want:
        assert torch.equal(g[k], g2[k]), k


def test_step_sizes_from_projection_sensitivities():
    """The impulse and output-sensitivity paths with the transformed step sizes."""
    ssm = _ssm()
    L = 2300
    cfg = synth.make_real(B=1, D=20, N=16, L=L, seed=77, projection_output=True)
    t = {k: _dev(cfg[k], "f32") for k in ("delta", "x", "Bm", "C", "A", "delta_bias")}
    t["delta_softplus"] = True
    out = ssm.output_sensitivity(t_out=1500, want_y=True, **t)
    imp = ssm.impulse_sensitivity(t_out=1500, want_y=False, **t)   # separate sensitivity pass
    impy = ssm.impulse_sensitivity(t_out=1500, want_y=True, **t)   # formed by the forward's main pass
    torch.cuda.synchronize()
    delta = oracle.step_sizes(cfg["delta"], cfg["delta_bias"], True)
    kw = dict(delta=delta, x=cfg["x"], A=cfg["A"], Bm=cfg["Bm"], C=cfg["C"], B=1, D=20, L=L, N=16)
    sx, sd = oracle.output_sens(**kw, t_out=1500)
    sz, _ = oracle.step_size_grads(sd, cfg["delta"], cfg["delta_bias"], True)
    y, _ = oracle.real_fwd(**kw)
    assert_close("s_x", out["s_x"], sx, **F32)
    assert_close("s_z", out["s_delta"], sz, **F32)
    assert_close("y", out["y"], y, **F32)
    assert_close("impulse s", imp["s"], sx, **F32)
    assert_close("impulse s (with y)", impy["s"], sx, **F32)
    assert_close("impulse y", impy["y"], y, **F32)
