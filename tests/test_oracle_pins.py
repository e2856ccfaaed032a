"""Pins of the fp64 oracle against facts the mathematics fixes (CPU only).

Each test computes its expected value by an independent route (an unrolled
brute-force sum, a closed form, a dense-matrix product, finite differences of
the forward, an automaton simulation, a worked example) so that a dropped
term, a wrong sign, an off-by-one index or a transposed operand in oracle.c
fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(1234)


def close(a, b, rtol=1e-12, atol=1e-14):
    a = np.asarray(a)
    b = np.asarray(b)
    assert a.shape == b.shape, (a.shape, b.shape)
    err = np.abs(a - b)
    bound = atol + rtol * np.abs(b)
    bad = err > bound
    assert not bad.any(), f"max err {err.max():.3e} at {np.unravel_index(np.argmax(err - bound), err.shape)}"


def small_real(B=2, D=3, N=4, L=17, seed=0):
    g = np.random.default_rng(seed)
    return dict(
        delta=np.log1p(np.exp(g.standard_normal((B, D, L)))),
        x=g.standard_normal((B, D, L)),
        A=-np.exp(g.uniform(-3, -1, (D, N))),
        Bm=g.standard_normal((B, L, N)) / 2,
        C=g.standard_normal((B, L, N)) / 2,
        h0=g.standard_normal((B, D, N)),
        gy=g.standard_normal((B, D, L)),
        ghlast=g.standard_normal((B, D, N)),
        B=B, D=D, N=N, L=L,
    )


# ---------------------------------------------------------------------------
# real forward
# ---------------------------------------------------------------------------
def brute_real(a, b, C, h0):
    """h_t = sum_{s<=t} (prod_{r=s+1..t} a_r) b_s + (prod_{r<=t} a_r) h0, unrolled."""
    L, N = a.shape
    y = np.zeros(L)
    H = np.zeros((L, N))
    for t in range(L):
        for n in range(N):
            v = h0[n]
            for r in range(0, t + 1):
                v = v * a[r, n]
            acc = v
            for s in range(t + 1):
                p = b[s, n]
                for r in range(s + 1, t + 1):
                    p = p * a[r, n]
                acc += p
            H[t, n] = acc
        y[t] = sum(C[t, n] * H[t, n] for n in range(N))
    return y, H


def test_real_selective_fwd_bruteforce():
    p = small_real(B=2, D=2, N=3, L=20)
    y, hl = oracle.real_fwd(delta=p["delta"], x=p["x"], A=p["A"], Bm=p["Bm"], C=p["C"], h0=p["h0"],
                            B=2, D=2, L=20, N=3)
    for bi in range(2):
        for di in range(2):
            a = np.exp(p["delta"][bi, di][:, None] * p["A"][di][None, :])
            bb = (p["delta"][bi, di] * p["x"][bi, di])[:, None] * p["Bm"][bi]
            yb, H = brute_real(a, bb, p["C"][bi], p["h0"][bi, di])
            close(y[bi, di], yb, rtol=1e-12, atol=1e-13)
            close(hl[bi, di], H[-1], rtol=1e-12, atol=1e-13)


def test_real_dense_fwd_bruteforce():
    g = np.random.default_rng(7)
    B, D, L, N = 1, 2, 24, 4
    a = g.uniform(-1.1, 1.1, (B, D, L, N))
    b = g.standard_normal((B, D, L, N))
    C = g.standard_normal((B, L, N))
    h0 = g.standard_normal((B, D, N))
    y, hl = oracle.real_fwd(a=a, b=b, C=C, h0=h0, B=B, D=D, L=L, N=N)
    for di in range(D):
        yb, H = brute_real(a[0, di], b[0, di], C[0], h0[0, di])
        close(y[0, di], yb, rtol=1e-11, atol=1e-12)
        close(hl[0, di], H[-1], rtol=1e-11, atol=1e-12)


def test_real_geometric_closed_form():
    B, D, L, N = 1, 3, 300, 4
    alpha = np.array([0.3, 0.9, 0.999, 1.0])
    beta = np.array([1.0, -2.0, 0.5, 0.25])
    h0 = RNG.standard_normal((B, D, N))
    a = np.broadcast_to(alpha, (B, D, L, N)).copy()
    b = np.broadcast_to(beta, (B, D, L, N)).copy()
    C = np.zeros((B, L, N))
    C[:, :, 1] = 1.0  # y reads state 1 only
    y, hl = oracle.real_fwd(a=a, b=b, C=C, h0=h0, B=B, D=D, L=L, N=N)
    t1 = L  # number of steps taken
    for n in range(N):
        if alpha[n] == 1.0:
            want = h0[0, :, n] + t1 * beta[n]
        else:
            want = alpha[n] ** t1 * h0[0, :, n] + beta[n] * (1 - alpha[n] ** t1) / (1 - alpha[n])
        close(hl[0, :, n], want, rtol=1e-12, atol=1e-12)
    ts = np.arange(1, L + 1)
    want_y = alpha[1] ** ts[None, :] * h0[0, :, 1][:, None] + beta[1] * (1 - alpha[1] ** ts) / (1 - alpha[1])
    close(y[0], want_y, rtol=1e-12, atol=1e-12)


def test_real_prefix_sum_special_case():
    """A = 0 gives a_t = 1: the state is the prefix sum of the input terms."""
    p = small_real(B=1, D=2, N=3, L=50)
    A = np.zeros_like(p["A"])
    y, hl = oracle.real_fwd(delta=p["delta"], x=p["x"], A=A, Bm=p["Bm"], C=p["C"], h0=p["h0"],
                            B=1, D=2, L=50, N=3)
    for di in range(2):
        bb = (p["delta"][0, di] * p["x"][0, di])[:, None] * p["Bm"][0]
        H = p["h0"][0, di][None, :] + np.cumsum(bb, axis=0)
        close(hl[0, di], H[-1], rtol=1e-12, atol=1e-12)
        close(y[0, di], (p["C"][0] * H).sum(axis=1), rtol=1e-11, atol=1e-12)


def test_real_golden_worked_example():
    g = json.load(open(os.path.join(GOLD, "dense_real_worked.json")))
    L, N = g["L"], g["N"]
    a = np.array(g["a"]).reshape(1, 1, L, N)
    b = np.array(g["b"]).reshape(1, 1, L, N)
    C = np.array(g["C"]).reshape(1, L, N)
    h0 = np.array(g["h0"]).reshape(1, 1, N)
    y, hl = oracle.real_fwd(a=a, b=b, C=C, h0=h0, B=1, D=1, L=L, N=N)
    assert y.ravel().tolist() == g["y"]
    assert hl.ravel().tolist() == g["h_last"]
    gr = oracle.real_bwd(a=a, b=b, C=C, h0=h0, gy=np.array(g["gy"]).reshape(1, 1, L), B=1, D=1, L=L, N=N)
    assert gr["gb"].ravel().tolist() == g["gb"]
    assert gr["ga"].ravel().tolist() == g["ga"]
    assert gr["gh0"].ravel().tolist() == g["gh0"]


# ---------------------------------------------------------------------------
# real backward
# ---------------------------------------------------------------------------
def _loss_real(p, **over):
    q = dict(p)
    q.update(over)
    kw = {k: q[k] for k in ("delta", "x", "A", "Bm", "C", "h0")}
    y, hl = oracle.real_fwd(**kw, B=q["B"], D=q["D"], L=q["L"], N=q["N"])
    return float((y * q["gy"]).sum() + (hl * q["ghlast"]).sum())


def fd_check(loss, p, name, grad, rtol=2e-6, atol=1e-8):
    base = p[name]
    num = np.zeros_like(base)
    it = np.nditer(base, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        v = base[idx]
        eps = 1e-6 * max(1.0, abs(v))
        hi = base.copy()
        hi[idx] = v + eps
        lo = base.copy()
        lo[idx] = v - eps
        num[idx] = (loss(p, **{name: hi}) - loss(p, **{name: lo})) / (2 * eps)
    close(grad, num, rtol=rtol, atol=atol)


@pytest.mark.parametrize("name,gname", [("delta", "gdelta"), ("x", "gx"), ("A", "gA"),
                                        ("Bm", "gBm"), ("C", "gC"), ("h0", "gh0")])
def test_real_selective_bwd_fd(name, gname):
    p = small_real(B=2, D=2, N=3, L=9, seed=3)
    g = oracle.real_bwd(delta=p["delta"], x=p["x"], A=p["A"], Bm=p["Bm"], C=p["C"], h0=p["h0"],
                        gy=p["gy"], ghlast=p["ghlast"], B=2, D=2, L=9, N=3)
    fd_check(_loss_real, p, name, g[gname])


def _dense_p(seed=5, B=2, D=2, L=8, N=3):
    g = np.random.default_rng(seed)
    return dict(a=g.uniform(-1, 1, (B, D, L, N)), b=g.standard_normal((B, D, L, N)),
                C=g.standard_normal((B, L, N)), h0=g.standard_normal((B, D, N)),
                gy=g.standard_normal((B, D, L)), ghlast=g.standard_normal((B, D, N)),
                B=B, D=D, L=L, N=N)


def _loss_dense(p, **over):
    q = dict(p)
    q.update(over)
    y, hl = oracle.real_fwd(a=q["a"], b=q["b"], C=q["C"], h0=q["h0"], B=q["B"], D=q["D"], L=q["L"], N=q["N"])
    return float((y * q["gy"]).sum() + (hl * q["ghlast"]).sum())


@pytest.mark.parametrize("name,gname", [("a", "ga"), ("b", "gb"), ("C", "gC"), ("h0", "gh0")])
def test_real_dense_bwd_fd(name, gname):
    p = _dense_p()
    g = oracle.real_bwd(a=p["a"], b=p["b"], C=p["C"], h0=p["h0"], gy=p["gy"], ghlast=p["ghlast"],
                        B=2, D=2, L=8, N=3)
    fd_check(_loss_dense, p, name, g[gname])


def test_real_adjoint_identity():
    """y and h_last are linear in (b, h0): <gy,y> + <ghl,h_last> = <gb,b> + <gh0,h0>."""
    p = _dense_p(seed=11, B=2, D=3, L=64, N=4)
    y, hl = oracle.real_fwd(a=p["a"], b=p["b"], C=p["C"], h0=p["h0"], B=2, D=3, L=64, N=4)
    g = oracle.real_bwd(a=p["a"], b=p["b"], C=p["C"], h0=p["h0"], gy=p["gy"], ghlast=p["ghlast"],
                        B=2, D=3, L=64, N=4)
    lhs = (y * p["gy"]).sum() + (hl * p["ghlast"]).sum()
    rhs = (g["gb"] * p["b"]).sum() + (g["gh0"] * p["h0"]).sum()
    assert abs(lhs - rhs) <= 1e-11 * max(1.0, abs(lhs))


# ---------------------------------------------------------------------------
# impulse sensitivity
# ---------------------------------------------------------------------------
def test_impulse_closed_forms():
    cfg = synth.make_impulse(B=1, D=6, N=16, L=3000, seed=2)
    dl = synth.widen(cfg["delta"])[0]
    A = synth.widen(cfg["A"])
    Bm = synth.widen(cfg["Bm"])[0]
    C = synth.widen(cfg["C"])[0]
    L = 3000
    s = oracle.impulse_sens(delta=cfg["delta"], A=cfg["A"], Bm=cfg["Bm"], C=cfg["C"], B=1, D=6, L=L, N=16)
    y, _ = oracle.real_fwd(delta=cfg["delta"], x=cfg["x"], A=cfg["A"], Bm=cfg["Bm"], C=cfg["C"],
                           B=1, D=6, L=L, N=16)
    for di in range(6):
        # suffix sums S_t = sum_{s=t+1}^{L-1} delta_s and prefix sums P_t = sum_{s=1}^{t} delta_s,
        # each rounded once (math.fsum), a different rounding path from any product loop
        S = np.array([math.fsum(dl[di, t + 1:]) for t in range(L)])
        P = np.array([math.fsum(dl[di, 1:t + 1]) for t in range(L)])
        want_s = dl[di] * (Bm * C[L - 1][None, :] * np.exp(A[di][None, :] * S[:, None])).sum(axis=1)
        want_y = dl[di, 0] * (C * Bm[0][None, :] * np.exp(A[di][None, :] * P[:, None])).sum(axis=1)
        close(s[0, di], want_s, rtol=1e-10, atol=1e-300)
        close(y[0, di], want_y, rtol=1e-10, atol=1e-300)


def test_impulse_linearity_and_backward():
    cfg = synth.make_impulse(B=2, D=3, N=8, L=400, seed=4, with_xrand=True)
    kw = dict(delta=cfg["delta"], A=cfg["A"], Bm=cfg["Bm"], C=cfg["C"], B=2, D=3, L=400, N=8)
    for t_out in (399, 150):
        s = oracle.impulse_sens(**kw, t_out=t_out)
        y, _ = oracle.real_fwd(x=cfg["x_rand"], **kw)
        lin = (s * synth.widen(cfg["x_rand"])).sum(axis=2)
        close(lin, y[:, :, t_out], rtol=1e-11, atol=1e-13)
        gy = np.zeros((2, 3, 400))
        gy[:, :, t_out] = 1.0
        g = oracle.real_bwd(x=cfg["x_rand"], gy=gy, **kw)
        close(g["gx"], s, rtol=1e-12, atol=1e-300)
        assert np.all(s[:, :, t_out + 1:] == 0.0)


@pytest.mark.parametrize("softplus", [True, False])
def test_step_size_pullback_fd(softplus):
    """Gradients w.r.t. the projection output z and the bias through delta = softplus(z + bias),
    by central differences of the forward loss; softplus of a known value; identity without softplus."""
    p = small_real(B=2, D=3, N=4, L=11, seed=23)
    g = np.random.default_rng(24)
    z = g.standard_normal((2, 3, 11)) * 2.0
    bias = g.standard_normal(3)
    kw = {k: p[k] for k in ("x", "A", "Bm", "C", "h0", "B", "D", "L", "N")}

    def loss(q, **over):
        zz = over.get("z", z)
        bb = over.get("bias", bias)
        y, hl = oracle.real_fwd(delta=oracle.step_sizes(zz, bb, softplus), **kw)
        return float((y * p["gy"]).sum() + (hl * p["ghlast"]).sum())
    dl = oracle.step_sizes(z, bias, softplus)
    gd = oracle.real_bwd(delta=dl, gy=p["gy"], ghlast=p["ghlast"], **kw)["gdelta"]
    gz, gb = oracle.step_size_grads(gd, z, bias, softplus)
    fd_check(loss, {"z": z, "bias": bias}, "z", gz)
    fd_check(loss, {"z": z, "bias": bias}, "bias", gb)
    if softplus:
        close(oracle.step_sizes(np.zeros((1, 1, 1)), None, True), np.full((1, 1, 1), math.log(2.0)), rtol=1e-15)
    else:
        close(oracle.step_sizes(z, None, False), z, rtol=0, atol=0)


@pytest.mark.parametrize("t_out", [16, 9, 0])
def test_output_sensitivity_delta_fd(t_out):
    """d y[t_out] / d delta_t by central differences of the forward (h0 and x nonzero)."""
    p = small_real(B=1, D=2, N=4, L=17, seed=21)
    kw = {k: p[k] for k in ("delta", "x", "A", "Bm", "C", "h0", "B", "D", "L", "N")}
    sx, sd = oracle.output_sens(**kw, t_out=t_out)

    def f(q, delta):
        y, _ = oracle.real_fwd(**dict(kw, delta=delta))
        return float(y[:, :, t_out].sum())
    fd_check(f, dict(p), "delta", sd, rtol=2e-6, atol=1e-9)
    assert np.all(sd[:, :, t_out + 1:] == 0.0) and np.all(sx[:, :, t_out + 1:] == 0.0)


def test_output_sensitivity_matches_backward():
    """Equal to the general backward's gdelta and gx at gy = e_{t_out}, and s_x to the impulse routine."""
    p = small_real(B=2, D=3, N=5, L=60, seed=22)
    kw = {k: p[k] for k in ("delta", "x", "A", "Bm", "C", "h0", "B", "D", "L", "N")}
    for t_out in (59, 31):
        sx, sd = oracle.output_sens(**kw, t_out=t_out)
        gy = np.zeros((2, 3, 60))
        gy[:, :, t_out] = 1.0
        g = oracle.real_bwd(**kw, gy=gy)
        close(sd, g["gdelta"], rtol=1e-12, atol=1e-14)
        close(sx, g["gx"], rtol=1e-12, atol=1e-14)
        si = oracle.impulse_sens(**{k: p[k] for k in ("delta", "A", "Bm", "C", "B", "D", "L", "N")}, t_out=t_out)
        close(sx, si, rtol=1e-13, atol=1e-300)


# ---------------------------------------------------------------------------
# complex scan
# ---------------------------------------------------------------------------
def small_complex(B=2, H=2, M=3, L=12, seed=0):
    g = np.random.default_rng(seed)
    return dict(r=np.log1p(np.exp(g.standard_normal((B, H, L)))), phi=g.standard_normal((B, H, L)),
                lam=g.uniform(0.9, 0.999, (H, M)), theta=g.uniform(0, np.pi, (H, M)),
                u=g.standard_normal((B, H, L, M)) + 1j * g.standard_normal((B, H, L, M)),
                c=g.standard_normal((H, M)) + 1j * g.standard_normal((H, M)),
                h0=g.standard_normal((B, H, M)) + 1j * g.standard_normal((B, H, M)),
                gy=g.standard_normal((B, H, L)),
                ghlast=g.standard_normal((B, H, M)) + 1j * g.standard_normal((B, H, M)),
                B=B, H=H, M=M, L=L)


def test_complex_fwd_matrix_route():
    """Each mode as a 2x2 real rotation-scaling matrix acting on (Re h, Im h)."""
    p = small_complex(B=2, H=2, M=3, L=40)
    y, hl = oracle.complex_fwd(**{k: p[k] for k in ("r", "phi", "lam", "theta", "u", "c", "h0")},
                               B=2, H=2, L=40, M=3)
    for bi in range(2):
        for hi in range(2):
            v = np.stack([p["h0"][bi, hi].real, p["h0"][bi, hi].imag], axis=1)  # (M,2)
            for t in range(40):
                acc = 0.0
                for m in range(3):
                    rho = p["lam"][hi, m] ** p["r"][bi, hi, t]
                    w = p["phi"][bi, hi, t] * p["theta"][hi, m]
                    R = rho * np.array([[np.cos(w), -np.sin(w)], [np.sin(w), np.cos(w)]])
                    v[m] = R @ v[m] + np.array([p["u"][bi, hi, t, m].real, p["u"][bi, hi, t, m].imag])
                    acc += p["c"][hi, m].real * v[m, 0] - p["c"][hi, m].imag * v[m, 1]
                assert abs(acc - y[bi, hi, t]) <= 1e-12 * max(1, abs(acc))
            close(hl[bi, hi], v[:, 0] + 1j * v[:, 1], rtol=1e-12, atol=1e-12)


def test_complex_geometric():
    B, H, M, L = 1, 1, 4, 200
    lam = np.array([[0.95, 0.99, 0.999, 0.9]])
    theta = np.array([[0.3, 1.0, 2.0, 3.0]])
    r = np.full((B, H, L), 0.7)
    phi = np.full((B, H, L), 1.3)
    uc = np.array([1 + 2j, -0.5j, 0.25, 3 - 1j])
    u = np.broadcast_to(uc, (B, H, L, M)).copy()
    h0 = np.array([[[0.5 - 0.5j, 1j, -1, 2]]])
    c = np.ones((H, M), dtype=complex)
    _, hl = oracle.complex_fwd(r=r, phi=phi, lam=lam, theta=theta, u=u, c=c, h0=h0, B=B, H=H, L=L, M=M)
    a = np.exp(0.7 * np.log(lam[0]) + 1j * 1.3 * theta[0])
    want = a ** L * h0[0, 0] + uc * (1 - a ** L) / (1 - a)
    close(hl[0, 0], want, rtol=1e-12, atol=1e-12)


def test_complex_reduces_to_real():
    """theta = 0 with real u, c, h0 is the real dense scan with a = lam^r."""
    p = small_complex(B=2, H=3, M=4, L=30, seed=9)
    theta = np.zeros_like(p["theta"])
    u = p["u"].real + 0j
    c = p["c"].real + 0j
    h0 = p["h0"].real + 0j
    y, hl = oracle.complex_fwd(r=p["r"], phi=p["phi"], lam=p["lam"], theta=theta, u=u, c=c, h0=h0,
                               B=2, H=3, L=30, M=4)
    B, H, L, M = 2, 3, 30, 4
    a = (p["lam"][None, :, None, :] ** p["r"][:, :, :, None]).reshape(B * H, 1, L, M)
    C = np.broadcast_to(c.real[None, :, None, :], (B, H, L, M)).reshape(B * H, L, M)
    yr, hr = oracle.real_fwd(a=a, b=u.real.reshape(B * H, 1, L, M), C=C, h0=h0.real.reshape(B * H, 1, M),
                             B=B * H, D=1, L=L, N=M)
    close(y, yr.reshape(B, H, L), rtol=1e-12, atol=1e-12)
    close(hl.real, hr.reshape(B, H, M), rtol=1e-12, atol=1e-12)
    assert np.all(hl.imag == 0)


def test_complex_modulus_invariant():
    p = small_complex(B=1, H=2, M=5, L=500, seed=10)
    r = np.zeros_like(p["r"])
    u = np.zeros_like(p["u"])
    _, hl = oracle.complex_fwd(r=r, phi=p["phi"], lam=p["lam"], theta=p["theta"], u=u, c=p["c"],
                               h0=p["h0"], B=1, H=2, L=500, M=5)
    close(np.abs(hl), np.abs(p["h0"]), rtol=1e-12, atol=1e-14)


def _loss_complex(p, **over):
    q = dict(p)
    q.update(over)
    kw = {k: q[k] for k in ("r", "phi", "lam", "theta", "c", "h0")}
    u = q["u_re"] + 1j * q["u_im"]
    y, hl = oracle.complex_fwd(u=u, **kw, B=q["B"], H=q["H"], L=q["L"], M=q["M"])
    return float((y * q["gy"]).sum() + (hl.real * q["ghlast"].real).sum() + (hl.imag * q["ghlast"].imag).sum())


@pytest.mark.parametrize("name", ["r", "phi", "lam", "theta", "u_re", "u_im", "c_re", "c_im",
                                  "h0_re", "h0_im"])
def test_complex_bwd_fd(name):
    p = small_complex(B=2, H=2, M=3, L=10, seed=12)
    g = oracle.complex_bwd(**{k: p[k] for k in ("r", "phi", "lam", "theta", "u", "c", "h0", "gy", "ghlast")},
                           B=2, H=2, L=10, M=3)
    p["u_re"], p["u_im"] = p["u"].real.copy(), p["u"].imag.copy()
    base, part = (name.split("_") + [None])[:2]
    if part is None:
        fd_check(_loss_complex, p, name, g["g" + name], rtol=5e-6)
        return
    grad = getattr(g["g" + base], "real" if part == "re" else "imag")
    if base == "u":
        fd_check(_loss_complex, p, name, grad, rtol=5e-6)
        return

    def loss(q, **over):
        key = list(over)[0]
        arr = over[key]
        other = q[base].imag if part == "re" else q[base].real
        z = arr + 1j * other if part == "re" else other + 1j * arr
        return _loss_complex(q, **{base: z})

    q = dict(p)
    q[name] = getattr(p[base], "real" if part == "re" else "imag").copy()
    fd_check(loss, q, name, grad, rtol=5e-6)


def test_complex_adjoint_identity():
    p = small_complex(B=2, H=2, M=4, L=50, seed=13)
    kw = {k: p[k] for k in ("r", "phi", "lam", "theta", "u", "c", "h0")}
    y, hl = oracle.complex_fwd(**kw, B=2, H=2, L=50, M=4)
    g = oracle.complex_bwd(**kw, gy=p["gy"], ghlast=p["ghlast"], B=2, H=2, L=50, M=4)

    def rp(a, b):
        return (a.real * b.real + a.imag * b.imag).sum()

    lhs = (y * p["gy"]).sum() + rp(hl, p["ghlast"])
    rhs = rp(g["gu"], p["u"]) + rp(g["gh0"], p["h0"])
    assert abs(lhs - rhs) <= 1e-11 * max(1.0, abs(lhs))


def _dense_complex(B=2, H=2, M=3, L=10, seed=14):
    g = np.random.default_rng(seed)
    rho = g.uniform(0.8, 0.999, (B, H, L, M))
    ang = g.uniform(-np.pi, np.pi, (B, H, L, M))
    return dict(a=rho * np.exp(1j * ang),
                u=g.standard_normal((B, H, L, M)) + 1j * g.standard_normal((B, H, L, M)),
                c=g.standard_normal((H, M)) + 1j * g.standard_normal((H, M)),
                h0=g.standard_normal((B, H, M)) + 1j * g.standard_normal((B, H, M)),
                gy=g.standard_normal((B, H, L)),
                ghlast=g.standard_normal((B, H, M)) + 1j * g.standard_normal((B, H, M)), B=B, H=H, L=L, M=M)


def test_complex_dense_matches_shared_controls():
    """Given transitions a = lam^r e^{i phi theta} (formed in numpy) reproduce the shared-control oracle:
    y, h_last, gu, gc, gh0."""
    p = small_complex(B=2, H=3, M=4, L=60, seed=15)
    a = (p["lam"][None, :, None, :] ** p["r"][:, :, :, None]) * \
        np.exp(1j * p["phi"][:, :, :, None] * p["theta"][None, :, None, :])
    kw = dict(u=p["u"], c=p["c"], h0=p["h0"], B=2, H=3, L=60, M=4)
    y, hl = oracle.complex_dense_fwd(a=a, **kw)
    ys, hs = oracle.complex_fwd(r=p["r"], phi=p["phi"], lam=p["lam"], theta=p["theta"], **kw)
    close(y, ys, rtol=1e-12, atol=1e-12)
    close(hl, hs, rtol=1e-12, atol=1e-12)
    g = oracle.complex_dense_bwd(a=a, gy=p["gy"], ghlast=p["ghlast"], **kw)
    gs = oracle.complex_bwd(r=p["r"], phi=p["phi"], lam=p["lam"], theta=p["theta"], gy=p["gy"],
                            ghlast=p["ghlast"], **kw)
    for k in ("gu", "gc", "gh0"):
        close(g[k], gs[k], rtol=1e-11, atol=1e-11)


def test_complex_dense_geometric():
    """Constant a per mode: h_L = a^L h0 + u (1 - a^L) / (1 - a) for a constant u."""
    B, H, M, L = 1, 1, 3, 150
    ac = np.array([0.97 * np.exp(0.4j), 0.5 - 0.6j, 0.999j])
    uc = np.array([1 - 1j, 2.0, -0.5j])
    h0 = np.array([[[0.3, -1j, 1 + 1j]]])
    _, hl = oracle.complex_dense_fwd(a=np.broadcast_to(ac, (B, H, L, M)).copy(),
                                     u=np.broadcast_to(uc, (B, H, L, M)).copy(), c=np.ones((H, M), complex),
                                     h0=h0, B=B, H=H, L=L, M=M)
    close(hl[0, 0], ac ** L * h0[0, 0] + uc * (1 - ac ** L) / (1 - ac), rtol=1e-12, atol=1e-12)


def _loss_dense_complex(q, **over):
    r = dict(q)
    r.update(over)
    z = {k: r[k + "_re"] + 1j * r[k + "_im"] for k in ("a", "u", "c", "h0")}
    y, hl = oracle.complex_dense_fwd(**z, B=r["B"], H=r["H"], L=r["L"], M=r["M"])
    return float((y * r["gy"]).sum() + (hl.real * r["ghlast"].real).sum() + (hl.imag * r["ghlast"].imag).sum())


@pytest.mark.parametrize("name", ["a_re", "a_im", "u_re", "u_im", "c_re", "c_im", "h0_re", "h0_im"])
def test_complex_dense_bwd_fd(name):
    """Central differences of the loss in the real and imaginary parts of every input: the gradient of a real
    loss w.r.t. z = x + iy is dL/dx + i dL/dy."""
    p = _dense_complex()
    g = oracle.complex_dense_bwd(**{k: p[k] for k in ("a", "u", "c", "h0", "gy", "ghlast")},
                                 B=p["B"], H=p["H"], L=p["L"], M=p["M"])
    q = dict(p)
    for k in ("a", "u", "c", "h0"):
        q[k + "_re"], q[k + "_im"] = p[k].real.copy(), p[k].imag.copy()
    base, part = name.split("_")
    grad = getattr(g["g" + base], "real" if part == "re" else "imag")
    fd_check(_loss_dense_complex, q, name, grad, rtol=5e-6)


@pytest.mark.parametrize("name", ["lam", "theta"])
def test_complex_rtrl_fd(name):
    """Forward-mode (RTRL) parameter gradients against central differences of the forward scan."""
    p = small_complex(B=2, H=2, M=3, L=10, seed=14)
    g = oracle.complex_rtrl(**{k: p[k] for k in ("r", "phi", "lam", "theta", "u", "c", "h0", "gy", "ghlast")},
                            B=2, H=2, L=10, M=3)
    p["u_re"], p["u_im"] = p["u"].real.copy(), p["u"].imag.copy()
    fd_check(_loss_complex, p, name, g["g" + name], rtol=5e-6)


def test_complex_rtrl_equals_bptt():
    """Forward-mode gradients equal the reverse-mode (adjoint) ones of the same loss; y equals the forward scan."""
    p = small_complex(B=3, H=2, M=5, L=120, seed=15)
    kw = {k: p[k] for k in ("r", "phi", "lam", "theta", "u", "c", "h0")}
    rt = oracle.complex_rtrl(**kw, gy=p["gy"], ghlast=p["ghlast"], B=3, H=2, L=120, M=5)
    bw = oracle.complex_bwd(**kw, gy=p["gy"], ghlast=p["ghlast"], B=3, H=2, L=120, M=5)
    y, _ = oracle.complex_fwd(**kw, B=3, H=2, L=120, M=5)
    close(rt["glam"], bw["glam"], rtol=1e-11, atol=1e-12)
    close(rt["gtheta"], bw["gtheta"], rtol=1e-11, atol=1e-12)
    close(rt["y"], y, rtol=1e-14, atol=1e-14)


# ---------------------------------------------------------------------------
# PD scan
# ---------------------------------------------------------------------------
def test_pd_select_bruteforce_with_ties():
    g = np.random.default_rng(3)
    logits = g.integers(-2, 3, (2, 3, 50, 8)).astype(np.float32)  # many exact ties
    sel = oracle.pd_select(logits)
    want = np.argmax(logits, axis=-1)  # numpy returns the first maximum
    assert np.array_equal(sel, want)


def test_pd_dfa_exact():
    """Config-shaped dictionary read as an automaton: d=1, b=0, h0=e_q0 gives h_t = e_{q_t}."""
    cfg = synth.make_pd(B=2, H=4, N=16, L=600, K=8, seed=5)
    B, H, N, L, K = 2, 4, 16, 600, 8
    sel = oracle.pd_select(cfg["logits"])
    dct = cfg["dict"]
    q0 = np.array([[3, 0, 15, 7], [1, 2, 9, 11]])
    h0 = np.zeros((B, H, N))
    for bi in range(B):
        for hi in range(H):
            h0[bi, hi, q0[bi, hi]] = 1.0
    C = np.broadcast_to(2.0 ** np.arange(N), (B, H, L, N)).copy()
    y, hl = oracle.pd_fwd(sel=sel, dict=dct, d=np.ones((B, H, L, N)), b=np.zeros((B, H, L, N)), C=C,
                          h0=h0, B=B, H=H, L=L, N=N, K=K)
    for bi in range(B):
        for hi in range(H):
            q = q0[bi, hi]
            for t in range(L):
                q = dct[hi, sel[bi, hi, t], q]
                assert y[bi, hi, t] == 2.0 ** q
            assert np.array_equal(hl[bi, hi], np.eye(N)[q])


def test_pd_golden_mod3():
    g = json.load(open(os.path.join(GOLD, "pd_mod3_counter.json")))
    N, K = g["N"], g["K"]
    sym = np.array(g["symbols"])
    L = len(sym)
    logits = np.zeros((1, 1, L, K), dtype=np.float32)
    logits[0, 0, np.arange(L), sym] = 1.0
    sel = oracle.pd_select(logits)
    h0 = np.zeros((1, 1, N))
    h0[0, 0, 0] = 1
    C = np.broadcast_to(np.array([1.0, 2.0, 4.0]), (1, 1, L, N)).copy()
    y, hl = oracle.pd_fwd(sel=sel, dict=np.array([g["dict"]], dtype=np.int32), d=np.ones((1, 1, L, N)),
                          b=np.zeros((1, 1, L, N)), C=C, h0=h0, B=1, H=1, L=L, N=N, K=K)
    assert y.ravel().tolist() == g["y"]
    assert hl.ravel().tolist() == np.eye(N)[g["states"][-1]].tolist()


def test_pd_dense_matrix_route():
    cfg = synth.make_pd(B=2, H=3, N=16, L=200, K=8, seed=6)
    B, H, N, L, K = 2, 3, 16, 200, 8
    sel = oracle.pd_select(cfg["logits"])
    h0 = RNG.standard_normal((B, H, N))
    kw = dict(sel=sel, dict=cfg["dict"], d=cfg["d"], b=cfg["b"], C=cfg["C"], h0=h0, B=B, H=H, L=L, N=N, K=K)
    y, hl = oracle.pd_fwd(**kw)
    y2, hl2 = oracle.pd_fwd(**kw, dense=True)
    close(y, y2, rtol=1e-13, atol=1e-13)
    # numpy dense products, written here independently of oracle.c
    d = synth.widen(cfg["d"])
    b = synth.widen(cfg["b"])
    C = synth.widen(cfg["C"])
    for bi in range(B):
        for hi in range(H):
            h = h0[bi, hi].copy()
            for t in range(L):
                P = np.zeros((N, N))
                P[cfg["dict"][hi, sel[bi, hi, t]], np.arange(N)] = 1.0
                h = P @ np.diag(d[bi, hi, t]) @ h + b[bi, hi, t]
                assert abs(C[bi, hi, t] @ h - y[bi, hi, t]) <= 1e-12 * max(1, abs(y[bi, hi, t]))
            close(hl[bi, hi], h, rtol=1e-12, atol=1e-12)


def test_pd_gather_composition_is_dense_product():
    """(P2 D2)(P1 D1) = P_{pi2[pi1]} diag(D2[pi1] * D1): closure of PD matrices, bit-exact."""
    g = np.random.default_rng(8)
    N = 16
    for _ in range(50):
        p1, p2 = g.integers(0, N, N), g.integers(0, N, N)
        d1, d2 = g.standard_normal(N), g.standard_normal(N)
        M1 = np.zeros((N, N))
        M1[p1, np.arange(N)] = d1
        M2 = np.zeros((N, N))
        M2[p2, np.arange(N)] = d2
        dense = M2 @ M1
        pc = p2[p1]
        dc = d2[p1] * d1
        comp = np.zeros((N, N))
        comp[pc, np.arange(N)] = dc
        assert np.array_equal(dense, comp)


def test_pd_column_sum_invariant():
    cfg = synth.make_pd(B=1, H=2, N=16, L=300, K=8, seed=7)
    sel = oracle.pd_select(cfg["logits"])
    h0 = RNG.standard_normal((1, 2, 16))
    y, _ = oracle.pd_fwd(sel=sel, dict=cfg["dict"], d=np.ones((1, 2, 300, 16)), b=np.zeros((1, 2, 300, 16)),
                         C=np.ones((1, 2, 300, 16)), h0=h0, B=1, H=2, L=300, N=16, K=8)
    close(y, np.broadcast_to(h0.sum(axis=2)[:, :, None], y.shape), rtol=1e-13, atol=1e-13)


def test_pd_reduces_to_real():
    """K = 1 with the identity selector is the diagonal real scan with a = d."""
    cfg = synth.make_pd(B=2, H=2, N=16, L=100, K=1, seed=9)
    dct = np.broadcast_to(np.arange(16, dtype=np.int32), (2, 1, 16)).copy()
    sel = np.zeros((2, 2, 100), dtype=np.int32)
    y, hl = oracle.pd_fwd(sel=sel, dict=dct, d=cfg["d"], b=cfg["b"], C=cfg["C"], B=2, H=2, L=100, N=16, K=1)
    # the real scan takes C per (batch, t): map each (b,h) to its own batch row
    yr, hr = oracle.real_fwd(a=cfg["d"].reshape(4, 1, 100, 16), b=cfg["b"].reshape(4, 1, 100, 16),
                             C=cfg["C"].reshape(4, 100, 16), B=4, D=1, L=100, N=16)
    close(y, yr.reshape(2, 2, 100), rtol=1e-13, atol=1e-14)
    close(hl, hr.reshape(2, 2, 16), rtol=1e-13, atol=1e-14)


def _pd_small(seed=14):
    cfg = synth.make_pd(B=1, H=2, N=5, L=7, K=3, seed=seed)
    g = np.random.default_rng(seed)
    return dict(sel=oracle.pd_select(cfg["logits"]), dict=cfg["dict"], d=synth.widen(cfg["d"]),
                b=synth.widen(cfg["b"]), C=synth.widen(cfg["C"]), h0=g.standard_normal((1, 2, 5)),
                gy=g.standard_normal((1, 2, 7)), ghlast=g.standard_normal((1, 2, 5)),
                B=1, H=2, L=7, N=5, K=3)


def _loss_pd(p, **over):
    q = dict(p)
    q.update(over)
    y, hl = oracle.pd_fwd(**{k: q[k] for k in ("sel", "dict", "d", "b", "C", "h0", "B", "H", "L", "N", "K")})
    return float((y * q["gy"]).sum() + (hl * q["ghlast"]).sum())


@pytest.mark.parametrize("name,gname", [("d", "gd"), ("b", "gb"), ("C", "gC"), ("h0", "gh0")])
def test_pd_bwd_fd(name, gname):
    p = _pd_small()
    g = oracle.pd_bwd(**{k: p[k] for k in ("sel", "dict", "d", "b", "C", "h0", "gy", "ghlast",
                                            "B", "H", "L", "N", "K")})
    fd_check(_loss_pd, p, name, g[gname])


def _pd_ste_small(seed=15):
    cfg = synth.make_pd(B=1, H=2, N=5, L=7, K=3, seed=seed)
    g = np.random.default_rng(seed)
    return dict(logits=synth.widen(cfg["logits"]), sel=oracle.pd_select(cfg["logits"]), dict=cfg["dict"],
                d=synth.widen(cfg["d"]), b=synth.widen(cfg["b"]), C=synth.widen(cfg["C"]),
                h0=g.standard_normal((1, 2, 5)), gy=g.standard_normal((1, 2, 7)),
                ghlast=g.standard_normal((1, 2, 5)), B=1, H=2, L=7, N=5, K=3)


def _onehot(sel, K):
    return (sel[..., None] == np.arange(K)).astype(np.float64)


def _ste(p, tau):
    return oracle.pd_ste(**{k: p[k] for k in ("logits", "sel", "dict", "d", "b", "C", "h0", "gy", "ghlast",
                                              "B", "H", "L", "N", "K")}, tau=tau)


def _loss_mix(p, w):
    y, hl = oracle.pd_mix_fwd(w=w, **{k: p[k] for k in ("dict", "d", "b", "C", "h0", "B", "H", "L", "N", "K")})
    return float((y * p["gy"]).sum() + (hl * p["ghlast"]).sum())


def test_pd_mixture_at_onehot_is_hard_forward():
    """The mixture transition with one-hot weights is the PD forward (gather route vs dense matrices)."""
    p = _pd_ste_small()
    y, hl = oracle.pd_mix_fwd(w=_onehot(p["sel"], 3), **{k: p[k] for k in ("dict", "d", "b", "C", "h0",
                                                                            "B", "H", "L", "N", "K")})
    y2, hl2 = oracle.pd_fwd(**{k: p[k] for k in ("sel", "dict", "d", "b", "C", "h0", "B", "H", "L", "N", "K")})
    close(y, y2, rtol=1e-13, atol=1e-14)
    close(hl, hl2, rtol=1e-13, atol=1e-14)


def test_pd_ste_selection_weight_gradient_fd():
    """gw = dLoss/dw of the dense mixture forward at the one-hot selection, by central differences
    (the loss is affine in each single weight, so the difference quotient is exact up to rounding)."""
    p = _pd_ste_small()
    gw = _ste(p, 0.7)["gw"]
    w0 = _onehot(p["sel"], 3)
    q = dict(p, w=w0)
    fd_check(lambda q_, w: _loss_mix(q_, w), q, "w", gw, rtol=1e-8, atol=1e-10)


@pytest.mark.parametrize("tau", [0.25, 1.0, 3.0])
def test_pd_ste_logit_gradient_fd(tau):
    """glogits = d/dlogits of sum_k gw_k softmax(logits/tau)_k with gw held fixed (finite differences)."""
    p = _pd_ste_small(seed=16)
    r = _ste(p, tau)
    gw = r["gw"]

    def f(q, logits):
        z = logits / tau
        e = np.exp(z - z.max(axis=-1, keepdims=True))
        return float((gw * e / e.sum(axis=-1, keepdims=True)).sum())
    fd_check(f, dict(p), "logits", r["glogits"], rtol=1e-6, atol=1e-10)


def test_pd_ste_uniform_limit():
    """Large tau: softmax -> uniform, so tau * glogits -> (gw - mean_k gw) / K."""
    p = _pd_ste_small(seed=17)
    tau = 1e7
    r = _ste(p, tau)
    want = (r["gw"] - r["gw"].mean(axis=-1, keepdims=True)) / 3
    close(r["glogits"] * tau, want, rtol=1e-5, atol=1e-9)


# ---------------------------------------------------------------------------
# generators
# ---------------------------------------------------------------------------
def test_generators_reproducible_and_rounded():
    a = synth.make_real(B=1, D=4, N=16, L=64, dtype="bf16", seed=0)
    b = synth.make_real(B=1, D=4, N=16, L=64, dtype="bf16", seed=0)
    for k in ("x", "delta", "Bm", "C", "gy", "A"):
        assert a[k].tobytes() == b[k].tobytes()
    assert a["x"].dtype == np.uint16 and a["A"].dtype == np.float32
    # bf16 round-to-nearest-even on float32 bits
    v = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e-3], dtype=np.float32)
    bits = synth.f32_to_bf16_bits(v)
    back = synth.bf16_bits_to_f32(bits)
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == 1.015625 and back[3] == -2.5
    assert abs(back[4] - 3.0e-3) <= 2 ** -8 * 3.0e-3
    c = synth.make_real(B=1, D=64, N=16, L=512, seed=0)
    dl = synth.widen(c["delta"])
    assert np.all(dl > 0)
    A = synth.widen(c["A"])
    assert np.all((A <= -np.exp(-3.0) * (1 - 1e-6)) & (A >= -np.exp(-1.0) * (1 + 1e-6)))
    assert abs(synth.widen(c["x"]).mean()) < 0.05 and abs(synth.widen(c["x"]).std() - 1) < 0.05


# ---------------------------------------------------------------------------
# general selective form: zero-order hold and per-channel B_t, C_t
# ---------------------------------------------------------------------------
def _sel_kw(p, disc=0, perd=False):
    return dict(delta=p["delta"], x=p["x"], A=p["A"], Bm=p["Bm"], C=p["C"], h0=p["h0"], disc=disc, perd=perd,
                B=p["B"], D=p["D"], L=p["L"], N=p["N"])


def _perd(p, seed):
    """The same problem with B_t, C_t drawn per channel (B,D,L,N)."""
    g = np.random.default_rng(seed)
    q = dict(p)
    q["Bm"] = g.standard_normal((p["B"], p["D"], p["L"], p["N"])) / 2
    q["C"] = g.standard_normal((p["B"], p["D"], p["L"], p["N"])) / 2
    return q


def test_general_euler_equals_real_scan():
    """The general routine in its Euler, shared-B/C form is the selective scan (forward and backward)."""
    p = small_real(B=2, D=3, N=4, L=30, seed=41)
    y, hl = oracle.sel_fwd(**_sel_kw(p))
    y0, hl0 = oracle.real_fwd(delta=p["delta"], x=p["x"], A=p["A"], Bm=p["Bm"], C=p["C"], h0=p["h0"],
                              B=2, D=3, L=30, N=4)
    close(y, y0, rtol=1e-13)
    close(hl, hl0, rtol=1e-13)
    g = oracle.sel_bwd(**_sel_kw(p), gy=p["gy"], ghlast=p["ghlast"])
    g0 = oracle.real_bwd(delta=p["delta"], x=p["x"], A=p["A"], Bm=p["Bm"], C=p["C"], h0=p["h0"], gy=p["gy"],
                         ghlast=p["ghlast"], B=2, D=3, L=30, N=4)
    for k in ("gdelta", "gx", "gA", "gBm", "gC", "gh0"):
        close(g[k], g0[k], rtol=1e-11, atol=1e-13)


def test_zoh_is_the_exact_ode_solution_for_held_inputs():
    """With delta, x and B held constant, the zero-order-hold scan samples the exact solution of
    dh/dt = A h + B x at t = (k+1) delta: h_k = e^{A (k+1) delta} h0 + (e^{A (k+1) delta} - 1) / A B x
    (a closed form computed here, not a recurrence)."""
    B, D, N, L = 1, 2, 3, 40
    g = np.random.default_rng(42)
    dl = np.array([0.3, 1.7])
    xv = np.array([0.8, -1.3])
    A = -np.exp(g.uniform(-3, 1, (D, N)))
    Bv = g.standard_normal(N)
    Cv = g.standard_normal(N)
    h0 = g.standard_normal((B, D, N))
    p = dict(delta=np.broadcast_to(dl[None, :, None], (B, D, L)).copy(),
             x=np.broadcast_to(xv[None, :, None], (B, D, L)).copy(), A=A,
             Bm=np.broadcast_to(Bv, (B, L, N)).copy(), C=np.broadcast_to(Cv, (B, L, N)).copy(), h0=h0,
             B=B, D=D, N=N, L=L)
    y, hl = oracle.sel_fwd(**_sel_kw(p, disc=1))
    T = (np.arange(L) + 1.0)[:, None]
    for d in range(D):
        e = np.exp(A[d][None, :] * T * dl[d])
        H = e * h0[0, d][None, :] + (e - 1.0) / A[d][None, :] * Bv[None, :] * xv[d]
        close(y[0, d], H @ Cv, rtol=1e-11, atol=1e-13)
        close(hl[0, d], H[-1], rtol=1e-11, atol=1e-13)


def test_zoh_at_zero_A_is_the_euler_scan():
    """A = 0: the zero-order-hold input term is delta x B (its limit), so both discretisations agree."""
    p = small_real(B=2, D=2, N=3, L=25, seed=43)
    p["A"] = np.zeros_like(p["A"])
    y1, h1 = oracle.sel_fwd(**_sel_kw(p, disc=1))
    y0, h0 = oracle.real_fwd(delta=p["delta"], x=p["x"], A=p["A"], Bm=p["Bm"], C=p["C"], h0=p["h0"],
                             B=2, D=2, L=25, N=3)
    close(y1, y0, rtol=1e-14)
    close(h1, h0, rtol=1e-14)


def test_zoh_input_term_bruteforce():
    """Every state by the unrolled O(L^2) sum with b_s = expm1(delta A) / A x B, a written out per step."""
    p = small_real(B=1, D=2, N=3, L=18, seed=44)
    y, _ = oracle.sel_fwd(**_sel_kw(p, disc=1))
    for di in range(2):
        z = p["delta"][0, di][:, None] * p["A"][di][None, :]
        a = np.exp(z)
        bb = np.expm1(z) / p["A"][di][None, :] * (p["x"][0, di][:, None] * p["Bm"][0])
        yb, _ = brute_real(a, bb, p["C"][0], p["h0"][0, di])
        close(y[0, di], yb, rtol=1e-12, atol=1e-14)


def _loss_sel(p, disc, perd, **over):
    q = dict(p)
    q.update(over)
    y, hl = oracle.sel_fwd(**_sel_kw(q, disc=disc, perd=perd))
    return float((y * q["gy"]).sum() + (hl * q["ghlast"]).sum())


@pytest.mark.parametrize("name,gname", [("delta", "gdelta"), ("x", "gx"), ("A", "gA"), ("Bm", "gBm"),
                                        ("C", "gC"), ("h0", "gh0")])
@pytest.mark.parametrize("disc,perd", [(1, False), (0, True), (1, True)])
def test_general_selective_bwd_fd(name, gname, disc, perd):
    """Central differences of the general forward in every input entry (ZOH and / or per-channel B_t, C_t;
    one A entry set to 0 and one tiny, so the A = 0 limit and the series branch of d coef / d A are
    covered)."""
    p = small_real(B=2, D=2, N=3, L=9, seed=45)
    p["A"][0, 1] = 0.0
    p["A"][1, 2] = -3e-5
    if perd:
        p = _perd(p, 46)
    g = oracle.sel_bwd(**_sel_kw(p, disc=disc, perd=perd), gy=p["gy"], ghlast=p["ghlast"])
    fd_check(lambda q, **o: _loss_sel(q, disc, perd, **o), p, name, g[gname])


def test_perd_bruteforce():
    """Per-channel B_t, C_t: every output by the unrolled O(L^2) sum on that channel's own B, C."""
    p = _perd(small_real(B=2, D=3, N=3, L=16, seed=47), 48)
    y, _ = oracle.sel_fwd(**_sel_kw(p, perd=True))
    for bi in range(2):
        for di in range(3):
            a = np.exp(p["delta"][bi, di][:, None] * p["A"][di][None, :])
            bb = (p["delta"][bi, di] * p["x"][bi, di])[:, None] * p["Bm"][bi, di]
            yb, _ = brute_real(a, bb, p["C"][bi, di], p["h0"][bi, di])
            close(y[bi, di], yb, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("disc", [0, 1])
def test_perd_with_channel_independent_BC_equals_shared(disc):
    """B_t, C_t repeated over the channels: the per-channel form gives the shared form's y, and its per-channel
    gB, gC summed over the channels give the shared form's sums."""
    p = small_real(B=2, D=3, N=4, L=21, seed=49)
    q = dict(p)
    q["Bm"] = np.repeat(p["Bm"][:, None], 3, axis=1)
    q["C"] = np.repeat(p["C"][:, None], 3, axis=1)
    y, hl = oracle.sel_fwd(**_sel_kw(p, disc=disc))
    yq, hq = oracle.sel_fwd(**_sel_kw(q, disc=disc, perd=True))
    close(yq, y, rtol=1e-13)
    g = oracle.sel_bwd(**_sel_kw(p, disc=disc), gy=p["gy"], ghlast=p["ghlast"])
    gq = oracle.sel_bwd(**_sel_kw(q, disc=disc, perd=True), gy=p["gy"], ghlast=p["ghlast"])
    close(gq["gBm"].sum(axis=1), g["gBm"], rtol=1e-11, atol=1e-13)
    close(gq["gC"].sum(axis=1), g["gC"], rtol=1e-11, atol=1e-13)
    for k in ("gdelta", "gx", "gA", "gh0"):
        close(gq[k], g[k], rtol=1e-11, atol=1e-13)


# ---------------------------------------------------------------------------
# scalar transition per head (the chunked-matrix form's problem)
# ---------------------------------------------------------------------------
def small_head(B=2, H=2, P=3, N=4, L=20, seed=0):
    g = np.random.default_rng(seed)
    return dict(delta=np.log1p(np.exp(g.standard_normal((B, H, L)))), x=g.standard_normal((B, H * P, L)),
                A=-np.exp(g.uniform(-3, 0, H)), Bm=g.standard_normal((B, L, N)) / 2, C=g.standard_normal((B, L, N)) / 2,
                h0=g.standard_normal((B, H * P, N)), gy=g.standard_normal((B, H * P, L)),
                ghlast=g.standard_normal((B, H * P, N)), B=B, H=H, P=P, N=N, L=L)


def _head_kw(p):
    return {k: p[k] for k in ("delta", "x", "A", "Bm", "C", "h0", "B", "H", "P", "L", "N")}


def test_head_quadratic_form():
    """y = (L o C B^T) (delta x) + decayed h0: the masked-matrix (quadratic) form of the scan written out with
    numpy matrix products, Lmat[t, s] = exp(A (S_t - S_s)) for s <= t with S the prefix sums of delta."""
    p = small_head(B=2, H=2, P=3, N=4, L=24, seed=61)
    y, _ = oracle.head_fwd(**_head_kw(p))
    for b in range(2):
        G = p["C"][b] @ p["Bm"][b].T                       # (L, L): C_t . B_s
        for h in range(2):
            S = np.cumsum(p["delta"][b, h])
            Lm = np.tril(np.exp(p["A"][h] * (S[:, None] - S[None, :])))
            for q in range(3):
                d = h * 3 + q
                u = p["delta"][b, h] * p["x"][b, d]
                ref = (Lm * G) @ u + (p["C"][b] @ p["h0"][b, d]) * np.exp(p["A"][h] * S)
                close(y[b, d], ref, rtol=1e-11, atol=1e-13)


def test_head_equals_diagonal_scan():
    """The scalar-per-head scan is the diagonal selective scan with delta repeated over the head's channels
    and A[d, n] = A[h] for every state: forward, and the backward with gdelta / gA summed over the head."""
    p = small_head(B=2, H=3, P=2, N=4, L=30, seed=62)
    H, P = 3, 2
    dexp = np.repeat(p["delta"], P, axis=1)
    Aexp = np.repeat(p["A"], P)[:, None] * np.ones((1, 4))
    kw = dict(delta=dexp, x=p["x"], A=Aexp, Bm=p["Bm"], C=p["C"], h0=p["h0"], B=2, D=H * P, L=30, N=4)
    y0, hl0 = oracle.real_fwd(**kw)
    y, hl = oracle.head_fwd(**_head_kw(p))
    close(y, y0, rtol=1e-12)
    close(hl, hl0, rtol=1e-12)
    g0 = oracle.real_bwd(**kw, gy=p["gy"], ghlast=p["ghlast"])
    g = oracle.head_bwd(**_head_kw(p), gy=p["gy"], ghlast=p["ghlast"])
    close(g["gdelta"], g0["gdelta"].reshape(2, H, P, 30).sum(axis=2), rtol=1e-11, atol=1e-13)
    close(g["gA"], g0["gA"].reshape(H, P * 4).sum(axis=1), rtol=1e-11, atol=1e-13)
    for k in ("gx", "gBm", "gC", "gh0"):
        close(g[k], g0[k], rtol=1e-11, atol=1e-13)


def _loss_head(p, **over):
    q = dict(p)
    q.update(over)
    y, hl = oracle.head_fwd(**_head_kw(q))
    return float((y * q["gy"]).sum() + (hl * q["ghlast"]).sum())


@pytest.mark.parametrize("name,gname", [("delta", "gdelta"), ("x", "gx"), ("A", "gA"), ("Bm", "gBm"),
                                        ("C", "gC"), ("h0", "gh0")])
def test_head_bwd_fd(name, gname):
    p = small_head(B=2, H=2, P=2, N=3, L=9, seed=63)
    g = oracle.head_bwd(**_head_kw(p), gy=p["gy"], ghlast=p["ghlast"])
    fd_check(_loss_head, p, name, g[gname])
