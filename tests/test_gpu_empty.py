"""Empty problems (no batch rows, channels, heads or steps) on the GPU: the calls
succeed, h_last is h0, gh0 is gh_last, parameter gradients are zero, and
outputs with no elements keep their (empty) shapes."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _ssm():
    import selective_state_space_chunked_amd as ssm
    return ssm


def _r(*shape, dtype=torch.float32, seed=0):
    g = torch.Generator().manual_seed(seed)
    if dtype == torch.complex64:
        return torch.complex(torch.randn(*shape, generator=g), torch.randn(*shape, generator=g)).to(DEV)
    return torch.randn(*shape, generator=g).to(DEV)


@pytest.mark.parametrize("B,D,L", [(2, 3, 0), (0, 3, 50), (2, 0, 50)])
def test_empty_selective(B, D, L):
    ssm = _ssm()
    N = 16
    t = dict(delta=_r(B, D, L).abs(), x=_r(B, D, L), A=-_r(D, N).abs(), Bm=_r(B, L, N), C=_r(B, L, N),
             h0=_r(B, D, N, seed=1))
    f = ssm.scan_fwd(ssm.SSM_REAL_SELECTIVE, want_h_last=True, want_ckpt=True, **t)
    ghl = _r(B, D, N, seed=2)
    want = ("gdelta", "gx", "gA", "gBm", "gC", "gh0")
    g = ssm.scan_bwd(ssm.SSM_REAL_SELECTIVE, gy=_r(B, D, L), gh_last=ghl, ckpt=f["ckpt"], want=want, **t)
    torch.cuda.synchronize()
    assert f["y"].shape == (B, D, L)
    if L == 0:
        assert torch.equal(f["h_last"], t["h0"])
        assert torch.equal(g["gh0"], ghl)
    assert not g["gA"].any()   # no terms: B = 0 or L = 0, or D = 0 (no entries)
    assert g["gdelta"].shape == (B, D, L) and g["gBm"].shape == (B, L, N)
    assert not g["gBm"].any() and not g["gC"].any()   # sums over no channels (elements when D = 0 only)


@pytest.mark.parametrize("B,D,L", [(2, 3, 0), (2, 0, 50)])
def test_empty_real_dense(B, D, L):
    ssm = _ssm()
    N = 8
    t = dict(a=_r(B, D, L, N), b=_r(B, D, L, N), C=_r(B, L, N), h0=_r(B, D, N, seed=1))
    f = ssm.scan_fwd(ssm.SSM_REAL_DENSE, want_h_last=True, **t)
    ghl = _r(B, D, N, seed=2)
    g = ssm.scan_bwd(ssm.SSM_REAL_DENSE, gy=_r(B, D, L), gh_last=ghl, **t)
    torch.cuda.synchronize()
    assert torch.equal(f["h_last"], t["h0"])
    assert torch.equal(g["gh0"], ghl)
    assert g["gC"].shape == (B, L, N) and not g["gC"].any()


@pytest.mark.parametrize("B,H,L", [(2, 3, 0), (0, 3, 40)])
def test_empty_complex(B, H, L):
    ssm = _ssm()
    M = 8
    t = dict(r=_r(B, H, L).abs(), phi=_r(B, H, L), lam=torch.full((H, M), 0.95, device=DEV), theta=_r(H, M),
             u=_r(B, H, L, M, dtype=torch.complex64), c=_r(H, M, dtype=torch.complex64),
             h0=_r(B, H, M, dtype=torch.complex64, seed=3))
    f = ssm.scan_fwd(ssm.SSM_COMPLEX_SHARED, want_h_last=True, **t)
    ghl = _r(B, H, M, dtype=torch.complex64, seed=4)
    g = ssm.scan_bwd(ssm.SSM_COMPLEX_SHARED, gy=_r(B, H, L), gh_last=ghl, **t)
    rt = ssm.complex_rtrl(gy=_r(B, H, L), gh_last=ghl, **t)
    torch.cuda.synchronize()
    assert f["y"].shape == (B, H, L)
    assert torch.equal(f["h_last"], t["h0"])
    assert torch.equal(g["gh0"], ghl)
    for k in ("glam", "gtheta", "gc"):
        assert not g[k].any(), k
    for k in ("glam", "gtheta"):
        assert not rt[k].any(), k


@pytest.mark.parametrize("B,H,L", [(2, 3, 0), (0, 3, 40)])
def test_empty_complex_dense(B, H, L):
    ssm = _ssm()
    M = 8
    t = dict(a=_r(B, H, L, M, dtype=torch.complex64), u=_r(B, H, L, M, dtype=torch.complex64),
             c=_r(H, M, dtype=torch.complex64), h0=_r(B, H, M, dtype=torch.complex64, seed=3))
    f = ssm.scan_fwd(ssm.SSM_COMPLEX_DENSE, want_h_last=True, **t)
    ghl = _r(B, H, M, dtype=torch.complex64, seed=4)
    g = ssm.scan_bwd(ssm.SSM_COMPLEX_DENSE, gy=_r(B, H, L), gh_last=ghl, **t)
    torch.cuda.synchronize()
    assert f["y"].shape == (B, H, L) and g["ga"].shape == (B, H, L, M)
    assert torch.equal(f["h_last"], t["h0"])
    assert torch.equal(g["gh0"], ghl)
    assert not g["gc"].any()


@pytest.mark.parametrize("B,H,L", [(2, 3, 0), (0, 3, 70)])
def test_empty_pd(B, H, L):
    ssm = _ssm()
    N, K = 16, 4
    dct = torch.from_numpy(np.random.default_rng(5).integers(0, N, (H, K, N)).astype(np.int32)).to(DEV)
    t = dict(logits=_r(B, H, L, K), dict=dct, d=_r(B, H, L, N), b=_r(B, H, L, N), C=_r(B, H, L, N),
             h0=_r(B, H, N, seed=6))
    f = ssm.pd_scan_fwd(want_h_last=True, want_ckpt=True, **t)
    ghl = _r(B, H, N, seed=7)
    g = ssm.pd_scan_bwd(gy=_r(B, H, L), gh_last=ghl, **t)
    torch.cuda.synchronize()
    assert f["y"].shape == (B, H, L) and f["sel"].shape == (B, H, L)
    assert torch.equal(f["h_last"], t["h0"])
    assert torch.equal(g["gh0"], ghl)


@pytest.mark.parametrize("B,D", [(0, 4), (2, 0)])
def test_empty_sensitivities(B, D):
    ssm = _ssm()
    L, N = 100, 16
    t = dict(delta=_r(B, D, L).abs(), x=_r(B, D, L), A=-_r(D, N).abs(), Bm=_r(B, L, N), C=_r(B, L, N))
    s = ssm.impulse_sensitivity(t_out=50, **t)
    o = ssm.output_sensitivity(t_out=50, **t)
    rows = ssm.sensitivity_rows(t_out0=10, rows=4, **t)
    torch.cuda.synchronize()
    assert s["s"].shape == (B, D, L) and o["s_delta"].shape == (B, D, L) and rows.shape == (4, B, D, L)
