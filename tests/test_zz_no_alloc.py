"""The allocation-free forward (ssm_scan_fwd_noalloc) against ssm_scan_fwd, through the C ABI: two calls
in a row on the static scratch, the second with a smaller input, for the modes whose forward uses
scratch memory (segment summaries and carries), bit for bit."""
import ctypes

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def T(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _ssm():
    import selective_state_space_chunked_amd as ssm
    return ssm


def _ws_need(ssm, mode, tensors):
    from selective_state_space_chunked_amd import binding
    args, _, _ = binding._scan_args(mode, **tensors)
    n = ctypes.c_size_t(0)
    assert binding.lib().ssm_workspace_bytes(binding.SSM_OP_SCAN_FWD, ctypes.byref(args), ctypes.byref(n)) == 0
    return n.value


def _compare(ssm, mode, tensors):
    assert _ws_need(ssm, mode, tensors) > 0      # the forward uses scratch memory at this shape
    ref = ssm.scan_fwd(mode, want_h_last=True, want_ckpt=True, **tensors)
    got = ssm.scan_fwd_noalloc(mode, want_h_last=True, want_ckpt=True, **tensors)
    torch.cuda.synchronize()
    for k in ("y", "h_last", "ckpt"):
        assert torch.equal(got[k], ref[k]), k


def _selective(B, D, L, seed):
    cfg = synth.make_real(B=B, D=D, N=16, L=L, seed=seed)
    return {k: T(cfg[k]) for k in ("delta", "x", "Bm", "C", "A")}


def _complex(B, H, L, seed):
    cfg = synth.make_complex(B=B, H=H, M=64, L=L, seed=seed)
    return {k: T(cfg[k]) for k in ("r", "phi", "lam", "theta", "u", "c")}


def test_noalloc_forward_two_calls_selective():
    ssm = _ssm()
    _compare(ssm, ssm.SSM_REAL_SELECTIVE, _selective(2, 64, 6000, 1))
    _compare(ssm, ssm.SSM_REAL_SELECTIVE, _selective(1, 16, 1500, 2))     # smaller: stale scratch beyond it


def test_noalloc_forward_two_calls_complex():
    ssm = _ssm()
    _compare(ssm, ssm.SSM_COMPLEX_SHARED, _complex(4, 8, 3000, 3))
    _compare(ssm, ssm.SSM_COMPLEX_SHARED, _complex(1, 2, 700, 4))


def test_noalloc_forward_after_other_calls():
    """Interleaved with workspace calls and a backward (which uses its own workspace)."""
    ssm = _ssm()
    t = _selective(1, 32, 4000, 5)
    f = ssm.scan_fwd_noalloc(ssm.SSM_REAL_SELECTIVE, want_ckpt=True, **t)
    g = ssm.scan_bwd(ssm.SSM_REAL_SELECTIVE, gy=torch.randn_like(t["x"]), ckpt=f["ckpt"], want=("gx",), **t)
    f2 = ssm.scan_fwd_noalloc(ssm.SSM_REAL_SELECTIVE, want_ckpt=True, **t)
    torch.cuda.synchronize()
    assert torch.equal(f["y"], f2["y"]) and torch.equal(f["ckpt"], f2["ckpt"])
    assert torch.isfinite(g["gx"]).all()
