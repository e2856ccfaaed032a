"""Element-wise comparison of a GPU result against the fp64 oracle.

Pass iff every element satisfies |g - o| <= atol + rtol * |o| (complex: the
modulus) and the GPU value is finite wherever the oracle's is.  The message
names the worst element and the max absolute / relative errors.
"""
import numpy as np
import torch

# tolerances: fp32 streams 1e-4 relative / 1e-5 absolute; bf16 streams 2e-2 relative
F32 = dict(rtol=1e-4, atol=1e-5)
BF16 = dict(rtol=2e-2, atol=1e-5)


def to_np(t):
    if isinstance(t, torch.Tensor):
        t = t.detach()
        if t.dtype == torch.bfloat16:
            t = t.float()
        return t.cpu().numpy()
    return np.asarray(t)


def assert_close(name, gpu, ora, rtol, atol):
    g = to_np(gpu).astype(np.complex128 if np.iscomplexobj(to_np(gpu)) else np.float64)
    o = np.asarray(ora)
    assert g.shape == o.shape, f"{name}: shape {g.shape} vs oracle {o.shape}"
    fin_o = np.isfinite(o)
    bad_fin = fin_o & ~np.isfinite(g)
    assert not bad_fin.any(), f"{name}: {int(bad_fin.sum())} non-finite GPU values where the oracle is finite"
    err = np.abs(g - o)
    bound = atol + rtol * np.abs(o)
    viol = (err > bound) & fin_o
    rel = np.where(np.abs(o) > atol / rtol, err / np.maximum(np.abs(o), 1e-300), 0.0)
    if viol.any():
        idx = np.unravel_index(np.argmax(np.where(viol, err - bound, -np.inf)), err.shape)
        raise AssertionError(
            f"{name}: {int(viol.sum())}/{err.size} elements out of tolerance (rtol={rtol}, atol={atol}); "
            f"worst at {idx}: gpu={g[idx]!r} oracle={o[idx]!r}; max abs err {err.max():.3e}, "
            f"max rel err {rel.max():.3e}")
    return float(err.max()), float(rel.max())
