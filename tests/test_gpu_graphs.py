"""HIP graph capture: every entry point enqueues only kernels on the caller's stream and allocates nothing, so a captured forward + backward
replays correctly.  Each replay follows eager work and a synchronisation, the
inputs change between replays (copied into the captured tensors), and every
replay is compared bit for bit with an eager call on the same inputs."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _ssm():
    import selective_state_space_chunked_amd as ssm
    return ssm


def T(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _capture(fn):
    """Capture fn() (which writes only into tensors it closes over) into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                      # warm-up outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _replay_and_check(g, outs, inputs, new_inputs, eager):
    """For each new input set: copy into the captured inputs, do unrelated eager
    work, replay, and compare every output with eager(new inputs)."""
    for k, nin in enumerate(new_inputs):
        for name, t in nin.items():
            inputs[name].copy_(t)
        junk = torch.randn(1 << 20, device=DEV).sum()   # eager work between replays
        torch.cuda.synchronize()
        for o in outs.values():
            o.fill_(float("nan")) if o.is_floating_point() or o.is_complex() else o.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        ref = eager({name: t.clone() for name, t in inputs.items()})
        torch.cuda.synchronize()
        for name, o in outs.items():
            assert torch.equal(o, ref[name]), f"replay {k}: {name} differs from the eager call"
        del junk


def test_graph_selective_fwd_bwd():
    ssm = _ssm()
    S = ssm.SSM_REAL_SELECTIVE

    def mk(seed):
        cfg = synth.make_real(B=2, D=48, N=16, L=700, seed=seed)
        return {k: T(cfg[k]) for k in ("delta", "x", "Bm", "C", "A", "gy")}

    inp = mk(0)
    want = ("gdelta", "gx", "gA", "gBm", "gC", "gh0")

    def eager(i):
        t = {k: v for k, v in i.items() if k != "gy"}
        f = ssm.scan_fwd(S, want_h_last=True, want_ckpt=True, **t)
        g = ssm.scan_bwd(S, gy=i["gy"], ckpt=f["ckpt"], want=want, **t)
        return {**{"y": f["y"], "h_last": f["h_last"], "ckpt": f["ckpt"]}, **g}

    outs = eager(inp)
    t = {k: v for k, v in inp.items() if k != "gy"}
    fo = {k: outs[k] for k in ("y", "h_last", "ckpt")}
    go = {k: outs[k] for k in want}

    def step():
        ssm.scan_fwd(S, want_h_last=True, want_ckpt=True, out=fo, **t)
        ssm.scan_bwd(S, gy=inp["gy"], ckpt=fo["ckpt"], want=want, out=go, **t)

    g = _capture(step)
    _replay_and_check(g, outs, inp, [mk(1), mk(2), mk(3)], eager)


def test_graph_complex_fwd_bwd_rtrl():
    ssm = _ssm()
    Cx = ssm.SSM_COMPLEX_SHARED

    def mk(seed):
        cfg = synth.make_complex(B=2, H=3, M=64, L=300, seed=seed)
        return {k: T(cfg[k]) for k in ("r", "phi", "lam", "theta", "u", "c", "gy")}

    inp = mk(0)
    want = ("gu", "gr", "gphi", "glam", "gtheta", "gc", "gh0")

    def eager(i):
        t = {k: v for k, v in i.items() if k != "gy"}
        f = ssm.scan_fwd(Cx, want_h_last=True, want_ckpt=True, **t)
        g = ssm.scan_bwd(Cx, gy=i["gy"], ckpt=f["ckpt"], want=want, **t)
        r = ssm.complex_rtrl(gy=i["gy"], **t)
        return {"y": f["y"], "h_last": f["h_last"], "ckpt": f["ckpt"], **g,
                "rtrl_y": r["y"], "rtrl_glam": r["glam"], "rtrl_gtheta": r["gtheta"]}

    outs = eager(inp)
    t = {k: v for k, v in inp.items() if k != "gy"}
    fo = {k: outs[k] for k in ("y", "h_last", "ckpt")}
    go = {k: outs[k] for k in want}
    ro = {"y": outs["rtrl_y"], "glam": outs["rtrl_glam"], "gtheta": outs["rtrl_gtheta"]}

    def step():
        ssm.scan_fwd(Cx, want_h_last=True, want_ckpt=True, out=fo, **t)
        ssm.scan_bwd(Cx, gy=inp["gy"], ckpt=fo["ckpt"], want=want, out=go, **t)
        ssm.complex_rtrl(gy=inp["gy"], out=ro, **t)

    g = _capture(step)
    _replay_and_check(g, outs, inp, [mk(1), mk(2)], eager)


def test_graph_complex_dense_fwd_bwd():
    """Given complex transitions: forward with checkpoints, backward from them and backward recomputing them."""
    ssm = _ssm()
    Cx = ssm.SSM_COMPLEX_DENSE

    def mk(seed):
        cfg = synth.make_complex_dense(B=2, H=3, M=64, L=300, seed=seed)
        return {k: T(cfg[k]) for k in ("a", "u", "c", "gy")}

    inp = mk(0)
    want = ("ga", "gu", "gc", "gh0")

    def eager(i):
        t = {k: v for k, v in i.items() if k != "gy"}
        f = ssm.scan_fwd(Cx, want_h_last=True, want_ckpt=True, **t)
        g = ssm.scan_bwd(Cx, gy=i["gy"], ckpt=f["ckpt"], want=want, **t)
        g2 = ssm.scan_bwd(Cx, gy=i["gy"], want=("ga", "gc"), **t)
        return {"y": f["y"], "h_last": f["h_last"], "ckpt": f["ckpt"], **g, "ga2": g2["ga"], "gc2": g2["gc"]}

    outs = eager(inp)
    t = {k: v for k, v in inp.items() if k != "gy"}
    fo = {k: outs[k] for k in ("y", "h_last", "ckpt")}
    go = {k: outs[k] for k in want}
    go2 = {"ga": outs["ga2"], "gc": outs["gc2"]}

    def step():
        ssm.scan_fwd(Cx, want_h_last=True, want_ckpt=True, out=fo, **t)
        ssm.scan_bwd(Cx, gy=inp["gy"], ckpt=fo["ckpt"], want=want, out=go, **t)
        ssm.scan_bwd(Cx, gy=inp["gy"], want=("ga", "gc"), out=go2, **t)

    g = _capture(step)
    _replay_and_check(g, outs, inp, [mk(1), mk(2)], eager)


def test_graph_pd_fwd_bwd_ste():
    ssm = _ssm()

    def mk(seed):
        cfg = synth.make_pd(B=2, H=4, N=16, L=500, K=8, seed=seed)
        return {k: T(cfg[k]) for k in ("logits", "dict", "d", "b", "C", "gy")}

    inp = mk(0)
    want = ("gd", "gb", "gC", "gh0", "glogits")

    def eager(i):
        t = {k: v for k, v in i.items() if k != "gy"}
        f = ssm.pd_scan_fwd(want_ckpt=True, **t)
        tb = {k: v for k, v in t.items() if k != "logits"}
        g = ssm.pd_scan_bwd(gy=i["gy"], ckpt=f["ckpt"], sel=f["sel"], ste_logits=t["logits"], tau=0.7, want=want,
                            **tb)
        return {"y": f["y"], "sel": f["sel"], "ckpt": f["ckpt"], **g}

    outs = eager(inp)
    t = {k: v for k, v in inp.items() if k != "gy"}
    tb = {k: v for k, v in t.items() if k != "logits"}
    fo = {k: outs[k] for k in ("y", "sel", "ckpt")}
    go = {k: outs[k] for k in want}

    def step():
        ssm.pd_scan_fwd(want_ckpt=True, out=fo, **t)
        ssm.pd_scan_bwd(gy=inp["gy"], ckpt=fo["ckpt"], sel=fo["sel"], ste_logits=t["logits"], tau=0.7, want=want,
                        out=go, **tb)

    g = _capture(step)
    _replay_and_check(g, outs, inp, [mk(1), mk(2)], eager)


def test_graph_sensitivities():
    """Impulse sensitivity, output sensitivity (with its forward into the workspace) and Jacobian rows."""
    ssm = _ssm()

    def mk(seed):
        cfg = synth.make_real(B=1, D=40, N=16, L=900, seed=seed)
        return {k: T(cfg[k]) for k in ("delta", "x", "Bm", "C", "A")}

    inp = mk(10)

    def eager(i):
        a = ssm.impulse_sensitivity(t_out=700, **i)
        b = ssm.output_sensitivity(t_out=650, want_y=True, **i)
        r = ssm.sensitivity_rows(t_out0=600, rows=16, **i)
        return {"s": a["s"], "y": a["y"], "s_x": b["s_x"], "s_delta": b["s_delta"], "y2": b["y"], "rows": r}

    outs = eager(inp)
    ao = {"s": outs["s"], "y": outs["y"]}
    bo = {"s_x": outs["s_x"], "s_delta": outs["s_delta"], "y": outs["y2"]}

    def step():
        ssm.impulse_sensitivity(t_out=700, out=ao, **inp)
        ssm.output_sensitivity(t_out=650, want_y=True, out=bo, **inp)
        ssm.sensitivity_rows(t_out0=600, rows=16, out=outs["rows"], **inp)

    g = _capture(step)
    _replay_and_check(g, outs, inp, [mk(11), mk(12)], eager)
