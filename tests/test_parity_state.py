"""Initial state and continuation on the GPU (msm_scan_fwd_state / msm_scan_bwd_state through
the C ABI) against the fp64 oracle, plus the split-sequence identities at workload sizes."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import assert_close, dev, host, inputs_to_device, log, sample_channels, sub_problem

pytestmark = pytest.mark.gpu

W = workloads.WORKLOADS
SMALL = W["bwd"].replace(Bt=2, L=100, D=70, N=16)


def run_fwd_state(inp, g, h0, v0, plan=None):
    import torch
    import selective_state_space_msm_amd as msm
    y, lh, lv = msm.msm_scan_fwd(g["x"], g["delta"], g["A"], g["B"], g["C"], inp["beta"],
                                 inp["alpha"], g["Dskip"], return_last_state=True, plan=plan,
                                 h0=None if h0 is None else dev(h0),
                                 v0=None if v0 is None else dev(v0))
    torch.cuda.synchronize()
    return y, lh, lv


def run_bwd_state(inp, g, h0, v0, dlh, dlv, plan=None):
    import torch
    import selective_state_space_msm_amd as msm
    t = lambda a: None if a is None else dev(a)
    out = msm.msm_scan_bwd(g["x"], g["delta"], g["A"], g["B"], g["C"], g["dy"], inp["beta"],
                           inp["alpha"], g["Dskip"], plan=plan, h0=t(h0), v0=t(v0),
                           dlast_h=t(dlh), dlast_v=t(dlv), state_grads=True)
    torch.cuda.synchronize()
    return out


def check_fwd(inp, h0, v0, plan=None, tag=""):
    io = inp["io"]
    log("fwd-state %s shape=%s io=%s plan=%s" % (tag, inp["x"].shape, io, plan))
    y, lh, lv = run_fwd_state(inp, inputs_to_device(inp), h0, v0, plan)
    oy, olh, olv = oracle.fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["beta"],
                              inp["alpha"], Dskip=inp["Dskip"], h0=h0, v0=v0)
    assert_close(host(y), oy, io, "y " + tag)
    assert_close(host(lh), olh, "f32", "last_h " + tag)
    assert_close(host(lv), olv, "f32", "last_v " + tag)


def check_bwd(inp, h0, v0, dlh, dlv, plan=None, tag=""):
    io = inp["io"]
    log("bwd-state %s shape=%s io=%s plan=%s" % (tag, inp["x"].shape, io, plan))
    got = run_bwd_state(inp, inputs_to_device(inp), h0, v0, dlh, dlv, plan)
    want = oracle.bwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["dy"],
                      inp["beta"], inp["alpha"], Dskip=inp["Dskip"], h0=h0, v0=v0, dlast_h=dlh,
                      dlast_v=dlv)
    for k in ("dx", "ddelta", "dA", "dB", "dC", "dDskip", "dh0", "dv0"):
        if want[k] is None:
            continue
        tol = "f32" if k in ("dA", "dDskip", "dh0", "dv0") and io == "f32" else io
        assert_close(host(got[k]), want[k], tol, "%s %s" % (k, tag))


# ---- forward from an initial state ----

@pytest.mark.parametrize("beta", [0.9, 0.0])
@pytest.mark.parametrize("chunks", [1, 2, 4])
def test_fwd_tiny(beta, chunks):
    w = W["tiny"].replace(beta=beta)
    inp = workloads.make_inputs(w)
    h0, v0 = workloads.make_state(w, 201)
    check_fwd(inp, h0, v0, plan={"states_per_wave": 2, "chunks": chunks}, tag="tiny")


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("plan", [None, {"states_per_wave": 4, "chunks": 3},
                                  {"states_per_wave": 16, "chunks": 1}])
def test_fwd_small_ragged(io, plan):
    w = SMALL.replace(io=io, dskip=True, beta=0.8, alpha=0.7)
    inp = workloads.make_inputs(w, a_kind="random", seed=211)
    h0, v0 = workloads.make_state(w, 212)
    check_fwd(inp, h0, v0, plan=plan, tag="small")
    # only one of the two states given: the other starts at zero
    check_fwd(inp, h0, None, plan=plan, tag="small h0 only")
    check_fwd(inp, None, v0, plan=plan, tag="small v0 only")


@pytest.mark.parametrize("N", [3, 33])
def test_fwd_state_counts(N):
    w = SMALL.replace(L=45, D=40, N=N, dskip=True)
    inp = workloads.make_inputs(w, a_kind="random", seed=220 + N)
    h0, v0 = workloads.make_state(w, 230 + N)
    check_fwd(inp, h0, v0, tag="N=%d" % N)
    check_fwd(inp, h0, v0, plan={"states_per_wave": 4, "chunks": 2}, tag="N=%d chunked" % N)


def test_fwd_continuation_long():
    """The long workload scanned in two calls (the second started from the first one's final
    state) against one call over the whole sequence, and sampled channels against the oracle."""
    import torch
    w = W["long"]
    inp = workloads.make_inputs(w)
    g = inputs_to_device(inp)
    y, lh, lv = run_fwd_state(inp, g, None, None)
    L1 = 40000
    g1 = {k: (v[:, :L1].contiguous() if k in ("x", "delta", "B", "C") else v) for k, v in g.items()}
    g2 = {k: (v[:, L1:].contiguous() if k in ("x", "delta", "B", "C") else v) for k, v in g.items()}
    import selective_state_space_msm_amd as msm
    y1, lh1, lv1 = msm.msm_scan_fwd(g1["x"], g1["delta"], g1["A"], g1["B"], g1["C"], inp["beta"],
                                    inp["alpha"], g1["Dskip"], return_last_state=True)
    y2, lh2, lv2 = msm.msm_scan_fwd(g2["x"], g2["delta"], g2["A"], g2["B"], g2["C"], inp["beta"],
                                    inp["alpha"], g2["Dskip"], return_last_state=True, h0=lh1,
                                    v0=lv1)
    torch.cuda.synchronize()
    yc = torch.cat([y1, y2], dim=1)
    assert_close(host(yc), host(y), w.io, "continued y vs one call")
    assert_close(host(lh2), host(lh), "f32", "continued last_h vs one call")
    dsel = sample_channels(w.D, 6, seed=w.seed)
    sub = sub_problem(inp, dsel=dsel)
    oy, olh, _ = oracle.fwd(sub["x"], sub["delta"], sub["A"], sub["B"], sub["C"], inp["beta"],
                            inp["alpha"], Dskip=sub["Dskip"])
    assert_close(host(yc)[:, :, dsel], oy, w.io, "continued y vs oracle")
    assert_close(host(lh2)[:, dsel], olh, "f32", "continued last_h vs oracle")


# ---- backward with initial state and terminal adjoints ----

@pytest.mark.parametrize("beta", [0.9, 0.0])
@pytest.mark.parametrize("K", [1, 2])
def test_bwd_tiny(beta, K):
    w = W["tiny"].replace(beta=beta)
    inp = workloads.make_inputs(w, with_dy=True)
    h0, v0 = workloads.make_state(w, 301)
    dlh, dlv = workloads.make_state(w, 302)
    check_bwd(inp, h0, v0, dlh, dlv, plan={"states_per_wave": K}, tag="tiny")


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("K", [1, 2, 4])
@pytest.mark.parametrize("L", [100, 96, 1])
def test_bwd_small(io, K, L):
    # L = 100: the last tile holds 4 rows; L = 96: it is full; L = 1: one step in total
    w = SMALL.replace(io=io, L=L, dskip=True, beta=0.85, alpha=0.6)
    inp = workloads.make_inputs(w, a_kind="random", seed=311)
    h0, v0 = workloads.make_state(w, 312)
    dlh, dlv = workloads.make_state(w, 313)
    check_bwd(inp, h0, v0, dlh, dlv, plan={"states_per_wave": K}, tag="small L=%d" % L)
    check_bwd(inp, None, None, dlh, None, plan={"states_per_wave": K}, tag="small dlast_h only")


@pytest.mark.parametrize("N", [5, 33])
def test_bwd_state_counts(N):
    w = SMALL.replace(L=37, D=45, N=N, dskip=True)
    inp = workloads.make_inputs(w, a_kind="random", seed=320 + N)
    h0, v0 = workloads.make_state(w, 330 + N)
    dlh, dlv = workloads.make_state(w, 340 + N)
    check_bwd(inp, h0, v0, dlh, dlv, tag="N=%d" % N)


def test_bwd_split_sequence():
    """A sequence differentiated in two calls (the second part first, its dh0 / dv0 passed as
    the first part's terminal adjoints) against the oracle's backward of the whole sequence."""
    import torch
    w = SMALL.replace(L=150, dskip=True, beta=0.9)
    inp = workloads.make_inputs(w, a_kind="random", seed=351)
    h0, v0 = workloads.make_state(w, 352)
    L1 = 61
    g = inputs_to_device(inp)
    part = lambda sl: {k: (v[:, sl].contiguous() if k in ("x", "delta", "B", "C", "dy") else v)
                       for k, v in g.items()}
    g1, g2 = part(slice(0, L1)), part(slice(L1, w.L))
    import selective_state_space_msm_amd as msm
    _, lh1, lv1 = msm.msm_scan_fwd(g1["x"], g1["delta"], g1["A"], g1["B"], g1["C"], inp["beta"],
                                   inp["alpha"], g1["Dskip"], return_last_state=True, h0=dev(h0),
                                   v0=dev(v0))
    o2 = msm.msm_scan_bwd(g2["x"], g2["delta"], g2["A"], g2["B"], g2["C"], g2["dy"], inp["beta"],
                          inp["alpha"], g2["Dskip"], h0=lh1, v0=lv1, state_grads=True)
    o1 = msm.msm_scan_bwd(g1["x"], g1["delta"], g1["A"], g1["B"], g1["C"], g1["dy"], inp["beta"],
                          inp["alpha"], g1["Dskip"], h0=dev(h0), v0=dev(v0), dlast_h=o2["dh0"],
                          dlast_v=o2["dv0"], state_grads=True)
    torch.cuda.synchronize()
    want = oracle.bwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["dy"],
                      inp["beta"], inp["alpha"], Dskip=inp["Dskip"], h0=h0, v0=v0)
    for k in ("dx", "ddelta", "dB", "dC"):
        assert_close(np.concatenate([host(o1[k]), host(o2[k])], axis=1), want[k], w.io,
                     "split %s" % k)
    for k in ("dA", "dDskip"):
        assert_close(host(o1[k]) + host(o2[k]), want[k], "f32", "split %s" % k)
    for k in ("dh0", "dv0"):
        assert_close(host(o1[k]), want[k], "f32", "split %s" % k)
