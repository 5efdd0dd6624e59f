"""The decode step on the GPU (msm_scan_step through the C ABI) against the fp64 oracle's step,
chained over a sequence against the sequence forward, and at the serving workload size."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import assert_close, dev, host, log

pytestmark = pytest.mark.gpu

W = workloads.WORKLOADS


def to_dev(si):
    io = si["io"]
    g = {k: dev(si[k], io) for k in ("x", "delta", "z", "B", "C")}
    g["A"] = dev(si["A"])
    g["Dskip"] = None if si["Dskip"] is None else dev(si["Dskip"])
    g["delta_bias"] = None if si["delta_bias"] is None else dev(si["delta_bias"])
    g["h"], g["v"] = dev(si["h"]), dev(si["v"])
    return g


def gpu_step(si, g, use_z=True, use_bias=True, zoh=False):
    import torch
    import selective_state_space_msm_amd as msm
    y = msm.msm_scan_step(g["x"], g["delta"], g["A"], g["B"], g["C"], g["h"], g["v"], si["beta"],
                          si["alpha"], g["Dskip"], z=g["z"] if use_z else None,
                          delta_bias=g["delta_bias"] if use_bias else None,
                          delta_softplus=si["softplus"], zero_order_hold=zoh)
    torch.cuda.synchronize()
    return y


def oracle_step(si, use_z=True, use_bias=True, zoh=False):
    return oracle.step(si["x"], si["delta"], si["A"], si["B"], si["C"], si["h"], si["v"],
                       si["beta"], si["alpha"], Dskip=si["Dskip"], z=si["z"] if use_z else None,
                       delta_bias=si["delta_bias"] if use_bias else None,
                       delta_softplus=si["softplus"], zoh=zoh)


def check_step(si, use_z=True, use_bias=True, tag="", zoh=False):
    log("step %s Bt=%d D=%d N=%d io=%s softplus=%s z=%s bias=%s"
        % (tag, si["x"].shape[0], si["x"].shape[1], si["A"].shape[1], si["io"], si["softplus"],
           use_z, use_bias))
    g = to_dev(si)
    y = gpu_step(si, g, use_z, use_bias, zoh)
    oy, oh, ov = oracle_step(si, use_z, use_bias, zoh)
    assert_close(host(y), oy, si["io"], "y " + tag)
    assert_close(host(g["h"]), oh, "f32", "h " + tag)
    assert_close(host(g["v"]), ov, "f32", "v " + tag)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("N", [1, 3, 4, 6, 16, 33, 64])
def test_state_counts(io, N):
    w = W["decode"].replace(Bt=3, D=70, N=N, io=io)
    check_step(workloads.make_step_inputs(w, seed=500 + N), tag="N=%d" % N)


@pytest.mark.parametrize("softplus,use_z,use_bias", [(True, False, True), (False, True, False),
                                                     (False, False, False), (True, True, False)])
def test_extras(softplus, use_z, use_bias):
    w = W["decode"].replace(Bt=5, D=130, N=16, io="f32", dskip=False, beta=0.0)
    si = workloads.make_step_inputs(w, seed=520, softplus=softplus)
    check_step(si, use_z, use_bias, tag="extras")


def test_unaligned_states():
    """States at a 4-byte offset (not 16-byte aligned) take the element-wise path."""
    import torch
    w = W["decode"].replace(Bt=2, D=66, N=16, io="bf16")
    si = workloads.make_step_inputs(w, seed=530)
    g = to_dev(si)
    n = si["h"].size
    for k in ("h", "v"):
        buf = torch.zeros(n + 1, dtype=torch.float32, device="cuda")
        view = buf[1:].view(si[k].shape)
        view.copy_(g[k])
        g[k] = view
    assert g["h"].data_ptr() % 16 != 0
    y = gpu_step(si, g)
    oy, oh, ov = oracle_step(si)
    assert_close(host(y), oy, si["io"], "unaligned y")
    assert_close(host(g["h"]), oh, "f32", "unaligned h")
    assert_close(host(g["v"]), ov, "f32", "unaligned v")


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_prefill_then_decode(io):
    """A prompt scanned by the fused forward (last states returned), then tokens decoded one at
    a time from those states: every output and the final states against the oracle's forward
    over prompt + tokens, and the decoded tokens against one GPU forward call."""
    import torch
    import selective_state_space_msm_amd as msm
    Bt, L1, L2, D, N = 2, 37, 12, 96, 16
    w = W["m130m"].replace(Bt=Bt, L=L1 + L2, D=D, N=N, io=io, dskip=True)
    inp = workloads.make_inputs(w, a_kind="random", seed=540)
    ex = workloads.make_fused_extras(w, 541)
    raw, z, bias = ex["delta_raw"], ex["z"], ex["delta_bias"]
    want, _, wh, wv = oracle.fused_fwd(inp["x"], raw, inp["A"], inp["B"], inp["C"], inp["beta"],
                                       inp["alpha"], Dskip=inp["Dskip"], z=z, delta_bias=bias,
                                       delta_softplus=True)
    d = lambda a: dev(a, io)
    A, Ds, bd = dev(inp["A"]), dev(inp["Dskip"]), dev(bias)
    x, dl, B, C, zz = (d(a) for a in (inp["x"], raw, inp["B"], inp["C"], z))
    sl = lambda t, a, b: t[:, a:b].contiguous()
    y1, h, v = msm.msm_selective_scan_fwd(sl(x, 0, L1), sl(dl, 0, L1), A, sl(B, 0, L1),
                                          sl(C, 0, L1), inp["beta"], inp["alpha"], Ds,
                                          z=sl(zz, 0, L1), delta_bias=bd, delta_softplus=True,
                                          return_last_state=True)
    ys = []
    for t in range(L1, L1 + L2):
        ys.append(msm.msm_scan_step(x[:, t].contiguous(), dl[:, t].contiguous(), A,
                                    B[:, t].contiguous(), C[:, t].contiguous(), h, v,
                                    inp["beta"], inp["alpha"], Ds, z=zz[:, t].contiguous(),
                                    delta_bias=bd, delta_softplus=True))
    yall = msm.msm_selective_scan_fwd(x, dl, A, B, C, inp["beta"], inp["alpha"], Ds, z=zz,
                                      delta_bias=bd, delta_softplus=True)
    torch.cuda.synchronize()
    yd = torch.stack(ys, dim=1)
    assert_close(host(y1), want[:, :L1], io, "prefill y")
    assert_close(host(yd), want[:, L1:], io, "decoded y")
    assert_close(host(h), wh, "f32", "decoded final h")
    assert_close(host(v), wv, "f32", "decoded final v")
    assert_close(host(yd), host(yall)[:, L1:], io, "decoded y vs one forward call")


def test_full_size_decode():
    """The serving workload (1024 sequences x 4096 channels x 16 states): every output and
    state against the oracle, then a second step from the updated states."""
    w = W["decode"]
    log("full-size decode: drawing inputs")
    si = workloads.make_step_inputs(w)
    g = to_dev(si)
    y = gpu_step(si, g)
    log("  oracle step")
    oy, oh, ov = oracle_step(si)
    assert_close(host(y), oy, w.io, "y")
    assert_close(host(g["h"]), oh, "f32", "h")
    assert_close(host(g["v"]), ov, "f32", "v")
    # second token from the states the GPU wrote (the oracle continues from its own)
    si2 = workloads.make_step_inputs(w, seed=w.seed + 100)
    for k in ("A", "Dskip", "delta_bias"):  # the layer's parameters stay those of the first token
        si2[k] = si[k]
    for k in ("x", "delta", "z", "B", "C"):
        g[k] = dev(si2[k], w.io)
    y2 = gpu_step(si2, g)
    si2["h"], si2["v"] = oh, ov
    oy2, oh2, ov2 = oracle_step(si2)
    assert_close(host(y2), oy2, w.io, "second y")
    assert_close(host(g["h"]), oh2, "f32", "second h")


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("N", [4, 5, 16, 33, 64])
def test_zero_order_hold(io, N):
    w = W["decode"].replace(Bt=3, D=70, N=N, io=io)
    check_step(workloads.make_step_inputs(w, seed=560 + N), tag="zoh N=%d" % N, zoh=True)
