"""The fused op on the GPU (msm_selective_scan_fwd / msm_selective_scan_bwd through the C ABI:
delta bias + softplus, SiLU output gate, with and without initial state) against the fp64
oracle's fused op, at small sizes in full and at workload sizes on sampled outputs."""
import numpy as np
import pytest

import oracle
import workloads
from conditioning import assert_close_cond, spread
from gpu_util import assert_close, dev, host, inputs_to_device, log

pytestmark = pytest.mark.gpu

W = workloads.WORKLOADS
SMALL = W["bwd"].replace(Bt=2, L=100, D=70, N=16)
FWD_OUT = ("y", "last_h", "last_v")
BWD_OUT = ("dx", "ddelta", "dA", "dB", "dC", "dDskip", "dz", "ddelta_bias", "dh0", "dv0")
F32_OUT = ("last_h", "last_v", "dA", "dDskip", "ddelta_bias", "dh0", "dv0")


def fused_inputs(w, seed, softplus=True, use_z=True, use_bias=True, a_kind="random",
                 with_dy=True, zoh=False):
    inp = workloads.make_inputs(w, a_kind=a_kind, seed=seed, with_dy=with_dy)
    ex = workloads.make_fused_extras(w, seed + 7, softplus=softplus)
    inp["delta"] = ex["delta_raw"]
    inp["z"] = ex["z"] if use_z else None
    inp["delta_bias"] = ex["delta_bias"] if use_bias else None
    inp["softplus"] = softplus
    inp["zoh"] = zoh
    return inp


def to_device(inp):
    g = inputs_to_device(inp)
    g["z"] = None if inp["z"] is None else dev(inp["z"], inp["io"])
    g["delta_bias"] = None if inp["delta_bias"] is None else dev(inp["delta_bias"])
    return g


def gpu_fwd(inp, g, plan=None, h0=None, v0=None):
    import torch
    import selective_state_space_msm_amd as msm
    y, lh, lv = msm.msm_selective_scan_fwd(
        g["x"], g["delta"], g["A"], g["B"], g["C"], inp["beta"], inp["alpha"], g["Dskip"],
        z=g["z"], delta_bias=g["delta_bias"], delta_softplus=inp["softplus"],
        zero_order_hold=inp.get("zoh", False),
        h0=None if h0 is None else dev(h0), v0=None if v0 is None else dev(v0),
        return_last_state=True, plan=plan)
    torch.cuda.synchronize()
    return dict(y=y, last_h=lh, last_v=lv)


def gpu_bwd(inp, g, plan=None, h0=None, v0=None, dlh=None, dlv=None):
    import torch
    import selective_state_space_msm_amd as msm
    t = lambda a: None if a is None else dev(a)
    o = msm.msm_selective_scan_bwd(
        g["x"], g["delta"], g["A"], g["B"], g["C"], g["dy"], inp["beta"], inp["alpha"],
        g["Dskip"], z=g["z"], delta_bias=g["delta_bias"], delta_softplus=inp["softplus"],
        zero_order_hold=inp.get("zoh", False), h0=t(h0), v0=t(v0), dlast_h=t(dlh),
        dlast_v=t(dlv), state_grads=True, plan=plan)
    torch.cuda.synchronize()
    return o


def oracle_fwd(inp, h0=None, v0=None):
    y, _, lh, lv = oracle.fused_fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"],
                                    inp["beta"], inp["alpha"], Dskip=inp["Dskip"], z=inp["z"],
                                    delta_bias=inp["delta_bias"],
                                    delta_softplus=inp["softplus"], h0=h0, v0=v0,
                                    zoh=inp.get("zoh", False))
    return dict(y=y, last_h=lh, last_v=lv)


def oracle_bwd(inp, h0=None, v0=None, dlh=None, dlv=None):
    return oracle.fused_bwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["dy"],
                            inp["beta"], inp["alpha"], Dskip=inp["Dskip"], z=inp["z"],
                            delta_bias=inp["delta_bias"], delta_softplus=inp["softplus"],
                            h0=h0, v0=v0, dlast_h=dlh, dlast_v=dlv, zoh=inp.get("zoh", False))


FUSED_KEYS = ("x", "delta", "B", "C", "dy", "z")


def check_bias_reduction(got_bias, got_ddelta, io, what):
    """ddelta_bias is the sum over batch rows and steps of the raw-delta gradient: the kernel
    sums its unrounded values, so the difference from the sum of the stored (rounded) ddelta is
    at most the rounding of those elements plus the rounding of the result."""
    dd = np.asarray(got_ddelta, np.float64)
    want = dd.sum(axis=(0, 1))
    u = 2.0 ** -24 if io == "f32" else 2.0 ** -8
    lim = 1e-6 + u * np.abs(dd).sum(axis=(0, 1)) + 2.0 ** -23 * np.abs(want)
    err = np.abs(np.asarray(got_bias, np.float64) - want)
    assert np.all(err <= lim), "%s: %d of %d channels differ from the sum of ddelta (worst %.3g, " \
        "allowed %.3g)" % (what, (err > lim).sum(), err.size, err.max(), lim[np.argmax(err - lim)])


def compare(got, want, names, io, tag, sp=None):
    """Every output against the oracle; sp (conditioning.spread of the oracle) adds the
    conditioning term to the bound of the outputs it holds."""
    for k in names:
        if want.get(k) is None:
            assert got.get(k) is None, k
            continue
        tol = "f32" if (k in F32_OUT and io == "f32") or k in ("last_h", "last_v") else io
        if k == "ddelta_bias":
            check_bias_reduction(host(got[k]), host(got["ddelta"]), io, "%s %s" % (k, tag))
        if sp is not None and k in sp:
            n = assert_close_cond(host(got[k]), want[k], sp[k], tol, "%s %s" % (k, tag))
            if n:
                log("  %s %s: %d elements needed the conditioning term" % (k, tag, n))
        else:
            assert_close(host(got[k]), want[k], tol, "%s %s" % (k, tag))


def check(inp, fplan=None, bplan=None, state=False, tag="", cond_outputs=BWD_OUT):
    io = inp["io"]
    w = inp["x"].shape
    h0 = v0 = dlh = dlv = None
    if state:
        rng = np.random.default_rng(5)
        h0, v0, dlh, dlv = (rng.standard_normal((w[0], w[2], inp["A"].shape[1])).astype(np.float32)
                            for _ in range(4))
    log("fused %s shape=%s io=%s softplus=%s z=%s bias=%s zoh=%s state=%s plans=%s/%s"
        % (tag, w, io, inp["softplus"], inp["z"] is not None, inp["delta_bias"] is not None,
           inp.get("zoh", False), state, fplan, bplan))
    g = to_device(inp)
    compare(gpu_fwd(inp, g, fplan, h0, v0), oracle_fwd(inp, h0, v0), FWD_OUT, io, "fwd " + tag)
    # gradients are differences of large per-state terms (and ddelta_bias sums ddelta over every
    # row and step while the sum itself cancels): each is held to the bound plus the oracle's
    # own spread under one fp32 rounding of the inputs (tests/conditioning.py); ddelta_bias also
    # to the sum of the returned ddelta (check_bias_reduction)
    fn = lambda q: oracle_bwd(q, h0, v0, dlh, dlv)
    want, sp = spread(fn, inp, FUSED_KEYS, cond_outputs)
    compare(gpu_bwd(inp, g, bplan, h0, v0, dlh, dlv), want, BWD_OUT, io, "bwd " + tag, sp)


EXTRAS = [(True, True, True), (False, True, True), (True, False, False), (False, False, True),
          (True, True, False), (False, True, False)]


@pytest.mark.parametrize("softplus,use_z,use_bias", EXTRAS)
@pytest.mark.parametrize("beta", [0.9, 0.0])
def test_tiny(softplus, use_z, use_bias, beta):
    w = W["tiny"].replace(beta=beta, dskip=True)
    inp = fused_inputs(w, 401, softplus, use_z, use_bias)
    check(inp, {"states_per_wave": 2, "chunks": 2}, {"states_per_wave": 1}, tag="tiny")


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("K", [1, 2, 4])
def test_small_ragged(io, K):
    w = SMALL.replace(io=io, dskip=True, beta=0.85, alpha=0.6)
    inp = fused_inputs(w, 411)
    check(inp, {"states_per_wave": 4 if K == 4 else 2 * K, "chunks": K}, {"states_per_wave": K},
          tag="small K=%d" % K)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_small_with_state(io):
    w = SMALL.replace(io=io, L=45, dskip=True, beta=0.9)
    inp = fused_inputs(w, 421)
    check(inp, None, None, state=True, tag="small state")
    check(inp, {"states_per_wave": 16, "chunks": 1}, {"states_per_wave": 2}, state=True,
          tag="small state K16")


@pytest.mark.parametrize("N", [3, 9])
def test_state_counts(N):
    w = SMALL.replace(L=37, D=45, N=N, dskip=False)
    inp = fused_inputs(w, 430 + N)
    check(inp, tag="N=%d" % N)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("N", [20, 32, 33, 64])
def test_many_states(io, N):
    # 32 padded states (N = 20, 32): the half-wavefront backward with 8 wavefronts; 64 (N = 33,
    # 64): the 64-state forward kernels and the full-wavefront backward
    w = SMALL.replace(L=40, D=70, N=N, io=io, dskip=True)
    check(fused_inputs(w, 441 + N), tag="N=%d" % N, state=True)
    check(fused_inputs(w.replace(dskip=False, beta=0.0), 442 + N, softplus=False), tag="N=%d" % N)


def test_plain_equivalence():
    """No extras through the fused entry points gives the plain entry points' results bit for
    bit; the fused kernels with a zero bias, no softplus and no gate agree within rounding."""
    import torch
    import selective_state_space_msm_amd as msm
    w = SMALL.replace(dskip=True)
    inp = workloads.make_inputs(w, a_kind="random", seed=451, with_dy=True)
    g = inputs_to_device(inp)
    args = (g["x"], g["delta"], g["A"], g["B"], g["C"])
    y0 = msm.msm_scan_fwd(*args, inp["beta"], inp["alpha"], g["Dskip"])
    y1 = msm.msm_selective_scan_fwd(*args, inp["beta"], inp["alpha"], g["Dskip"])
    zero = torch.zeros(w.D, dtype=torch.float32, device="cuda")
    y2 = msm.msm_selective_scan_fwd(*args, inp["beta"], inp["alpha"], g["Dskip"], delta_bias=zero)
    b0 = msm.msm_scan_bwd(*args, g["dy"], inp["beta"], inp["alpha"], g["Dskip"])
    b1 = msm.msm_selective_scan_bwd(*args, g["dy"], inp["beta"], inp["alpha"], g["Dskip"])
    b2 = msm.msm_selective_scan_bwd(*args, g["dy"], inp["beta"], inp["alpha"], g["Dskip"],
                                    delta_bias=zero)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    assert_close(host(y2), host(y0), w.io, "zero bias y")
    for k in ("dx", "ddelta", "dA", "dB", "dC", "dDskip"):
        assert torch.equal(b0[k], b1[k]), k
        assert_close(host(b2[k]), host(b0[k]), w.io, "zero bias " + k)
    q = dict(inp, z=None, delta_bias=np.zeros(w.D, np.float32), softplus=False)
    want, sp = spread(oracle_bwd, q, FUSED_KEYS, ("ddelta_bias",))
    assert_close_cond(host(b2["ddelta_bias"]), want["ddelta_bias"], sp["ddelta_bias"], w.io,
                      "zero bias ddelta_bias")
    check_bias_reduction(host(b2["ddelta_bias"]), host(b2["ddelta"]), w.io, "zero bias reduction")


def test_full_size_forward():
    """The headline forward shape with every extra: every output against the oracle."""
    w = W["m1p4b"].replace(dskip=True)
    log("full-size fused fwd: drawing inputs")
    inp = fused_inputs(w, 461, a_kind="s4d", with_dy=False)
    got = gpu_fwd(inp, to_device(inp))
    log("  oracle on the whole workload")
    want = oracle_fwd(inp)
    assert_close(host(got["y"]), want["y"], w.io, "y")
    assert_close(host(got["last_h"]), want["last_h"], "f32", "last_h")
    assert_close(host(got["last_v"]), want["last_v"], "f32", "last_v")


def test_full_size_backward():
    """The backward shape with every extra: every output of every batch row and channel against
    the oracle, with the conditioning term from two perturbed oracle runs."""
    w = W["bwd"].replace(dskip=True)
    log("full-size fused bwd: drawing inputs")
    inp = fused_inputs(w, 471, a_kind="s4d")
    got = gpu_bwd(inp, to_device(inp))
    log("  oracle on the whole workload (and two perturbed runs)")
    want, sp = spread(oracle_bwd, inp, FUSED_KEYS, BWD_OUT, trials=2)
    compare(got, want, ("dx", "ddelta", "dA", "dB", "dC", "dDskip", "dz", "ddelta_bias"), w.io,
            "full", sp)


# ---- zero-order hold ----

@pytest.mark.parametrize("softplus,use_z,use_bias", [(True, True, True), (False, False, False)])
@pytest.mark.parametrize("beta", [0.9, 0.0])
def test_zoh_tiny(softplus, use_z, use_bias, beta):
    w = W["tiny"].replace(beta=beta, dskip=True)
    inp = fused_inputs(w, 481, softplus, use_z, use_bias, zoh=True)
    check(inp, {"states_per_wave": 2, "chunks": 2}, {"states_per_wave": 1}, tag="zoh tiny")


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("K", [1, 2, 4])
def test_zoh_small(io, K):
    w = SMALL.replace(io=io, dskip=True, beta=0.85, alpha=0.6)
    inp = fused_inputs(w, 491, zoh=True)
    check(inp, {"states_per_wave": 4 if K == 4 else 2 * K, "chunks": K}, {"states_per_wave": K},
          state=True, tag="zoh small K=%d" % K)


@pytest.mark.parametrize("N", [5, 27, 33, 64])
def test_zoh_state_counts(N):
    w = SMALL.replace(L=40, D=70, N=N, dskip=True)
    check(fused_inputs(w, 500 + N, softplus=False, use_z=False, use_bias=False, zoh=True),
          tag="zoh N=%d" % N)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_zoh_series_switches(io):
    # decay arguments u = delta A on both sides of the switches between the series and the
    # quotient forms of phi (|u| = 1/8 in the forward, 1/4 in the backward) and psi (1/4), at
    # A = 0 exactly (g = delta), near 0 (long memory), and far enough out that e^u underflows
    # (A = -1000), with delta ~ U[0.4, 1.3].  Long memories at such steps make dA and ddelta
    # ill-conditioned (tests/test_conditioning.py): the backward's outputs are held to the fp32
    # bound plus the oracle's own spread under one fp32 rounding of the inputs.
    w = SMALL.replace(io=io, L=37, D=70, N=16, dskip=True)
    inp = fused_inputs(w, 541, softplus=False, use_z=False, use_bias=False, zoh=True)
    cols = np.array([0.0, -1e-4, -0.06, -0.11, -0.15, -0.2, -0.3, -0.45, -1000.0, -1.0, -2.0,
                     -4.0, -8.0, -0.1, -0.25, -0.5], dtype=np.float32)
    inp["A"] = np.ascontiguousarray(np.tile(cols, (w.D, 1)))
    rng = np.random.default_rng(542)
    inp["delta"] = rng.uniform(0.4, 1.3, size=inp["delta"].shape).astype(np.float32)
    if io == "bf16":
        inp["delta"] = workloads.round_to_bf16(inp["delta"])
    u = np.abs(inp["delta"][..., None] * cols)
    for edge in (0.125, 0.25):  # both sides of each switch occur
        assert ((u < edge) & (u > edge / 2)).any() and ((u > edge) & (u < 2 * edge)).any()
    assert (u > 104).any()  # e^u below the fp32 range
    check(inp, tag="zoh switches", cond_outputs=BWD_OUT)


def test_zoh_full_size():
    """The headline forward shape and the backward shape with the zero-order hold and every
    extra: every output against the oracle."""
    w = W["m1p4b"].replace(dskip=True)
    inp = fused_inputs(w, 511, a_kind="s4d", with_dy=False, zoh=True)
    got = gpu_fwd(inp, to_device(inp))
    want = oracle_fwd(inp)
    assert_close(host(got["y"]), want["y"], w.io, "zoh y")
    assert_close(host(got["last_h"]), want["last_h"], "f32", "zoh last_h")
    del got, want, inp
    wb = W["bwd"].replace(dskip=True)
    inp = fused_inputs(wb, 521, a_kind="s4d", zoh=True)
    got = gpu_bwd(inp, to_device(inp))
    want, sp = spread(oracle_bwd, inp, FUSED_KEYS, BWD_OUT, trials=2)
    compare(got, want, ("dx", "ddelta", "dA", "dB", "dC", "dDskip", "dz", "ddelta_bias"), wb.io,
            "zoh full", sp)
