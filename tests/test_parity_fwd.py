"""Forward parity: the HIP library (through the C ABI) against the fp64 oracle."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import (assert_close, host, inputs_to_device, log, run_fwd, sample_channels,
                      sub_problem)

pytestmark = pytest.mark.gpu

W = workloads.WORKLOADS


def oracle_fwd(inp):
    return oracle.fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["beta"],
                      inp["alpha"], Dskip=inp["Dskip"])


def check_full(inp, plan=None, tag=""):
    io = inp["io"]
    log("fwd %s shape=%s io=%s beta=%g alpha=%g plan=%s" % (tag, inp["x"].shape, io, inp["beta"],
                                                           inp["alpha"], plan))
    y, lh, lv = run_fwd(inp, plan=plan)
    oy, olh, olv = oracle_fwd(inp)
    e = assert_close(host(y), oy, io, "y " + tag)
    # the states are fp32 in every I/O mode and are compared at the fp32 tolerance
    assert_close(host(lh), olh, "f32", "last_h " + tag)
    assert_close(host(lv), olv, "f32", "last_v " + tag)
    return e


# ---- the tiny workload, both momentum settings, every plan the build offers ----

@pytest.mark.parametrize("beta", [0.9, 0.0])
@pytest.mark.parametrize("K", [1, 2, 4])
@pytest.mark.parametrize("chunks", [1, 2, 4])
def test_tiny_workload_all_plans(beta, K, chunks):
    inp = workloads.make_inputs(W["tiny"].replace(beta=beta))
    check_full(inp, plan={"states_per_wave": K, "chunks": chunks}, tag="tiny")


def test_tiny_workload_auto_plan():
    for beta in (0.9, 0.0):
        check_full(workloads.make_inputs(W["tiny"].replace(beta=beta)), tag="tiny-auto")


# ---- the half-wavefront layout of unchunked 16-state plans: workgroup order and edges ----
# 32-channel workgroups whose indices are permuted within each group of 16 (the two halves of a
# 64-channel block 8 apart); grids of 18 leave a tail of 2 unpermuted; D = 160 and D = 30
# leave a workgroup with no valid channel; 64 workgroups are all permuted.

@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(3, 70, 160), (9, 40, 30), (8, 100, 256)])
def test_half_wave_workgroup_order(io, shape):
    Bt, L, D = shape
    inp = workloads.make_inputs(W["m130m"].replace(Bt=Bt, L=L, D=D, N=16, io=io, beta=0.9,
                                                   alpha=0.7, dskip=True),
                                a_kind="random", seed=91)
    check_full(inp, plan={"states_per_wave": 2, "chunks": 1}, tag="half-wave %s" % (shape,))


# ---- several tiles, ragged time and channel tails, every state split and chunking ----

SMALL = W["m130m"].replace(Bt=2, L=200, D=100, N=16)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("K", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("chunks", [1, 3])
def test_small_ragged_plans(io, K, chunks):
    inp = workloads.make_inputs(SMALL.replace(io=io, beta=0.9, alpha=0.7, dskip=True),
                                a_kind="random", seed=77)
    check_full(inp, plan={"states_per_wave": K, "chunks": chunks}, tag="small")


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("beta,alpha,dskip", [(0.0, 1.0, False), (0.0, 1.0, True),
                                              (0.9, 1.0, False), (0.5, 2.5, True)])
def test_small_ragged_settings(io, beta, alpha, dskip):
    inp = workloads.make_inputs(SMALL.replace(io=io, beta=beta, alpha=alpha, dskip=dskip),
                                seed=78)
    check_full(inp, tag="settings")


@pytest.mark.parametrize("N", [1, 2, 3, 5, 8, 17, 24, 32, 33, 64])
def test_state_counts(N):
    inp = workloads.make_inputs(SMALL.replace(L=70, D=70, N=N, beta=0.8, dskip=True),
                                a_kind="random", seed=100 + N)
    check_full(inp, tag="N=%d" % N)
    check_full(inp, plan={"states_per_wave": 4, "chunks": 2}, tag="N=%d chunked" % N)


@pytest.mark.parametrize("shape", [(1, 1, 1, 16), (3, 1, 5, 4), (1, 17, 1, 16), (2, 16, 64, 16),
                                   (1, 33, 65, 16), (5, 48, 3, 2)])
def test_degenerate_shapes(shape):
    Bt, L, D, N = shape
    inp = workloads.make_inputs(SMALL.replace(Bt=Bt, L=L, D=D, N=N, dskip=True), seed=5)
    check_full(inp, tag="shape=%s" % (shape,))


@pytest.mark.parametrize("beta,alpha", [(1e-6, 1.0), (0.999, 1.0), (0.9, 0.0), (0.9, 10.0)])
def test_momentum_edge_cases(beta, alpha):
    inp = workloads.make_inputs(SMALL.replace(beta=beta, alpha=alpha, dskip=True), seed=9)
    check_full(inp, tag="edge")


def test_alpha_zero_gives_skip_only():
    inp = workloads.make_inputs(SMALL.replace(beta=0.9, alpha=0.0, dskip=True), seed=10)
    y, lh, lv = run_fwd(inp)
    np.testing.assert_array_equal(host(lh), 0.0)
    np.testing.assert_allclose(host(y), inp["Dskip"] * inp["x"].astype(np.float64), rtol=1e-6,
                               atol=1e-7)


def test_deterministic_across_runs():
    inp = workloads.make_inputs(SMALL.replace(io="bf16", beta=0.9, dskip=True), seed=11)
    g = inputs_to_device(inp)
    outs = [run_fwd(inp, g, plan={"states_per_wave": 4, "chunks": 3}) for _ in range(3)]
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert np.array_equal(host(a), host(b))


def test_plans_agree_with_each_other():
    inp = workloads.make_inputs(SMALL.replace(L=400, beta=0.9), seed=12)
    g = inputs_to_device(inp)
    ref = host(run_fwd(inp, g, plan={"states_per_wave": 16, "chunks": 1})[0])
    for K in (1, 2, 4, 8):
        for G in (1, 2, 5, 25):
            y = host(run_fwd(inp, g, plan={"states_per_wave": K, "chunks": G})[0])
            assert_close(y, ref, "f32", "plan K=%d G=%d vs K=16 G=1" % (K, G))


# ---- full-size workloads, in the launch configuration the bench times ----

def check_full_size(w, a_kind="s4d", beta=None):
    """Every output of the workload against the oracle on the whole workload."""
    wl = w if beta is None else w.replace(beta=beta)
    log("full-size %s beta=%g: drawing inputs" % (wl.name, wl.beta))
    inp = workloads.make_inputs(wl, a_kind=a_kind)
    y, lh, lv = run_fwd(inp)
    log("  oracle on the whole workload")
    oy, olh, olv = oracle_fwd(inp)
    assert_close(host(y), oy, wl.io, "y %s" % wl.name)
    assert_close(host(lh), olh, "f32", "last_h %s" % wl.name)
    assert_close(host(lv), olv, "f32", "last_v %s" % wl.name)


@pytest.mark.parametrize("beta", [0.0, 0.9])
def test_full_m130m(beta):
    check_full_size(W["m130m"], beta=beta)


def test_full_m1p4b():
    check_full_size(W["m1p4b"])


def test_full_m1p4b_unstructured_A():
    check_full_size(W["m1p4b"], a_kind="random")


def test_full_long_sequence():
    check_full_size(W["long"])


def test_batch_32():
    """Batch 32, one of the README's edge cases, forward and backward against the oracle."""
    inp = workloads.make_inputs(W["m130m"].replace(Bt=32, L=300, D=200, dskip=True),
                                a_kind="random", seed=15, with_dy=True)
    check_full(inp, tag="batch 32")
    from test_parity_bwd import check_full as check_bwd
    check_bwd(inp, tag="batch 32")


# ---- structure of the scan at full size, on the GPU's own outputs ----
# Properties that hold for the exact scan at any size (the oracle's pins check the same ones on
# small inputs): causality, linearity in x, homogeneity in alpha.

def _fwd_dev(g, beta, alpha, Dskip=None, x=None, plan=None):
    import torch
    import selective_state_space_msm_amd as msm
    y = msm.msm_scan_fwd(g["x"] if x is None else x, g["delta"], g["A"], g["B"], g["C"], beta,
                         alpha, Dskip, plan=plan)
    torch.cuda.synchronize()
    return y


def test_full_size_causality():
    """Changing x at one step changes no output before it, bit for bit (m130m shape, chunked
    and unchunked plans)."""
    import torch
    w = W["m130m"]
    inp = workloads.make_inputs(w, seed=21)
    g = inputs_to_device(inp)
    for plan in (None, {"states_per_wave": 2, "chunks": 4}):
        y0 = _fwd_dev(g, inp["beta"], inp["alpha"], plan=plan)
        for t in (1, 777, w.L - 1):
            x2 = g["x"].clone()
            x2[:, t, :] += 1.0
            y1 = _fwd_dev(g, inp["beta"], inp["alpha"], x=x2, plan=plan)
            assert torch.equal(y1[:, :t], y0[:, :t]), (t, plan)
            assert not torch.equal(y1[:, t], y0[:, t]), (t, plan)


def test_full_size_linearity_in_x():
    """y(x1 + x2) = y(x1) + y(x2) (m130m shape, fp32 I/O, no skip term): each of the three
    results is within atol + rtol |y| of its exact value, so the identity holds to the sum of
    the three bounds."""
    import torch
    w = W["m130m"]
    inp = workloads.make_inputs(w, seed=22)
    g = inputs_to_device(inp)
    x1 = g["x"]
    x2 = torch.flip(g["x"], dims=[2]).contiguous()
    ya = _fwd_dev(g, inp["beta"], inp["alpha"], x=x1).double()
    yb = _fwd_dev(g, inp["beta"], inp["alpha"], x=x2).double()
    yab = _fwd_dev(g, inp["beta"], inp["alpha"], x=(x1 + x2)).double()
    err = (yab - (ya + yb)).abs()
    lim = 3e-4 + 1e-5 * (ya.abs() + yb.abs() + yab.abs())
    assert bool((err <= lim).all()), float((err - lim).max())


def test_full_size_alpha_homogeneity():
    """y(alpha) - Dskip x = alpha (y(1) - Dskip x) (m130m shape, fp32 I/O, with the skip term),
    to the bounds of the two results (atol + rtol |y| each, the second scaled by alpha)."""
    w = W["m130m"].replace(dskip=True)
    inp = workloads.make_inputs(w, seed=23)
    g = inputs_to_device(inp)
    skip = (g["Dskip"][None, None, :] * g["x"]).double()
    f1 = _fwd_dev(g, inp["beta"], 1.0, g["Dskip"]).double()
    fa = _fwd_dev(g, inp["beta"], 0.37, g["Dskip"]).double()
    err = ((fa - skip) - 0.37 * (f1 - skip)).abs()
    lim = 1.37e-4 + 1e-5 * (fa.abs() + 0.37 * f1.abs())
    assert bool((err <= lim).all()), float((err - lim).max())


def _device_inputs(Bt, L, D, N, seed):
    """Seeded inputs drawn on the GPU (x ~ N(0,1), delta = softplus(N(-4,1)), B, C ~ N(0,1),
    A = -(n+1)): arrays of several GiB that the host need not hold."""
    import torch
    gen = torch.Generator(device="cuda").manual_seed(seed)
    x = torch.randn((Bt, L, D), generator=gen, device="cuda")
    delta = torch.nn.functional.softplus(torch.randn((Bt, L, D), generator=gen, device="cuda") - 4)
    B = torch.randn((Bt, L, N), generator=gen, device="cuda")
    C = torch.randn((Bt, L, N), generator=gen, device="cuda")
    A = -(torch.arange(N, dtype=torch.float32, device="cuda") + 1).repeat(D, 1).contiguous()
    return x, delta, A, B, C


def test_rows_beyond_32bit_offsets():
    """One batch row of 2^19 + 37 steps x 1024 fp32 channels is 2.1 GB per array, past the
    2^31-byte reach of the kernels' buffer offsets: a one-chunk plan must be split, and every
    plan must agree with the oracle on sampled channels."""
    import torch
    import selective_state_space_msm_amd as msm
    Bt, L, D, N = 1, (1 << 19) + 37, 1024, 16
    log("rows beyond 32-bit offsets: L=%d D=%d fp32" % (L, D))
    x, delta, A, B, C = _device_inputs(Bt, L, D, N, 71)
    dsel = sample_channels(D, 6, seed=72)
    sub = dict(x=host(x[:, :, dsel]), delta=host(delta[:, :, dsel]), A=host(A[dsel]), B=host(B),
               C=host(C))
    want, wh, _ = oracle.fwd(sub["x"], sub["delta"], sub["A"], sub["B"], sub["C"], 0.9, 1.0)
    for plan in ({"states_per_wave": 2, "chunks": 1}, None):
        y, lh, _ = msm.msm_scan_fwd(x, delta, A, B, C, 0.9, 1.0, return_last_state=True,
                                    plan=plan)
        torch.cuda.synchronize()
        assert_close(host(y[:, :, dsel]), want, "f32", "y plan %s" % plan)
        assert_close(host(lh[:, dsel]), wh, "f32", "last_h plan %s" % plan)
        del y, lh


@pytest.mark.parametrize("K,chunks", [(4, 1), (8, 1), (8, 3)])
def test_32_state_plans(K, chunks):
    inp = workloads.make_inputs(SMALL.replace(L=90, D=70, N=29, beta=0.85, dskip=True),
                                a_kind="random", seed=130 + K + chunks)
    check_full(inp, plan={"states_per_wave": K, "chunks": chunks}, tag="N=29 K=%d" % K)


def test_side_stream_calls_match_current_stream():
    """Calls enqueued on a side stream: the binding's own workspace and outputs are recorded on
    that stream; results equal the current-stream results."""
    import torch
    import selective_state_space_msm_amd as msm
    inp = workloads.make_inputs(SMALL.replace(L=300, beta=0.9, dskip=True), seed=14, with_dy=True)
    g = inputs_to_device(inp)
    dy = torch.from_numpy(inp["dy"]).to("cuda")
    ref_y = msm.msm_scan_fwd(g["x"], g["delta"], g["A"], g["B"], g["C"], 0.9, 1.0, g["Dskip"],
                             plan={"states_per_wave": 2, "chunks": 3})
    ref_g = msm.msm_scan_bwd(g["x"], g["delta"], g["A"], g["B"], g["C"], dy, 0.9, 1.0, g["Dskip"])
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    y = msm.msm_scan_fwd(g["x"], g["delta"], g["A"], g["B"], g["C"], 0.9, 1.0, g["Dskip"],
                         stream=side, plan={"states_per_wave": 2, "chunks": 3})
    gr = msm.msm_scan_bwd(g["x"], g["delta"], g["A"], g["B"], g["C"], dy, 0.9, 1.0, g["Dskip"],
                          stream=side)
    # memory allocated on the current stream meanwhile must not land on the side stream's buffers
    junk = [torch.full((1 << 20,), 7.0, device="cuda") for _ in range(8)]
    side.synchronize()
    assert np.array_equal(host(y), host(ref_y))
    for k in ("dx", "ddelta", "dA", "dB", "dC", "dDskip"):
        assert np.array_equal(host(gr[k]), host(ref_g[k])), k
    del junk


# ---- chunk summaries over a window of the chunk ----

@pytest.mark.parametrize("case", ["window", "long-memory", "slow-velocity", "zoh-window"])
def test_chunk_summary_windows(case):
    """Chunked plans whose summaries may cover only the chunk's last rows (the rows after which
    the start state's share is below 2^-32): steps large enough that a window is found
    (delta = softplus(N(-2, 1)), about 150 rows), steps so small that the whole chunk is needed
    (delta in [1e-5, 1e-4], the long-memory case), a velocity memory longer than a chunk
    (beta = 0.99: 2207 rows for 2^-32), and the fused zero-order-hold build with windows.
    Every output against the oracle."""
    import selective_state_space_msm_amd as msm
    w = W["m130m"].replace(Bt=2, L=8000, D=130, N=16, beta=0.99 if case == "slow-velocity" else 0.9,
                           dskip=True)
    inp = workloads.make_inputs(w, a_kind="random", seed=160)
    rng = np.random.default_rng(161)
    if case == "long-memory":
        inp["delta"] = np.exp(rng.uniform(np.log(1e-5), np.log(1e-4),
                                          size=inp["delta"].shape)).astype(np.float32)
    else:
        u = rng.normal(-2.0, 1.0, size=inp["delta"].shape)
        inp["delta"] = np.log1p(np.exp(u)).astype(np.float32)
    if case != "zoh-window":
        for plan in ({"states_per_wave": 2, "chunks": 4}, {"states_per_wave": 4, "chunks": 7}):
            check_full(inp, plan=plan, tag=case)
        return
    import torch
    g = inputs_to_device(inp)
    y, lh, lv = msm.msm_selective_scan_fwd(g["x"], g["delta"], g["A"], g["B"], g["C"], inp["beta"],
                                           inp["alpha"], g["Dskip"], zero_order_hold=True,
                                           return_last_state=True,
                                           plan={"states_per_wave": 2, "chunks": 5})
    torch.cuda.synchronize()
    oy, _, oh, ov = oracle.fused_fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"],
                                     inp["beta"], inp["alpha"], Dskip=inp["Dskip"], zoh=True)
    assert_close(host(y), oy, "f32", "zoh y windows")
    assert_close(host(lh), oh, "f32", "zoh last_h windows")
    assert_close(host(lv), ov, "f32", "zoh last_v windows")


@pytest.mark.parametrize("beta", [0.9, 0.0])
@pytest.mark.parametrize("N", [16, 13])
def test_chunk_summary_windows_per_wavefront(beta, N):
    """Summary windows that differ between the wavefronts of a workgroup: state 0 decays so
    slowly in half the channels (A = -0.05: the 2^-32 bound needs about 3400 rows, more than a
    chunk) that its wavefront maps the whole chunk, while the other states (A = -(n + 1)) stop
    at the velocity's bound (about 220 rows), so the workgroup's map is exact and some of its
    wavefronts' maps are truncated; with N = 13 the last wavefronts hold padded states.  (A much
    slower state, A = -1e-3 with a memory of about 7700 rows, is outside what an fp32 state can
    hold to the fp32 bound: a sequential fp32 scan of the same input misses it by 5.9x.)  Every
    output against the oracle."""
    w = W["m130m"].replace(Bt=2, L=6000, D=130, N=N, beta=beta, dskip=True)
    inp = workloads.make_inputs(w, seed=170 + N)
    rng = np.random.default_rng(171)
    u = rng.normal(-2.0, 1.0, size=inp["delta"].shape)
    inp["delta"] = np.log1p(np.exp(u)).astype(np.float32)
    A = -np.tile(np.arange(1, N + 1, dtype=np.float32), (w.D, 1))
    A[::2, 0] = -0.05
    inp["A"] = np.ascontiguousarray(A)
    for plan in ({"states_per_wave": 2, "chunks": 4}, {"states_per_wave": 4, "chunks": 7}):
        check_full(inp, plan=plan, tag="windows per wavefront N=%d beta=%g" % (N, beta))
