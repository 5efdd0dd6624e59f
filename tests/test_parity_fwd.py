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

def check_sampled(w, a_kind="s4d", beta=None, nsample=24):
    wl = w if beta is None else w.replace(beta=beta)
    log("full-size %s beta=%g: drawing inputs" % (wl.name, wl.beta))
    inp = workloads.make_inputs(wl, a_kind=a_kind)
    y, lh, lv = run_fwd(inp)
    dsel = sample_channels(wl.D, nsample, seed=wl.seed)
    log("  comparing %d channels x %d batch rows against the oracle" % (len(dsel), wl.Bt))
    sub = sub_problem(inp, dsel=dsel)
    oy, olh, olv = oracle_fwd(sub)
    y = host(y)[:, :, dsel]
    assert_close(y, oy, wl.io, "y %s" % wl.name)
    assert_close(host(lh)[:, dsel], olh, "f32", "last_h %s" % wl.name)
    assert_close(host(lv)[:, dsel], olv, "f32", "last_v %s" % wl.name)


@pytest.mark.parametrize("beta", [0.0, 0.9])
def test_full_m130m(beta):
    check_sampled(W["m130m"], beta=beta)


def test_full_m1p4b():
    check_sampled(W["m1p4b"])


def test_full_m1p4b_unstructured_A():
    check_sampled(W["m1p4b"], a_kind="random")


def test_full_long_sequence():
    check_sampled(W["long"], nsample=12)


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
